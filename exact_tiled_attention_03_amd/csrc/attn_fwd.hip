// attn_fwd.hip -- fused exact-attention forward for gfx950 (MI355X) and its C ABI.
//
// Method: "Triton in depth: from matmul to Flash Attention" (ybb.press),
// sections 3.2-3.3.  Each work-group owns one query tile of one (batch, head)
// and walks the key/value tiles once, keeping for every query row the running
// max m and running sum l of the exponentials; the fp32 output accumulator is
// rescaled by exp(m_old - m_new) whenever the max grows, and divided by l once
// after the loop.  Keys with index > query index are excluded when causal.
// The N x N score matrix never leaves registers.
//
// gfx950 mapping (not taken from the pages, which target NVIDIA tensor cores):
//
//  * Scores are produced transposed, S^T = K Q^T, with v_mfma_f32_32x32x16.
//    In the 32x32 accumulator layout a lane owns one column, so each lane
//    holds 16 scores of ONE query.  The row max is then 15 lane-local max ops
//    plus one exchange with lane^32 (the other half of the same column); the
//    row sum needs no exchange until the epilogue.
//  * The K rows fed to the A operand are permuted (kperm) so that the 16
//    accumulator registers of a lane map to two runs of 8 consecutive keys.
//    Those runs are exactly the B operand layout of the next MFMA,
//    O^T += V^T P^T, so P goes from the score accumulator to the P.V operand
//    without leaving the lane.
//  * V^T is needed as an A operand with 8 consecutive keys per lane; the
//    loader transposes 4x8 blocks in registers and stores V^T in LDS.
//  * K and V^T tiles are double-buffered in LDS with one-chunk row padding,
//    which makes the 16-byte operand reads bank-conflict free.
//  * Work-groups are remapped so that consecutive ids on one XCD (ids are
//    dealt round-robin over the 8 XCDs) cover the query tiles of the same
//    heads: a head's K/V then stays in that XCD's L2.  Causal tiles run
//    longest first to shorten the tail.
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA; lse is
//    returned in natural-log units.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cfloat>
#include <cstring>
#include <type_traits>

#include "attn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Compile-time tuning knobs (defaults are the shipped configuration).
#ifndef ETA_WAVES_PER_EU
#define ETA_WAVES_PER_EU 2      // waves per SIMD the register budget is sized for
#endif
#ifndef ETA_RESCALE_TH
#define ETA_RESCALE_TH 8.0f     // log2 headroom before the running max is raised
#endif
#ifndef ETA_LANE_SWAP
#define ETA_LANE_SWAP 1         // 1: v_permlane32_swap for the lane-pair exchange, 0: ds_bpermute
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// --- element type ------------------------------------------------------------
template <int DT> struct Elem;

template <> struct Elem<ATTN_F16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                     __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    // round-to-nearest-even of two floats, packed low/high
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f16x2_t p;
        p[0] = (_Float16)x;
        p[1] = (_Float16)y;
        return __builtin_bit_cast(unsigned, p);
    }
};

template <> struct Elem<ATTN_BF16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        bf16x2_t p;
        p[0] = (__bf16)x;
        p[1] = (__bf16)y;
        return __builtin_bit_cast(unsigned, p);
    }
};

struct FwdArgs {
    const u32x4_t* q;  // [BH, N, D] as 16-byte chunks
    const u32x4_t* k;
    const u32x4_t* v;
    uint16_t* o;
    float* lse;        // may be null
    int N;
    int BH;
    int nqt;           // query tiles per head
    float c;           // |scale| * log2(e)
    unsigned qsign;    // 0x80008000 when scale < 0 (Q negated exactly), else 0
};

// Value of x in the lane 32 positions away (the other half of the same accumulator column).
__device__ __forceinline__ float pair_max(float x) {
#if ETA_LANE_SWAP
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
    return fmaxf(x, __shfl_xor(x, 32));
#endif
}

__device__ __forceinline__ float pair_sum(float x) {
#if ETA_LANE_SWAP
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
#else
    return x + __shfl_xor(x, 32);
#endif
}

// Row of the K tile that feeds A-operand row m of the score MFMA.  With this
// permutation, accumulator register i of a lane in half h holds key
// 16*(i/8) + 8*h + (i%8) of the 32-key block.
__device__ __forceinline__ int kperm(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Tile configuration shared by the kernel and the host launcher.
//
// LDS holds two stages of K and V, each a BN x ROWB byte array written by
// direct global->LDS loads: one load instruction of a wave fills 1 KB of
// consecutive 16-byte slots, so rows are unpadded (ROWB = CPRP * 16 with CPRP
// the chunk count rounded up to a power of two) and bank conflicts are avoided
// by XOR-swizzling the 16-byte chunk index with a function of the row:
//  * K is read by the score MFMA as 16-byte chunks of 16 different rows at the
//    same logical chunk: chunk c of row r sits at c ^ kswz(r), kswz(r) =
//    (r / RPB) % CPRP with RPB rows per 256-byte bank line.
//  * V is read by 8-byte transpose loads, 4 consecutive rows x one 64-byte
//    granule per 32 lanes: the granule index g of row r sits at
//    g ^ ((r / RPB) % GPR), GPR granules per row.
template <int D> struct Cfg {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;             // threads per work-group
    static constexpr int BM = 32 * WAVES;             // queries per work-group (32 per wave)
    static constexpr int BN = 64;                     // keys per tile
    static constexpr int SB = BN / 32;                // 32-key score blocks per tile
    static constexpr int KSTEPS = D / 16;             // MFMA k-steps over the head dim
    static constexpr int DBLK = (D + 31) / 32;        // 32-row blocks of O^T
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row in HBM
    static constexpr int CPRP = CPR <= 8 ? 8 : 16;    // chunks per row in LDS
    static constexpr int ROWB = CPRP * 16;            // bytes per row in LDS
    static constexpr int RPB = 256 / ROWB;            // rows per 256-byte bank line
    static constexpr int GPR = CPRP / 4;              // 64-byte granules per row
    static constexpr int TILEB = BN * ROWB;           // bytes of one K or V tile
    static constexpr int KOFF = 0;                    // K stage s at KOFF + s * TILEB
    static constexpr int VOFF = 2 * TILEB;            // V stage s at VOFF + s * TILEB
    static constexpr int LDS = 4 * TILEB;
    static constexpr int IT = TILEB / (16 * NT);      // direct-load instructions per tile and thread
    static_assert(D % 16 == 0 && CPR <= CPRP, "head dim");
    static_assert(TILEB % (16 * NT) == 0, "a tile is a whole number of load rounds");
    static_assert(DBLK <= GPR, "transpose reads of the padded head dim stay inside a row");
    static_assert(VOFF + 2 * TILEB <= 65536, "LDS offsets fit the 16-bit immediate");
};

typedef __fp16 lds_v4h_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) lds_v4h_t* lds_v4h_ptr;
typedef __attribute__((address_space(3))) unsigned char* lds_bytes;

// 8 bytes from LDS through the gfx950 transpose read: within each 16-lane
// group, lane i receives element (i % 4) of the 8-byte rows addressed by lanes
// i/4, i/4 + 4, i/4 + 8, i/4 + 12.
__device__ __forceinline__ u32x2_t lds_read_tr(unsigned addr) {
    const lds_v4h_t t = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4h_ptr)(lds_bytes)(size_t)addr);
    return __builtin_bit_cast(u32x2_t, t);
}

__device__ __forceinline__ u32x4_t lds_read16(unsigned addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((lds_bytes)(size_t)addr);
}

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ETA_WAVES_PER_EU, ETA_WAVES_PER_EU)))
void attn_fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    using C = Cfg<D>;
    using E = Elem<DT>;
    constexpr int BN = C::BN, SB = C::SB, KSTEPS = C::KSTEPS, DBLK = C::DBLK, CPR = C::CPR;
    constexpr int CPRP = C::CPRP, ROWB = C::ROWB;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
    const unsigned lds0 = (unsigned)(size_t)(lds_bytes)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int hf = lane >> 5;   // which half of the 64-lane wave
    const int n = lane & 31;    // accumulator column = query within the wave's 32

    // ---- work-group -> (head, query tile): XCD-aware, causal longest first
    const int T = a.nqt * a.BH;
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int vidx = xcd * (T >> 3) + min(xcd, T & 7) + (L >> 3);
    const int bh = vidx / a.nqt;
    int qt = vidx - bh * a.nqt;
    if (CAUSAL) qt = a.nqt - 1 - qt;

    const int N = a.N;
    const int q0 = qt * C::BM;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + n;
    const size_t hoff = (size_t)bh * (size_t)N * CPR;   // head offset in 16-byte chunks

    // ---- Q fragments (B operand of S^T = K Q^T), loaded once
    u32x4_t qf[KSTEPS];
    if (qi < N) {
        const u32x4_t* src = a.q + hoff + (size_t)qi * CPR + hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = src[2 * ks] ^ a.qsign;
    } else {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
    }

    const int kend = CAUSAL ? min(N, q0 + C::BM) : N;
    const int nt = (kend + BN - 1) / BN;

    // ---- direct global -> LDS loads.  Slot (it, wave, lane) of a tile holds
    // row r = slot / CPRP, physical chunk p = slot % CPRP, i.e. logical chunk
    // p ^ swizzle(r); chunks past the head dim get an out-of-range offset and
    // read as zero, as do rows past N (the buffer ends at row N).
    unsigned kvo[C::IT], vvo[C::IT];
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
        const int slot = it * C::NT + wave * 64 + lane;
        const int r = slot / CPRP, p = slot % CPRP;
        const int kc = p ^ ((r / C::RPB) % CPRP);
        const int vc = p ^ (4 * ((r / C::RPB) % C::GPR));
        kvo[it] = kc < CPR ? (unsigned)(r * D * 2 + kc * 16) : 0x80000000u;
        vvo[it] = vc < CPR ? (unsigned)(r * D * 2 + vc * 16) : 0x80000000u;
    }
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k + hoff);
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v + hoff);
    auto issue_loads = [&](int j, int stage) {
        const int kt0 = j * BN;
        const int bytes = (N - kt0) * D * 2;            // rows kt0 .. N-1 are in range
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (size_t)kt0 * D * 2), 0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (size_t)kt0 * D * 2), 0, bytes, 0x00020000);
#pragma unroll
        for (int it = 0; it < C::IT; ++it) {
            const unsigned dst = (unsigned)((it * C::NT + wave * 64) * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(lds_bytes)(size_t)(lds0 + C::KOFF + stage * C::TILEB + dst), 16, kvo[it], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(lds_bytes)(size_t)(lds0 + C::VOFF + stage * C::TILEB + dst), 16, vvo[it], 0, 0, 0);
        }
    };

    // ---- per-lane LDS read addresses (stage 0; stage 1 adds TILEB)
    unsigned ka[KSTEPS];   // score A operand: row kperm(n), logical chunk 2*ks + hf
    {
        const int r = kperm(n);
        const int x = (r / C::RPB) % CPRP;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) ka[ks] = lds0 + C::KOFF + r * ROWB + (((2 * ks + hf) ^ x) * 16);
    }
    unsigned va[DBLK];     // P.V A operand via transpose reads (see lds_read_tr)
    {
        const int g16 = lane >> 4, s16 = lane & 15;
        const int r = 8 * (g16 >> 1) + (s16 >> 2);           // + 16*kk + 4*half, both multiples of 4
        const int x = (r / C::RPB) % C::GPR;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
            va[db] = lds0 + C::VOFF + r * ROWB + (4 * (db ^ x) + 2 * (g16 & 1) + ((s16 & 3) >> 1)) * 16 + 8 * (s16 & 1);
    }

    // ---- per-lane running state (one query row per lane, half the keys)
    f32x16_t o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
    float m = kNegInf;   // reference max of scale*log2(e)*score, shared by both halves
    float l = 0.f;       // sum over this half's keys of exp2(t - m)
    const float c = a.c;

    // One K/V tile for this wave; need_mask (wave-uniform) on diagonal/ragged tiles.
    auto tile = [&](auto stage_tag, bool need_mask, int kt0) {
        constexpr int ST = decltype(stage_tag)::value * C::TILEB;
        // S^T = K Q^T: two independent 32-key accumulators, interleaved
        f32x16_t s[SB];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) s[sb] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
                s[sb] = E::mfma(lds_read16(ka[ks] + ST + sb * 32 * ROWB), qf[ks], s[sb]);

        if (need_mask) {
            // key index of register i is kt0 + 8*hf + 32*sb + 16*(i/8) + i%8; it is
            // kept iff that is <= lim (the query for causal, N-1 for the tail)
            const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - (kt0 + 8 * hf);
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * sb + 16 * (i >> 3) + (i & 7) > lim) s[sb][i] = kNegInf;
        }

        // online softmax.  m is raised only when a tile's max exceeds it by more
        // than ETA_RESCALE_TH (log2 units), so p <= 2^TH and the O rescale is rare;
        // m, l and O always refer to the same m, so the result is unchanged.
        float mx = kNegInf;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
        const float mt = pair_max(mx) * c;           // c > 0, so -inf stays -inf
        const bool grow = mt > m + ETA_RESCALE_TH;
        const float mnew = grow ? mt : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;   // 0 when m was -inf
        m = mnew;
        const float nm = m > kNegInf ? -m : 0.f;

        u32x4_t pf[2 * SB];   // P^T as B operands of the P.V k-steps (16 keys each)
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], c, nm));
                part[i & 3] += p[i];
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                pf[2 * sb + hh] = u32x4_t{E::pack2(p[8 * hh + 0], p[8 * hh + 1]), E::pack2(p[8 * hh + 2], p[8 * hh + 3]),
                                          E::pack2(p[8 * hh + 4], p[8 * hh + 5]), E::pack2(p[8 * hh + 6], p[8 * hh + 7])};
        }
        l = l * alpha + ((part[0] + part[1]) + (part[2] + part[3]));

        if (__any(grow)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
        }
        // O^T += V^T P^T; V^T operand = two transpose reads of 4 keys each
#pragma unroll
        for (int kk = 0; kk < 2 * SB; ++kk)
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const u32x2_t lo = lds_read_tr(va[db] + ST + 16 * kk * ROWB);
                const u32x2_t hi = lds_read_tr(va[db] + ST + (16 * kk + 4) * ROWB);
                o[db] = E::mfma(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf[kk], o[db]);
            }
    };

    // one loop step: prefetch tile j+1 into the other stage, compute tile j, sync
    auto step = [&](auto stage_tag, int j) {
        constexpr int STAGE = decltype(stage_tag)::value;
        if (j + 1 < nt) issue_loads(j + 1, STAGE ^ 1);
        const int kt0 = j * BN;
        // tiles wholly above this wave's diagonal, or waves past N, do no math
        if (qw0 < N && (!CAUSAL || kt0 <= qw0 + 31))
            tile(stage_tag, (CAUSAL && kt0 + BN - 1 > qw0) || kt0 + BN > N, kt0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    issue_loads(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int j = 0; j < nt; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        if (j + 1 < nt) step(std::integral_constant<int, 1>{}, j + 1);
    }

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l)
    if (qw0 < N) {
        const float ltot = pair_sum(l);
        if (qi < N) {
            const float inv = 1.0f / ltot;
            uint16_t* orow = a.o + ((size_t)bh * N + qi) * D;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = db * 32 + 8 * g + 4 * hf;
                    if (d0 < D) {
                        const u32x2_t w = {E::pack2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                                           E::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
                        *reinterpret_cast<u32x2_t*>(orow + d0) = w;
                    }
                }
            if (a.lse != nullptr && hf == 0) a.lse[(size_t)bh * N + qi] = (m + __builtin_amdgcn_logf(ltot)) * kLn2;
        }
    }
#endif
}

// --- host side ---------------------------------------------------------------

template <int D, int DT, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)a.nqt * (unsigned)a.BH;
    hipLaunchKernelGGL((attn_fwd_kernel<D, DT, CAUSAL>), dim3(grid), dim3(Cfg<D>::NT), 0, stream, a);
    return hipGetLastError();
}

template <int D, int DT>
hipError_t dispatch_causal(const FwdArgs& a, int causal, hipStream_t s) {
    return causal ? launch<D, DT, true>(a, s) : launch<D, DT, false>(a, s);
}

template <int D>
hipError_t dispatch_dtype(const FwdArgs& a, int dtype, int causal, hipStream_t s) {
    return dtype == ATTN_BF16 ? dispatch_causal<D, ATTN_BF16>(a, causal, s) : dispatch_causal<D, ATTN_F16>(a, causal, s);
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int st = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (st == 1) return ATTN_OK;
        if (st == 2) return ATTN_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int N, int d, int causal, float scale, int dtype, void* stream) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 80 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return ATTN_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;

    const long long bh = (long long)B * H;
    const int bm = Cfg<128>::BM;   // the same for every head dim
    const long long nqt = ((long long)N + bm - 1) / bm;
    if (bh > INT32_MAX || nqt * bh > INT32_MAX) return ATTN_ERR_SHAPE;
    if ((long long)N * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;   // one head must fit a 32-bit buffer range
    const size_t tensor_bytes = (size_t)bh * (size_t)N * (size_t)d * 2u;
    if ((size_t)bh * (size_t)N * (size_t)d > (size_t)INT64_MAX / 4) return ATTN_ERR_SHAPE;
    const size_t lse_bytes = (size_t)bh * (size_t)N * 4u;
    if (overlaps(out, tensor_bytes, q, tensor_bytes) || overlaps(out, tensor_bytes, k, tensor_bytes) ||
        overlaps(out, tensor_bytes, v, tensor_bytes))
        return ATTN_ERR_ALIAS;
    if (lse && (overlaps(lse, lse_bytes, q, tensor_bytes) || overlaps(lse, lse_bytes, k, tensor_bytes) ||
                overlaps(lse, lse_bytes, v, tensor_bytes) || overlaps(lse, lse_bytes, out, tensor_bytes)))
        return ATTN_ERR_ALIAS;

    const int dev_status = check_device();
    if (dev_status != ATTN_OK) return dev_status;

    FwdArgs a;
    a.q = static_cast<const u32x4_t*>(q);
    a.k = static_cast<const u32x4_t*>(k);
    a.v = static_cast<const u32x4_t*>(v);
    a.o = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.N = N;
    a.BH = (int)bh;
    a.nqt = (int)nqt;
    // c must be > 0 so that masked scores (-inf) map to -inf; scale == 0 uses the
    // smallest normal float, which makes every exponent round to exactly 0
    a.c = scale == 0.f ? FLT_MIN : std::fabs(scale) * kLog2e;
    a.qsign = std::signbit(scale) && scale != 0.f ? 0x80008000u : 0u;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (d) {
        case 64: err = dispatch_dtype<64>(a, dtype, causal, s); break;
        case 80: err = dispatch_dtype<80>(a, dtype, causal, s); break;
        default: err = dispatch_dtype<128>(a, dtype, causal, s); break;
    }
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "q, k, v or out is NULL";
        case ATTN_ERR_SHAPE: return "B, H and N must be >= 1 and the grid must fit in 2^31-1 work-groups";
        case ATTN_ERR_HEAD_DIM: return "head dim must be 64, 80 or 128";
        case ATTN_ERR_DTYPE: return "dtype must be ATTN_F16 or ATTN_BF16";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_ALIGN: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
        case ATTN_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_CAUSAL: return "causal must be 0 or 1";
        case ATTN_ERR_ALIAS: return "out or lse overlaps an input or each other";
        default: return "unknown status";
    }
}
