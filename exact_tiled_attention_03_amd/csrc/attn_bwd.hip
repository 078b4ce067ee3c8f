// attn_bwd.hip -- exact-attention backward pass for gfx950 (MI355X) and its C ABI.
//
// Method: the derivative of the forward of "Triton in depth" 3.1-3.3 (the pages
// give no backward algorithm; "Triton: CUDA-level operators in Python" only
// names fused backward operators): with P_ij = exp(S_ij - lse_i) rebuilt from
// the forward's lse, dS = P * (dO V^T - D) where D_i = sum_c dO_ic O_ic,
// dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.  As in the forward, the N x N
// matrices are produced one tile at a time in registers and never reach HBM.
//
// Two kernels:
//  * dq:     a work-group owns 128 query rows (32 per wave) and walks the key
//            tiles like the forward: S^T = K Q^T and dP^T = V dO^T on MFMA with
//            the query's Q and dO rows in registers, dS^T formed in registers,
//            then dQ^T += K^T dS^T with K^T read through the transpose load.
//            It first forms D_i from the query's O and dO rows and writes it
//            to `delta` for the second kernel;
//  * dkdv:   a work-group owns 128 keys (32 per wave) and walks the query
//            tiles: S = Q K^T and dP = dO V^T with the key's K and V rows in
//            registers, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
//            read through the transpose load.
// In both, the score accumulator's rows follow the kperm order of the forward,
// so a lane's 16 accumulator registers are two runs of 8 consecutive rows and
// P (or dS), rounded to the input type, is the B operand of the next product
// without leaving the lane.
//
// LDS tiles (rows of 16-bit values, direct global->LDS loads, double-buffered)
// use one XOR swizzle that serves both access patterns: chunk c of row r sits
// at c ^ uswz(r).  For 256-byte rows uswz(r) = 4 (r % 4) + (r / 4) % 4: 16
// consecutive rows read at one logical chunk land on 16 distinct chunks, and
// the 4 rows of a transpose read land on 4 distinct 64-byte granules.  For
// 128-byte rows (two per bank line) uswz(r) = 4 ((r / 2) % 2) + (r / 4) % 4.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "attn_bwd.h"
#include "launch.h"
#include "lds_load.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

template <int DT> struct Elem;

template <> struct Elem<ATTN_F16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f16x2_t p;
        p[0] = (_Float16)x;
        p[1] = (_Float16)y;
        return __builtin_bit_cast(unsigned, p);
    }
    static __device__ __forceinline__ float lo(unsigned u) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
    }
    static __device__ __forceinline__ float hi(unsigned u) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16)); }
};

template <> struct Elem<ATTN_BF16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        bf16x2_t p;
        p[0] = (__bf16)x;
        p[1] = (__bf16)y;
        return __builtin_bit_cast(unsigned, p);
    }
    static __device__ __forceinline__ float lo(unsigned u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
};

struct BwdArgs {
    const u32x4_t* q;      // [BH, N, D] as 16-byte chunks
    const u32x4_t* k;
    const u32x4_t* v;
    const u32x4_t* o;
    const u32x4_t* dout;
    const float* lse;      // [BH, N]
    float* delta;          // [BH, N]
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int N, BH;
    int ntile, ngroups;    // per kernel: tiles of its own rows (queries or keys), work-groups per head
    float c;               // scale * log2(e), any sign
    float scale;
};

// x + the value in the lane 32 positions away, through v_permlane32_swap.
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of a 64-row tile that feeds MFMA A-operand row m (of a 32-row block):
// with it, accumulator register i of a lane in half h holds row
// 16*(i/8) + 8*h + (i%8) of the block.
__device__ __forceinline__ int kperm(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

template <int D> struct BCfg {
    static constexpr int WAVES = 4;
    static constexpr int NT = 256;
    static constexpr int OWN = 32 * WAVES;              // rows a work-group owns (queries for dq, keys for dkdv)
    static constexpr int BT = 64;                       // rows per streamed tile
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = (D + 31) / 32;
    static constexpr int CPR = D / 8;
    static constexpr int CPRP = CPR <= 8 ? 8 : 16;
    static constexpr int ROWB = CPRP * 16;
    static constexpr int TILEB = BT * ROWB;
    static constexpr int XOFF = 0;                      // stage s: tile X at s * STAGE, tile Y at s * STAGE + TILEB
    static constexpr int YOFF = TILEB;
    static constexpr int ROFF = 2 * TILEB;              // two rows of BT floats (lse, D of the tile's queries)
    static constexpr int STAGE = 2 * TILEB + 2 * BT * 4;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int IT = TILEB / (16 * NT);        // direct-load rounds per tile and thread
    static __device__ __forceinline__ int uswz(int r) {
        return CPRP == 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    }
    static_assert(IT >= 1 && TILEB % (16 * NT) == 0, "a tile is a whole number of load rounds");
    static_assert(DBLK * 4 <= CPRP, "transpose reads of the padded head dim stay inside a row");
};

typedef __fp16 lds_v4h_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) lds_v4h_t* lds_v4h_ptr;
typedef __attribute__((address_space(3))) unsigned char* lds_bytes;

__device__ __forceinline__ u32x2_t lds_read_tr(unsigned addr) {
    const lds_v4h_t t = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4h_ptr)(lds_bytes)(size_t)addr);
    return __builtin_bit_cast(u32x2_t, t);
}

__device__ __forceinline__ u32x4_t lds_read16(unsigned addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((lds_bytes)(size_t)addr);
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

#if defined(__HIP_DEVICE_COMPILE__)

// Work-group id -> (head, group), each XCD taking a contiguous run (as in the forward).
__device__ __forceinline__ void map_workgroup(const BwdArgs& a, int& bh, int& grp) {
    const int T = a.ngroups * a.BH;
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int vidx = xcd * (T >> 3) + min(xcd, T & 7) + (L >> 3);
    bh = vidx / a.ngroups;
    grp = vidx - bh * a.ngroups;
}

// Shared per-wave machinery: the two streamed tiles X, Y of a stage, the
// direct-load offsets, and the LDS addresses of row reads (A operand rows in
// kperm order) and of transpose reads.
template <int D>
struct Streams {
    using C = BCfg<D>;
    int lane, wave, hf, n;
    unsigned lds0;
    unsigned lo_off[C::IT];      // direct-load offset of round `it` within a tile's rows (or out of range)
    unsigned ra[C::KSTEPS];      // row read: tile row kperm(n), logical chunk 2 ks + hf
    unsigned ta[2][C::DBLK];     // transpose read: rows r + 4 h of a 16-row group, 8 bytes of d-block db

    __device__ __forceinline__ void init(unsigned lds_base, int tid, int wave_) {
        lane = tid & 63;
        wave = wave_;
        hf = lane >> 5;
        n = lane & 31;
        lds0 = lds_base;
#pragma unroll
        for (int it = 0; it < C::IT; ++it) {
            const int slot = (it * C::WAVES + wave) * 64 + lane;
            const int r = slot / C::CPRP, p = slot % C::CPRP;
            const int kc = p ^ C::uswz(r);
            lo_off[it] = kc < C::CPR ? (unsigned)(r * D * 2 + kc * 16) : 0x80000000u;
        }
        {
            const int r = kperm(n);                           // rows r and r + 32 share the swizzle
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) ra[ks] = r * C::ROWB + (((2 * ks + hf) ^ C::uswz(r)) * 16);
        }
        {
            const int g16 = lane >> 4, s16 = lane & 15;
            const int r = 8 * (g16 >> 1) + (s16 >> 2);     // + 16 kk + 4 h
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int db = 0; db < C::DBLK; ++db) {
                    const int rr = r + 4 * h;                 // uswz(rr + 16 kk) == uswz(rr)
                    const int c = 4 * db + 2 * (g16 & 1) + ((s16 & 3) >> 1);
                    ta[h][db] = rr * C::ROWB + ((c ^ C::uswz(rr)) * 16) + 8 * (s16 & 1);
                }
        }
    }

    // this wave's share of rows t0 .. t0+63 of `src` (rows past `rows` read as zero) into tile `which`
    __device__ __forceinline__ void issue(const unsigned char* src, int rows, int t0, int stage, int which) const {
        const int bytes = max(0, (rows - t0) * D * 2);
        const eta_desc_t desc = buffer_desc(src + (size_t)t0 * D * 2, bytes);
        const unsigned region = lds0 + stage * C::STAGE + (which ? C::YOFF : C::XOFF);
#pragma unroll
        for (int it = 0; it < C::IT; ++it)
            load_lds16(desc, lo_off[it], 0, region + (unsigned)((it * C::WAVES + wave) * 64 * 16));
    }

    // BT consecutive floats src[t0 ..] (zero past `rows`) into float row `which` of
    // the stage: one 4-byte direct load per lane of wave 0
    __device__ __forceinline__ void issue_floats(const float* src, int rows, int t0, int stage, int which) const {
        if (wave != 0) return;
        const int bytes = max(0, (rows - t0) * 4);
        load_lds4(buffer_desc(src + t0, bytes), (unsigned)(lane * 4), lds0 + stage * C::STAGE + C::ROFF + which * C::BT * 4);
    }

    // 8 consecutive floats of float row `which` starting at row r0 (a multiple of 8)
    __device__ __forceinline__ void floats8(int stage, int which, int r0, float (&out)[8]) const {
        const unsigned addr = lds0 + stage * C::STAGE + C::ROFF + which * C::BT * 4 + r0 * 4;
        const u32x4_t x = lds_read16(addr), y = lds_read16(addr + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[i] = __uint_as_float(x[i]);
            out[4 + i] = __uint_as_float(y[i]);
        }
    }

    // row read of A-operand block sb (rows 32 sb .. of the tile), k-step ks
    __device__ __forceinline__ u32x4_t row(int stage, int which, int sb, int ks) const {
        return lds_read16(lds0 + stage * C::STAGE + (which ? C::YOFF : C::XOFF) + ra[ks] + sb * 32 * C::ROWB);
    }

    // transpose read: the 32 x 16 A operand (d-block db, tile rows 16 kk .. 16 kk + 15)
    __device__ __forceinline__ u32x4_t tr(int stage, int which, int kk, int db) const {
        const unsigned base = lds0 + stage * C::STAGE + (which ? C::YOFF : C::XOFF) + 16 * kk * C::ROWB;
        const u32x2_t lo = lds_read_tr(base + ta[0][db]);
        const u32x2_t hi = lds_read_tr(base + ta[1][db]);
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
};

#endif  // __HIP_DEVICE_COMPILE__

// ---- dQ: a work-group owns 128 queries and walks the key tiles --------------------
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = BCfg<D>;
    using E = Elem<DT>;
    constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, CPR = C::CPR;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    Streams<D> st;
    st.init((unsigned)(size_t)(lds_bytes)smem, tid, wave);
    const int N = a.N;
    int bh, grp;
    map_workgroup(a, bh, grp);
    const int nitems = CAUSAL && grp != a.ntile - 1 - grp ? 2 : 1;
    const size_t hoff = (size_t)bh * (size_t)N * CPR;
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(a.k + hoff);
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(a.v + hoff);

    for (int item = 0; item < nitems; ++item) {
        const int qt = CAUSAL ? (item == 0 ? a.ntile - 1 - grp : grp) : grp;
        const int q0 = qt * C::OWN;
        const int qw0 = q0 + 32 * wave;
        const int qi = qw0 + st.n;
        // the query's Q and dO rows (B operands of S^T and dP^T), its O row (for
        // D) and lse, loaded raw: no arithmetic on them before the first tile
        // loads are issued, so their latency overlaps those loads
        u32x4_t qf[KSTEPS], df[KSTEPS], of[KSTEPS];
        float lse_raw = 0.f;
        if (qi < N) {
            const u32x4_t* qs = a.q + hoff + (size_t)qi * CPR + st.hf;
            const u32x4_t* ds = a.dout + hoff + (size_t)qi * CPR + st.hf;
            const u32x4_t* os = a.o + hoff + (size_t)qi * CPR + st.hf;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                qf[ks] = qs[2 * ks];
                df[ks] = ds[2 * ks];
                of[ks] = os[2 * ks];
            }
            lse_raw = a.lse[(size_t)bh * N + qi];
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = df[ks] = of[ks] = u32x4_t{0, 0, 0, 0};
        }
        f32x16_t acc[DBLK];
#pragma unroll
        for (int db = 0; db < DBLK; ++db) acc[db] = f32x16_t{};

        const int kend = CAUSAL ? min(N, q0 + C::OWN) : N;
        const int nt = (kend + C::BT - 1) / C::BT;
        float nlse2 = 0.f;                             // -lse log2(e), set once the first tiles are issued
        float dlt = 0.f;                               // D_i, likewise
        auto step = [&](int stg, int j) {
            if (j + 1 < nt) {
                st.issue(kb, N, (j + 1) * C::BT, stg ^ 1, 0);
                st.issue(vb, N, (j + 1) * C::BT, stg ^ 1, 1);
            }
            const int kt0 = j * C::BT;
            if (qw0 < N && !(CAUSAL && kt0 > qw0 + 31)) {
                f32x16_t s[2], dp[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) s[sb] = dp[sb] = f32x16_t{};
                {
                    // rounds of one S and one dP MFMA, the K and V rows of round
                    // r+1 read before round r's MFMAs (scheduling fences keep them there)
                    constexpr int R = 2 * KSTEPS;
                    u32x4_t ko[2], vo[2];
                    ko[0] = st.row(stg, 0, 0, 0);
                    vo[0] = st.row(stg, 1, 0, 0);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        if (r + 1 < R) {
                            ko[(r + 1) & 1] = st.row(stg, 0, (r + 1) & 1, (r + 1) >> 1);
                            vo[(r + 1) & 1] = st.row(stg, 1, (r + 1) & 1, (r + 1) >> 1);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        s[r & 1] = E::mfma(ko[r & 1], qf[r >> 1], s[r & 1]);
                        dp[r & 1] = E::mfma(vo[r & 1], df[r >> 1], dp[r & 1]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // dS^T = P^T (dP^T - D); register i of block sb is key kt0 + 32 sb + 16 (i/8) + 8 hf + i%8
                const bool edge = (CAUSAL && kt0 + C::BT - 1 > qw0) || kt0 + C::BT > N;
                const int hi = (CAUSAL ? min(qi, N - 1) : N - 1) - (kt0 + 8 * st.hf);
                u32x4_t dsf[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int sb = kk >> 1, reg = 8 * (kk & 1) + i;
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][reg], a.c, nlse2));
                        float ds = p * (dp[sb][reg] - dlt);
                        if (edge && 32 * sb + 16 * (reg >> 3) + (reg & 7) > hi) ds = 0.f;
                        v[i] = ds;
                    }
                    dsf[kk] = u32x4_t{E::pack2(v[0], v[1]), E::pack2(v[2], v[3]), E::pack2(v[4], v[5]), E::pack2(v[6], v[7])};
                }
                // dQ^T += K^T dS^T
                {
                    constexpr int R = 4 * DBLK;
                    u32x4_t to[2];
                    to[0] = st.tr(stg, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        if (r + 1 < R) to[(r + 1) & 1] = st.tr(stg, 0, (r + 1) / DBLK, (r + 1) % DBLK);
                        __builtin_amdgcn_sched_barrier(0);
                        acc[r % DBLK] = E::mfma(to[r & 1], dsf[r / DBLK], acc[r % DBLK]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            wait_loads();
            __syncthreads();
        };
        st.issue(kb, N, 0, 0, 0);
        st.issue(vb, N, 0, 0, 1);
        wait_loads();
        __syncthreads();
        // the empty asm keeps the compiler from scaling lse (and so waiting for
        // its load) before the tile loads above are issued
        asm volatile("" : "+v"(lse_raw));
        nlse2 = -lse_raw * kLog2e;
        // D_i = sum_c dO_ic O_ic: this lane's half of the row, then the other
        // half's from the lane 32 away; written for the dK/dV kernel and the caller
        float dpart = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dpart = __builtin_fmaf(E::lo(df[ks][i]), E::lo(of[ks][i]), dpart);
                dpart = __builtin_fmaf(E::hi(df[ks][i]), E::hi(of[ks][i]), dpart);
            }
        dlt = pair_sum(dpart);
        if (st.hf == 0 && qi < N) a.delta[(size_t)bh * N + qi] = dlt;
        for (int j = 0; j < nt; j += 2) {
            step(0, j);
            if (j + 1 < nt) step(1, j + 1);
        }
        // dQ = scale * acc, rounded; lane = query, registers 4 g .. 4 g + 3 = d0 .. d0 + 3
        if (qi < N) {
            uint16_t* row = a.dq + ((size_t)bh * N + qi) * D;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = db * 32 + 8 * g + 4 * st.hf;
                    if (d0 < D)
                        *reinterpret_cast<u32x2_t*>(row + d0) =
                            u32x2_t{E::pack2(acc[db][4 * g] * a.scale, acc[db][4 * g + 1] * a.scale),
                                    E::pack2(acc[db][4 * g + 2] * a.scale, acc[db][4 * g + 3] * a.scale)};
                }
        }
    }
#endif
}

// ---- dK, dV: a work-group owns 128 keys and walks the query tiles -----------------
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_bwd_dkdv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = BCfg<D>;
    using E = Elem<DT>;
    constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, CPR = C::CPR;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    Streams<D> st;
    st.init((unsigned)(size_t)(lds_bytes)smem, tid, wave);
    const int N = a.N;
    int bh, grp;
    map_workgroup(a, bh, grp);
    const int nitems = CAUSAL && grp != a.ntile - 1 - grp ? 2 : 1;
    const size_t hoff = (size_t)bh * (size_t)N * CPR;
    const unsigned char* qb = reinterpret_cast<const unsigned char*>(a.q + hoff);
    const unsigned char* ob = reinterpret_cast<const unsigned char*>(a.dout + hoff);
    const float* lse_h = a.lse + (size_t)bh * N;
    const float* dl_h = a.delta + (size_t)bh * N;

    for (int item = 0; item < nitems; ++item) {
        const int kbk = CAUSAL ? (item == 0 ? grp : a.ntile - 1 - grp) : grp;
        const int k0 = kbk * C::OWN;
        const int kw0 = k0 + 32 * wave;
        const int kj = kw0 + st.n;                       // this lane's key
        u32x4_t kf[KSTEPS], vf[KSTEPS];
        if (kj < N) {
            const u32x4_t* ks_ = a.k + hoff + (size_t)kj * CPR + st.hf;
            const u32x4_t* vs_ = a.v + hoff + (size_t)kj * CPR + st.hf;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                kf[ks] = ks_[2 * ks];
                vf[ks] = vs_[2 * ks];
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) kf[ks] = vf[ks] = u32x4_t{0, 0, 0, 0};
        }
        f32x16_t dk[DBLK], dv[DBLK];
#pragma unroll
        for (int db = 0; db < DBLK; ++db) dk[db] = dv[db] = f32x16_t{};

        // query tiles from the one holding key k0 (causal) to the last
        const int t_lo = CAUSAL ? k0 / C::BT : 0;
        const int nt = (N + C::BT - 1) / C::BT;
        auto issue_tile = [&](int t, int stg) {
            st.issue(qb, N, t * C::BT, stg, 0);
            st.issue(ob, N, t * C::BT, stg, 1);
            st.issue_floats(lse_h, N, t * C::BT, stg, 0);
            st.issue_floats(dl_h, N, t * C::BT, stg, 1);
        };
        auto step = [&](int stg, int t) {
            if (t + 1 < nt) issue_tile(t + 1, stg ^ 1);
            const int qt0 = t * C::BT;
            if (kw0 < N && !(CAUSAL && qt0 + C::BT - 1 < kw0)) {
                f32x16_t s[2], dp[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) s[sb] = dp[sb] = f32x16_t{};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb) {
                        s[sb] = E::mfma(st.row(stg, 0, sb, ks), kf[ks], s[sb]);
                        dp[sb] = E::mfma(st.row(stg, 1, sb, ks), vf[ks], dp[sb]);
                    }
                // P and dS; register i of block sb is query qt0 + 32 sb + 16 (i/8) + 8 hf + i%8,
                // kept when it is < N and (causal) >= the key; its lse and D are
                // read from the stage (rows 32 sb + 16 (i/8) + 8 hf + 0..7).  The
                // exponent arguments are formed first, masked (edge tiles only,
                // one uniform branch) to -inf, then exponentiated.
                float dr[4][8];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    float lr[8];
                    st.floats8(stg, 0, 16 * kk + 8 * st.hf, lr);
                    st.floats8(stg, 1, 16 * kk + 8 * st.hf, dr[kk]);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int sb = kk >> 1, reg = 8 * (kk & 1) + i;
                        s[sb][reg] = __builtin_fmaf(s[sb][reg], a.c, -lr[i] * kLog2e);
                    }
                }
                if ((CAUSAL && qt0 < kw0 + 31) || qt0 + C::BT > N) {
                    const int lim = (CAUSAL ? kj : 0) - (qt0 + 8 * st.hf);   // keep rows r with r >= lim
                    const int top = N - (qt0 + 8 * st.hf);                     // and r < top
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                        for (int reg = 0; reg < 16; ++reg) {
                            const int r = 32 * sb + 16 * (reg >> 3) + (reg & 7);
                            if (r >= top || r < lim) s[sb][reg] = -__builtin_huge_valf();
                        }
                }
                u32x4_t pf[4], dsf[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    float pv[8], dv8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int sb = kk >> 1, reg = 8 * (kk & 1) + i;
                        const float p = __builtin_amdgcn_exp2f(s[sb][reg]);
                        pv[i] = p;
                        dv8[i] = p * (dp[sb][reg] - dr[kk][i]);
                    }
                    pf[kk] = u32x4_t{E::pack2(pv[0], pv[1]), E::pack2(pv[2], pv[3]), E::pack2(pv[4], pv[5]), E::pack2(pv[6], pv[7])};
                    dsf[kk] = u32x4_t{E::pack2(dv8[0], dv8[1]), E::pack2(dv8[2], dv8[3]), E::pack2(dv8[4], dv8[5]),
                                      E::pack2(dv8[6], dv8[7])};
                }
                // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int db = 0; db < DBLK; ++db) {
                        dv[db] = E::mfma(st.tr(stg, 1, kk, db), pf[kk], dv[db]);
                        dk[db] = E::mfma(st.tr(stg, 0, kk, db), dsf[kk], dk[db]);
                    }
            }
            wait_loads();
            __syncthreads();
        };
        issue_tile(t_lo, 0);
        wait_loads();
        __syncthreads();
        for (int t = t_lo; t < nt; t += 2) {
            step(0, t);
            if (t + 1 < nt) step(1, t + 1);
        }
        if (kj < N) {
            uint16_t* krow = a.dk + ((size_t)bh * N + kj) * D;
            uint16_t* vrow = a.dv + ((size_t)bh * N + kj) * D;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = db * 32 + 8 * g + 4 * st.hf;
                    if (d0 < D) {
                        *reinterpret_cast<u32x2_t*>(krow + d0) =
                            u32x2_t{E::pack2(dk[db][4 * g] * a.scale, dk[db][4 * g + 1] * a.scale),
                                    E::pack2(dk[db][4 * g + 2] * a.scale, dk[db][4 * g + 3] * a.scale)};
                        *reinterpret_cast<u32x2_t*>(vrow + d0) =
                            u32x2_t{E::pack2(dv[db][4 * g], dv[db][4 * g + 1]), E::pack2(dv[db][4 * g + 2], dv[db][4 * g + 3])};
                    }
                }
        }
    }
#endif
}

// --- host side ---------------------------------------------------------------

template <int D, int DT, bool CAUSAL>
hipError_t launch(BwdArgs a, hipStream_t s) {
    using C = BCfg<D>;
    const int ntile = (a.N + C::OWN - 1) / C::OWN;
    a.ntile = ntile;
    a.ngroups = CAUSAL ? (ntile + 1) / 2 : ntile;
    const dim3 grid((unsigned)a.ngroups * (unsigned)a.BH), block(C::NT);
    const hipError_t e = launch_kernel(attn_bwd_dq_kernel<D, DT, CAUSAL>, grid, block, s, a);
    if (e != hipSuccess) return e;
    return launch_kernel(attn_bwd_dkdv_kernel<D, DT, CAUSAL>, grid, block, s, a);
}

template <int D, int DT>
hipError_t dispatch_causal(const BwdArgs& a, int causal, hipStream_t s) {
    return causal ? launch<D, DT, true>(a, s) : launch<D, DT, false>(a, s);
}

template <int D>
hipError_t dispatch_dtype(const BwdArgs& a, int dtype, int causal, hipStream_t s) {
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

// Device scratch of attn_bwd_noalloc: D_i of up to kNoallocRows rows.  One copy
// per GPU (each device that loads the library holds its own, until the process
// ends); host code reaches it only through the address hipGetSymbolAddress
// returns for the current device, never through the array's name.
constexpr long long kNoallocRows = ATTN_BWD_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[kNoallocRows];

std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];   // per device, under g_scratch_mu

// The current device's scratch address, looked up once per device (with that
// device current) and kept; nullptr if the lookup fails.
float* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    return g_scratch_ptr[dev];
}

// Host-side checks shared by both entry points (delta is checked by attn_bwd).
int check_args(const void* q, const void* k, const void* v, const void* out, const void* lse, const void* dout,
               void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, int dtype) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 80 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    const long long bh = (long long)B * H;
    const long long ntile = ((long long)N + 127) / 128;
    if (bh > INT32_MAX || ntile * bh > INT32_MAX || (long long)N * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv) & 15u)
        return ATTN_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;
    const size_t tb = (size_t)bh * (size_t)N * (size_t)d * 2u, rb = (size_t)bh * (size_t)N * 4u;
    const void* ins[6] = {q, k, v, out, dout, lse};
    const size_t insz[6] = {tb, tb, tb, tb, tb, rb};
    void* outs[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], tb, ins[j], insz[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], tb, outs[j], tb)) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

// Both kernels with D_i in `delta`; arguments already checked.
int run(const void* q, const void* k, const void* v, const void* out, const void* lse, const void* dout, void* dq,
        void* dk, void* dv, float* delta, int B, int H, int N, int d, int causal, float scale, int dtype,
        void* stream) {
    BwdArgs a;
    a.q = static_cast<const u32x4_t*>(q);
    a.k = static_cast<const u32x4_t*>(k);
    a.v = static_cast<const u32x4_t*>(v);
    a.o = static_cast<const u32x4_t*>(out);
    a.dout = static_cast<const u32x4_t*>(dout);
    a.lse = static_cast<const float*>(lse);
    a.delta = delta;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.N = N;
    a.BH = B * H;
    a.ntile = 0;
    a.ngroups = 0;
    a.c = scale * kLog2e;
    a.scale = scale;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (d) {
        case 64: err = dispatch_dtype<64>(a, dtype, causal, s); break;
        case 80: err = dispatch_dtype<80>(a, dtype, causal, s); break;
        default: err = dispatch_dtype<128>(a, dtype, causal, s); break;
    }
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* lse, const void* dout,
                        void* dq, void* dk, void* dv, void* delta, int B, int H, int N, int d, int causal, float scale,
                        int dtype, void* stream) {
    if (!delta) return ATTN_ERR_NULL;
    const int st = check_args(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, dtype);
    if (st != ATTN_OK) return st;
    if ((uintptr_t)delta & 3u) return ATTN_ERR_ALIGN;
    const long long bh = (long long)B * H;
    const size_t tb = (size_t)bh * (size_t)N * (size_t)d * 2u, rb = (size_t)bh * (size_t)N * 4u;
    const void* others[9] = {q, k, v, out, dout, dq, dk, dv, lse};
    for (int j = 0; j < 9; ++j)
        if (overlaps(delta, rb, others[j], j < 8 ? tb : rb)) return ATTN_ERR_ALIAS;
    const int dev_status = check_device();
    if (dev_status != ATTN_OK) return dev_status;
    return run(q, k, v, out, lse, dout, dq, dk, dv, static_cast<float*>(delta), B, H, N, d, causal, scale, dtype,
               stream);
}

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* lse,
                                const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                                float scale, int dtype, void* stream) {
    // sizes past the array are refused first, before the checks that derive spans from them
    if (B >= 1 && H >= 1 && N >= 1 && (long long)B * H * N > kNoallocRows) return ATTN_ERR_SHAPE;
    const int st = check_args(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, causal, scale, dtype);
    if (st != ATTN_OK) return st;
    const int dev_status = check_device();
    if (dev_status != ATTN_OK) return dev_status;
    float* delta = device_scratch();
    if (delta == nullptr) return ATTN_ERR_DEVICE;
    // every D_i the dK/dV kernel reads is written by the dQ kernel of the same call
    // first, so nothing of the previous call's contents needs clearing
    return run(q, k, v, out, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, stream);
}
