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
#include <cstring>

#include "attn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

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

// Row of the K tile that feeds A-operand row m of the score MFMA.  With this
// permutation, accumulator register i of a lane in half h holds key
// 16*(i/8) + 8*h + (i%8) of the 32-key block.
__device__ __forceinline__ int kperm(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Tile configuration shared by the kernel and the host launcher.
template <int D> struct Cfg {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;             // threads per work-group
    static constexpr int BM = 32 * WAVES;             // queries per work-group (32 per wave)
    static constexpr int BN = 64;                     // keys per tile
    static constexpr int SB = BN / 32;                // 32-key score blocks per tile
    static constexpr int KSTEPS = D / 16;             // MFMA k-steps over the head dim
    static constexpr int DBLK = (D + 31) / 32;        // 32-row blocks of O^T
    static constexpr int DPAD = DBLK * 32;
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int KSTRIDE = D * 2 + 16;        // bytes per K row in LDS (one pad chunk)
    static constexpr int VSTRIDE = BN * 2 + 16;       // bytes per V^T row in LDS
    static constexpr int KBUF = BN * KSTRIDE;
    static constexpr int VBUF = DPAD * VSTRIDE;
    static constexpr int STAGE = KBUF + VBUF;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int KCH = BN * CPR;              // 16-byte chunks in a K tile
    static constexpr int KIT = (KCH + NT - 1) / NT;
    static constexpr int VG = (BN / 4) * CPR;         // 4-key x 8-column groups in a V tile
    static constexpr int VIT = (VG + NT - 1) / NT;
    static_assert(D % 16 == 0, "head dim must be a multiple of 16");
};

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_kernel(FwdArgs a) {
    using C = Cfg<D>;
    using E = Elem<DT>;
    constexpr int BN = C::BN, SB = C::SB, KSTEPS = C::KSTEPS, DBLK = C::DBLK, CPR = C::CPR;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const u32x4_t* Qh = a.q + hoff;
    const u32x4_t* Kh = a.k + hoff;
    const u32x4_t* Vh = a.v + hoff;

    // ---- Q fragments (B operand of S^T = K Q^T), loaded once
    u32x4_t qf[KSTEPS];
    if (qi < N) {
        const u32x4_t* src = Qh + (size_t)qi * CPR + hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = src[2 * ks] ^ a.qsign;
    } else {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
    }

    const int kend = CAUSAL ? min(N, q0 + C::BM) : N;
    const int nt = (kend + BN - 1) / BN;

    // ---- global -> register staging for one K/V tile
    u32x4_t kreg[C::KIT];
    u32x4_t vreg[C::VIT][4];
    auto gload = [&](int j) {
        const int kt0 = j * BN;
#pragma unroll
        for (int it = 0; it < C::KIT; ++it) {
            const int ch = tid + it * C::NT;
            if (C::KCH % C::NT == 0 || ch < C::KCH) {
                const int row = ch / CPR, col = ch - (ch / CPR) * CPR;
                const int key = kt0 + row;
                kreg[it] = key < N ? Kh[(size_t)key * CPR + col] : u32x4_t{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int it = 0; it < C::VIT; ++it) {
            const int g = tid + it * C::NT;
            if (C::VG % C::NT == 0 || g < C::VG) {
                const int kg = g % (BN / 4), dc = g / (BN / 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kt0 + 4 * kg + r;
                    vreg[it][r] = key < N ? Vh[(size_t)key * CPR + dc] : u32x4_t{0, 0, 0, 0};
                }
            }
        }
    };
    // ---- register staging -> LDS stage `buf` (K row-major, V transposed)
    auto lstore = [&](int buf) {
        unsigned char* kb = smem + buf * C::STAGE;
        unsigned char* vb = kb + C::KBUF;
#pragma unroll
        for (int it = 0; it < C::KIT; ++it) {
            const int ch = tid + it * C::NT;
            if (C::KCH % C::NT == 0 || ch < C::KCH) {
                const int row = ch / CPR, col = ch - (ch / CPR) * CPR;
                *reinterpret_cast<u32x4_t*>(kb + row * C::KSTRIDE + col * 16) = kreg[it];
            }
        }
#pragma unroll
        for (int it = 0; it < C::VIT; ++it) {
            const int g = tid + it * C::NT;
            if (C::VG % C::NT == 0 || g < C::VG) {
                const int kg = g % (BN / 4), dc = g / (BN / 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    unsigned lo, hi;
                    if (e & 1) {
                        lo = (vreg[it][0][w] >> 16) | (vreg[it][1][w] & 0xffff0000u);
                        hi = (vreg[it][2][w] >> 16) | (vreg[it][3][w] & 0xffff0000u);
                    } else {
                        lo = (vreg[it][0][w] & 0xffffu) | (vreg[it][1][w] << 16);
                        hi = (vreg[it][2][w] & 0xffffu) | (vreg[it][3][w] << 16);
                    }
                    *reinterpret_cast<u32x2_t*>(vb + (dc * 8 + e) * C::VSTRIDE + kg * 8) = u32x2_t{lo, hi};
                }
            }
        }
    };

    // ---- per-lane running state (one query row per lane, half the keys)
    f32x16_t o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
    float m = kNegInf;   // running max of scale*log2(e)*score, shared by both halves
    float l = 0.f;       // running sum over this half's keys
    const float c = a.c;
    const int krow = kperm(n);

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nt) gload(j + 1);

        const int kt0 = j * BN;
        const bool active = qw0 < N && (!CAUSAL || kt0 <= qw0 + 31);
        if (active) {
            const unsigned char* kb = smem + buf * C::STAGE;
            const unsigned char* vb = kb + C::KBUF;

            // S^T = K Q^T
            f32x16_t s[SB];
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) {
                s[sb] = f32x16_t{};
                const unsigned char* kr = kb + (sb * 32 + krow) * C::KSTRIDE + hf * 16;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(kr + ks * 32);
                    s[sb] = E::mfma(av, qf[ks], s[sb]);
                }
            }

            // masks: only diagonal tiles (causal) and the ragged last tile
            const bool need_mask = (CAUSAL && kt0 + BN - 1 > qw0) || (kt0 + BN > N);
            auto masked = [&](int sb, int i) {
                const int key = kt0 + sb * 32 + 16 * (i >> 3) + 8 * hf + (i & 7);
                return key >= N || (CAUSAL && key > qi);
            };

            // online softmax
            float mraw = kNegInf;
            if (need_mask) {
#pragma unroll
                for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, masked(sb, i) ? kNegInf : s[sb][i]);
            } else {
#pragma unroll
                for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, s[sb][i]);
            }
            mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
            const float mt = mraw > kNegInf ? mraw * c : kNegInf;
            const float mnew = fmaxf(m, mt);
            const float muse = mnew > kNegInf ? mnew : 0.f;
            const float alpha = __builtin_amdgcn_exp2f(m - muse);
            m = mnew;

            u32x4_t pf[2 * SB];   // P^T as B operands of the P.V k-steps (16 keys each)
            float rs = 0.f;
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) {
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], c, -muse));
                    if (need_mask) e = masked(sb, i) ? 0.f : e;
                    p[i] = e;
                    rs += e;
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    pf[2 * sb + hh] = u32x4_t{E::pack2(p[8 * hh + 0], p[8 * hh + 1]), E::pack2(p[8 * hh + 2], p[8 * hh + 3]),
                                              E::pack2(p[8 * hh + 4], p[8 * hh + 5]), E::pack2(p[8 * hh + 6], p[8 * hh + 7])};
            }
            l = l * alpha + rs;

            // O^T = alpha * O^T + V^T P^T
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                o[db] *= alpha;
                const unsigned char* vr = vb + (db * 32 + n) * C::VSTRIDE + hf * 16;
#pragma unroll
                for (int kk = 0; kk < 2 * SB; ++kk) {
                    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(vr + kk * 32);
                    o[db] = E::mfma(av, pf[kk], o[db]);
                }
            }
        }

        if (j + 1 < nt) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l)
    if (qw0 < N) {
        const float ltot = l + __shfl_xor(l, 32);
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
    a.c = std::fabs(scale) * kLog2e;
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
