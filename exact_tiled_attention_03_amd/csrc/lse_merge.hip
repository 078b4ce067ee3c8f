// lse_merge.hip -- merge of attention results computed over disjoint key shards,
// for gfx950, and its C ABI.
//
// From the definition of lse (natural log of a row's softmax denominator): the
// shards' (O_g, lse_g) combine as lse = ln sum_g exp(lse_g) and
// O = sum_g exp(lse_g - lse) O_g.  Evaluated with m = max_g lse_g (kept as a
// running max, partial sums rescaled when it grows), w_g = exp2((lse_g - m)
// log2 e), O = (sum_g w_g O_g) / sum_g w_g, lse = m + ln sum_g w_g, all in
// fp32; a shard with lse_g = -inf has w_g = 0.
//
// gfx950 mapping: HBM-bound; 16 lanes own a row (one 16-byte chunk of 8
// values each, d <= 128), so one wave merges 4 rows and every load of a shard
// row is a contiguous 16-byte-per-lane access.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "attn_bwd.h"
#include "launch.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int DT> struct Ty;

template <> struct Ty<ATTN_F16> {
    static __device__ __forceinline__ float lo(unsigned u) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
    }
    static __device__ __forceinline__ float hi(unsigned u) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16)); }
    static __device__ __forceinline__ unsigned pack2(float a, float b) {
        f16x2_t p;
        p[0] = (_Float16)a;
        p[1] = (_Float16)b;
        return __builtin_bit_cast(unsigned, p);
    }
};

template <> struct Ty<ATTN_BF16> {
    static __device__ __forceinline__ float lo(unsigned u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
    static __device__ __forceinline__ unsigned pack2(float a, float b) {
        bf16x2_t p;
        p[0] = (__bf16)a;
        p[1] = (__bf16)b;
        return __builtin_bit_cast(unsigned, p);
    }
};

struct MergeArgs {
    const u32x4_t* o_parts;   // [G, R, CPR] 16-byte chunks
    const float* lse_parts;   // [G, R]
    u32x4_t* o;               // [R, CPR]
    float* lse;               // [R]
    long long R;
    int G, CPR;
};

// One pass over the shards, four at a time (their loads in flight together),
// with a running max m: when a shard's lse exceeds m, the partial sums are
// first multiplied by exp(m_old - m_new), as in the online softmax.
template <int DT>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using T = Ty<DT>;
    constexpr int U = 8;   // shards whose loads are issued together
    // the parts (read once) and the result (written once) bypass the caches
    const int sub = threadIdx.x & 15;
    const bool own = sub < a.CPR;
    const long long stride = (long long)gridDim.x * 16;
    for (long long r = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4; r < a.R; r += stride) {
        float m = kNegInf, tot = 0.f;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int g0 = 0; g0 < a.G; g0 += U) {
            float lg[U];
            u32x4_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = g0 + u;
                lg[u] = g < a.G ? a.lse_parts[(long long)g * a.R + r] : kNegInf;
                const u32x4_t* src = a.o_parts + ((long long)g * a.R + r) * a.CPR + sub;
                v[u] = u32x4_t{0, 0, 0, 0};
                if (g < a.G && own) v[u] = __builtin_nontemporal_load(src);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (lg[u] > m) {                                   // -inf never exceeds m
                    const float sc = __builtin_amdgcn_exp2f((m - lg[u]) * kLog2e);   // 0 while m is -inf
                    tot *= sc;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] *= sc;
                    m = lg[u];
                }
                const float w = lg[u] > kNegInf ? __builtin_amdgcn_exp2f((lg[u] - m) * kLog2e) : 0.f;
                tot += w;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned x = v[u][i];
                    acc[2 * i] = __builtin_fmaf(w, T::lo(x), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(w, T::hi(x), acc[2 * i + 1]);
                }
            }
        }
        const float inv = tot > 0.f ? 1.0f / tot : 0.f;
        const u32x4_t res{T::pack2(acc[0] * inv, acc[1] * inv), T::pack2(acc[2] * inv, acc[3] * inv),
                          T::pack2(acc[4] * inv, acc[5] * inv), T::pack2(acc[6] * inv, acc[7] * inv)};
        if (own) __builtin_nontemporal_store(res, a.o + r * a.CPR + sub);
        if (sub == 0) a.lse[r] = m > kNegInf ? m + __builtin_amdgcn_logf(tot) * kLn2 : kNegInf;
    }
#endif
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

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

}  // namespace

extern "C" int attn_lse_merge(const void* o_parts, const void* lse_parts, int G, void* o, void* lse, long long R,
                              int d, int dtype, void* stream) {
    if (!o_parts || !lse_parts || !o || !lse) return ATTN_ERR_NULL;
    if (G < 1 || R < 1 || R > (1LL << 40) / G) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 80 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (((uintptr_t)o_parts | (uintptr_t)o) % 16 || ((uintptr_t)lse_parts | (uintptr_t)lse) % 4) return ATTN_ERR_ALIGN;
    const uintptr_t op0 = (uintptr_t)o_parts, op1 = op0 + (uintptr_t)(G * R * d * 2);
    const uintptr_t lp0 = (uintptr_t)lse_parts, lp1 = lp0 + (uintptr_t)(G * R * 4);
    const uintptr_t o0 = (uintptr_t)o, o1 = o0 + (uintptr_t)(R * d * 2);
    const uintptr_t l0 = (uintptr_t)lse, l1 = l0 + (uintptr_t)(R * 4);
    if (overlaps(o0, o1, op0, op1) || overlaps(o0, o1, lp0, lp1) || overlaps(l0, l1, op0, op1) ||
        overlaps(l0, l1, lp0, lp1) || overlaps(o0, o1, l0, l1))
        return ATTN_ERR_ALIAS;
    const int dev_status = check_device();
    if (dev_status != ATTN_OK) return dev_status;
    MergeArgs a;
    a.o_parts = static_cast<const u32x4_t*>(o_parts);
    a.lse_parts = static_cast<const float*>(lse_parts);
    a.o = static_cast<u32x4_t*>(o);
    a.lse = static_cast<float*>(lse);
    a.R = R;
    a.G = G;
    a.CPR = d / 8;
    const long long groups = (R + 15) / 16;
    const dim3 grid((unsigned)(groups < 65536 ? groups : 65536)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == ATTN_BF16 ? launch_kernel(lse_merge_kernel<ATTN_BF16>, grid, block, s, a)
                                            : launch_kernel(lse_merge_kernel<ATTN_F16>, grid, block, s, a);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
