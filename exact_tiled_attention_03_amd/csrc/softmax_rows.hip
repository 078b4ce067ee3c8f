// softmax_rows.hip -- standalone fused row softmax for gfx950 and its C ABI.
//
// Method: "Triton: CUDA-level operators in Python", example 2, and "CS336
// Lecture 6", Level 1: one program per row; the row is loaded once (positions
// past the row end count as -inf), its max and its sum of exp(x - max) are
// reduced on chip, and y = exp(x - max) / sum is written once.  Rows longer
// than a work-group holds in registers follow the same lecture's Level 2
// tiling of a row reduction, combined with the running-max rescaling of the
// online softmax ("Triton in depth", section 3.2): one pass over the tiles
// keeps a running (max, sum) per thread, a second pass writes the outputs.
//
// gfx950 mapping: a work-group of NT threads owns a row; each thread holds
// ITEMS vectors of it in registers, consecutive threads on consecutive vectors
// so that each load instruction of a wave covers one contiguous span of HBM
// (1 KB with 16-byte vectors).  Rows whose starts are 16-byte aligned use
// 16-byte vectors (4 fp32 or 8 fp16/bf16 values); others use one element per
// lane.  The reductions are a butterfly over the 64 lanes of a wave followed by
// one LDS exchange between waves.  exp is evaluated as exp2 with log2(e) folded
// into one FMA.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "launch.h"
#include "softmax.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One element type: scalar and 16-byte conversions to and from float.
template <int DT> struct Ty;

template <> struct Ty<ATTN_F32> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float get(const unsigned char* p) { return *reinterpret_cast<const float*>(p); }
    static __device__ __forceinline__ void put(unsigned char* p, float v) { *reinterpret_cast<float*>(p) = v; }
    static __device__ __forceinline__ void unpack(const u32x4_t& w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
    }
    static __device__ __forceinline__ u32x4_t pack(const float* f) {
        return u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};

template <> struct Ty<ATTN_F16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float get(const unsigned char* p) {
        return (float)*reinterpret_cast<const _Float16*>(p);
    }
    static __device__ __forceinline__ void put(unsigned char* p, float v) { *reinterpret_cast<_Float16*>(p) = (_Float16)v; }
    // element i of the vector is copied to a scalar before any bit reinterpretation
    static __device__ __forceinline__ float half_bits(unsigned bits16) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
    }
    static __device__ __forceinline__ void unpack(const u32x4_t& w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned u = w[i];
            f[2 * i] = half_bits(u & 0xffffu);
            f[2 * i + 1] = half_bits(u >> 16);
        }
    }
    // two floats rounded to nearest even, packed low/high; the whole 2-vector is
    // reinterpreted, never one of its elements
    static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
        f16x2_t h;
        h[0] = (_Float16)lo;
        h[1] = (_Float16)hi;
        return __builtin_bit_cast(unsigned, h);
    }
    static __device__ __forceinline__ u32x4_t pack(const float* f) {
        return u32x4_t{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
    }
};

template <> struct Ty<ATTN_BF16> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float get(const unsigned char* p) {
        return __uint_as_float((unsigned)*reinterpret_cast<const unsigned short*>(p) << 16);
    }
    static __device__ __forceinline__ void put(unsigned char* p, float v) { *reinterpret_cast<__bf16*>(p) = (__bf16)v; }
    static __device__ __forceinline__ void unpack(const u32x4_t& w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
        bf16x2_t h;
        h[0] = (__bf16)lo;
        h[1] = (__bf16)hi;
        return __builtin_bit_cast(unsigned, h);
    }
    static __device__ __forceinline__ u32x4_t pack(const float* f) {
        return u32x4_t{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
    }
};

// A lane's unit of a row segment: N consecutive elements starting at element
// c0 of the segment that starts at `seg` (a uniform pointer), one 16-byte
// access when WIDE, else a single element.  Elements at or past `n` (the
// segment's valid length) read as -inf and are never written.  Indices are
// 32-bit, so the address is the uniform base plus one 32-bit lane offset.
// Loads marked LAST are the row's final read and stores are never read back
// by this kernel: both go out as nontemporal (streaming) accesses.
template <int DT, bool WIDE> struct Unit {
    using T = Ty<DT>;
    static constexpr int N = WIDE ? 16 / T::kBytes : 1;
    template <bool LAST>
    static __device__ __forceinline__ void load(const unsigned char* seg, int c0, int n, float (&f)[N]) {
        if (c0 + N <= n) {
            if constexpr (WIDE) {
                const u32x4_t* p = reinterpret_cast<const u32x4_t*>(seg + (unsigned)c0 * T::kBytes);
                T::unpack(LAST ? __builtin_nontemporal_load(p) : *p, f);
            } else {
                f[0] = T::get(seg + (unsigned)c0 * T::kBytes);
            }
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) f[e] = c0 + e < n ? T::get(seg + (unsigned)(c0 + e) * T::kBytes) : kNegInf;
        }
    }
    static __device__ __forceinline__ void store(unsigned char* seg, int c0, int n, const float (&f)[N]) {
        if (c0 + N <= n) {
            if constexpr (WIDE) __builtin_nontemporal_store(T::pack(f), reinterpret_cast<u32x4_t*>(seg + (unsigned)c0 * T::kBytes));
            else T::put(seg + (unsigned)c0 * T::kBytes, f[0]);
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e)
                if (c0 + e < n) T::put(seg + (unsigned)(c0 + e) * T::kBytes, f[e]);
        }
    }
};

struct SmArgs {
    const unsigned char* x;
    unsigned char* y;
    long long xs, ys;   // row strides in bytes
    long long rows;
    int cols;
};

#if defined(__HIP_DEVICE_COMPILE__)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Work-group reduction through one LDS slot per wave; every thread gets the result.
template <int NT, bool MAX>
__device__ __forceinline__ float group_reduce(float v, float* red) {
    constexpr int NW = NT / 64;
    v = MAX ? wave_max(v) : wave_sum(v);
    if constexpr (NW == 1) return v;
    const int wave = threadIdx.x >> 6;
    __syncthreads();                       // every wave has read the previous contents of red[]
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

#endif  // __HIP_DEVICE_COMPILE__

// One row per work-group with the whole row in registers: thread t holds units
// t, t + NT, ..., t + (ITEMS-1) NT.  The grid walks the rows with a stride of
// its size.  The row is read once, so its loads are streaming.
template <int DT, bool WIDE, int NT, int ITEMS>
__global__ __launch_bounds__(NT) void softmax_row_kernel(SmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using U = Unit<DT, WIDE>;
    constexpr int N = U::N;
    __shared__ float red[NT / 64];
    const int t = threadIdx.x;
    const int cols = a.cols;
    for (long long r = blockIdx.x; r < a.rows; r += gridDim.x) {
        const unsigned char* xr = a.x + r * a.xs;
        unsigned char* yr = a.y + r * a.ys;
        float f[ITEMS][N];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) U::template load<true>(xr, (it * NT + t) * N, cols, f[it]);
        float mx = kNegInf;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it)
#pragma unroll
            for (int e = 0; e < N; ++e) mx = fmaxf(mx, f[it][e]);
        mx = group_reduce<NT, true>(mx, red);
        const float nm = -mx * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it)
#pragma unroll
            for (int e = 0; e < N; ++e) {
                f[it][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[it][e], kLog2e, nm));   // -inf -> 0
                sum += f[it][e];
            }
        sum = group_reduce<NT, false>(sum, red);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
#pragma unroll
            for (int e = 0; e < N; ++e) f[it][e] *= inv;
            U::store(yr, (it * NT + t) * N, cols, f[it]);
        }
    }
#endif
}

// Rows too long for registers: tiles of NT * N * TI elements.  Pass 1 keeps a
// running max m and a running sum l of exp(x - m) per thread; when a tile
// raises m, l is first multiplied by exp(old m - new m).  Each tile's partial
// sum (TI * N terms) is added to l with compensated (Kahan) summation, so the
// rounding error of l does not grow with the row length.  The work-group then
// combines the threads' (m, l) pairs, and pass 2 reads the row again and
// writes exp(x - max) / sum.  Pass 1 loads are ordinary, so that the L2 and
// the last-level cache may still hold part of the row for pass 2; pass 2
// loads are streaming.
template <int DT, bool WIDE, int NT, int TI>
__global__ __launch_bounds__(NT) void softmax_row_tiled_kernel(SmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using U = Unit<DT, WIDE>;
    constexpr int N = U::N;
    constexpr int TILE = NT * N * TI;
    __shared__ float red[NT / 64];
    const int t = threadIdx.x;
    const long long cols = a.cols;
    for (long long r = blockIdx.x; r < a.rows; r += gridDim.x) {
        const unsigned char* xr = a.x + r * a.xs;
        unsigned char* yr = a.y + r * a.ys;
        float m = kNegInf, l = 0.f, comp = 0.f;   // l + comp: running sum of exp(x - m)
        for (long long base = 0; base < cols; base += TILE) {
            const unsigned char* xt = xr + base * U::T::kBytes;
            const int n = cols - base < TILE ? (int)(cols - base) : TILE;
            float f[TI][N];
#pragma unroll
            for (int it = 0; it < TI; ++it) U::template load<false>(xt, (it * NT + t) * N, n, f[it]);
            float tm = m;
#pragma unroll
            for (int it = 0; it < TI; ++it)
#pragma unroll
                for (int e = 0; e < N; ++e) tm = fmaxf(tm, f[it][e]);
            if (tm > m) {                                                 // -inf never exceeds m
                const float s = __builtin_amdgcn_exp2f((m - tm) * kLog2e);   // 0 when m was -inf
                l *= s;
                comp *= s;
                m = tm;
            }
            const float nm = m > kNegInf ? -m * kLog2e : 0.f;
            float part = 0.f;
#pragma unroll
            for (int it = 0; it < TI; ++it)
#pragma unroll
                for (int e = 0; e < N; ++e) part += __builtin_amdgcn_exp2f(__builtin_fmaf(f[it][e], kLog2e, nm));
            const float yv = part - comp;
            const float nl = l + yv;
            comp = (nl - l) - yv;
            l = nl;
        }
        const float gm = group_reduce<NT, true>(m, red);
        const float mine = m > kNegInf ? l * __builtin_amdgcn_exp2f((m - gm) * kLog2e) : 0.f;
        const float inv = 1.0f / group_reduce<NT, false>(mine, red);
        const float nm = -gm * kLog2e;
        for (long long base = 0; base < cols; base += TILE) {
            const unsigned char* xt = xr + base * U::T::kBytes;
            unsigned char* yt = yr + base * U::T::kBytes;
            const int n = cols - base < TILE ? (int)(cols - base) : TILE;
#pragma unroll
            for (int it = 0; it < TI; ++it) {
                const int c0 = (it * NT + t) * N;
                float f[N];
                U::template load<true>(xt, c0, n, f);
#pragma unroll
                for (int e = 0; e < N; ++e) f[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], kLog2e, nm)) * inv;
                U::store(yt, c0, n, f);
            }
        }
    }
#endif
}

// --- host side ---------------------------------------------------------------

// A thread holds at most 64 values of its row, which keeps a 1024-thread
// work-group within 128 VGPRs: rows up to 65536 elements stay in registers,
// longer ones take the tiled kernel.
constexpr int kMaxVals = 64;
// one work-group per row up to this many rows, then a stride loop over rows
constexpr long long kMaxGroups = 1LL << 16;

unsigned grid_for(long long rows) { return (unsigned)(rows < kMaxGroups ? rows : kMaxGroups); }

template <int DT, bool WIDE, int NT, int ITEMS>
hipError_t launch_row(const SmArgs& a, hipStream_t s) {
    return launch_kernel(softmax_row_kernel<DT, WIDE, NT, ITEMS>, dim3(grid_for(a.rows)), dim3(NT), s, a);
}

template <int DT, bool WIDE, int NT>
hipError_t launch_items(const SmArgs& a, int items, hipStream_t s) {
    constexpr int N = Unit<DT, WIDE>::N;
    switch (items) {
        case 1: return launch_row<DT, WIDE, NT, 1>(a, s);
        case 2: return launch_row<DT, WIDE, NT, 2>(a, s);
        case 4: return launch_row<DT, WIDE, NT, 4>(a, s);
        case 8: return launch_row<DT, WIDE, NT, 8>(a, s);
        case 16:
            if constexpr (16 * N <= kMaxVals) return launch_row<DT, WIDE, NT, 16>(a, s);
            break;
        case 32:
            if constexpr (32 * N <= kMaxVals) return launch_row<DT, WIDE, NT, 32>(a, s);
            break;
        case 64:
            if constexpr (64 * N <= kMaxVals) return launch_row<DT, WIDE, NT, 64>(a, s);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

int pow2_at_least(long long v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

template <int DT, bool WIDE>
hipError_t dispatch(const SmArgs& a, hipStream_t s) {
    constexpr int N = Unit<DT, WIDE>::N;
    constexpr int IMAX = kMaxVals / N;
    const long long nu = ((long long)a.cols + N - 1) / N;   // units per row
    // the smallest work-group whose threads cover the row with at most IMAX
    // units each, then the fewest units per thread (a power of two) that do:
    // more units per thread and fewer waves per row measured faster (fewer
    // waves to synchronise per row, more loads in flight per wave)
    if (nu <= 64LL * IMAX) return launch_items<DT, WIDE, 64>(a, pow2_at_least((nu + 63) / 64), s);
    if (nu <= 256LL * IMAX) return launch_items<DT, WIDE, 256>(a, pow2_at_least((nu + 255) / 256), s);
    if (nu <= 512LL * IMAX) return launch_items<DT, WIDE, 512>(a, pow2_at_least((nu + 511) / 512), s);
    if (nu <= 1024LL * IMAX) return launch_items<DT, WIDE, 1024>(a, pow2_at_least((nu + 1023) / 1024), s);
    constexpr int TI = WIDE ? 4 : 16;   // 16-byte vectors: 4 per tile; elements: 16 per tile
    return launch_kernel(softmax_row_tiled_kernel<DT, WIDE, 1024, TI>, dim3(grid_for(a.rows)), dim3(1024), s, a);
}

template <int DT>
hipError_t dispatch_layout(const SmArgs& a, bool wide, hipStream_t s) {
    return wide ? dispatch<DT, true>(a, s) : dispatch<DT, false>(a, s);
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

}  // namespace

extern "C" int softmax_rows(const void* x, long long x_stride, void* y, long long y_stride, int rows, int cols, int dtype,
                            void* stream) {
    if (!x || !y) return ATTN_ERR_NULL;
    if (rows < 1 || cols < 1 || x_stride < cols || y_stride < cols) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    const long long es = dtype == ATTN_F32 ? 4 : 2;
    // no buffer may span more than 2^48 bytes (far beyond any device memory);
    // this also keeps every byte offset below within long long
    constexpr long long kMaxSpan = 1LL << 48;
    if (x_stride > kMaxSpan / es || y_stride > kMaxSpan / es) return ATTN_ERR_SHAPE;
    const long long xs = x_stride * es, ys = y_stride * es;
    if ((long long)(rows - 1) > kMaxSpan / xs || (long long)(rows - 1) > kMaxSpan / ys) return ATTN_ERR_SHAPE;
    const uintptr_t xb = (uintptr_t)x, yb = (uintptr_t)y;
    if ((xb | yb) % (uintptr_t)es) return ATTN_ERR_ALIGN;
    // the byte spans [first row start, last row end); exactly in place is allowed,
    // any other overlap of the spans is not
    const uintptr_t xe = xb + (uintptr_t)((rows - 1) * xs + cols * es);
    const uintptr_t ye = yb + (uintptr_t)((rows - 1) * ys + cols * es);
    const bool in_place = xb == yb && xs == ys;
    if (!in_place && xb < ye && yb < xe) return ATTN_ERR_ALIAS;
    const int dev_status = check_device();
    if (dev_status != ATTN_OK) return dev_status;

    SmArgs a;
    a.x = static_cast<const unsigned char*>(x);
    a.y = static_cast<unsigned char*>(y);
    a.xs = xs;
    a.ys = ys;
    a.rows = rows;
    a.cols = cols;
    // 16-byte accesses need every row start of x and y on a 16-byte boundary
    // (a single row has only the one start, whatever the strides say)
    const bool wide = ((xb | yb) % 16 == 0) && (rows == 1 || (xs % 16 == 0 && ys % 16 == 0));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (dtype) {
        case ATTN_F32: err = dispatch_layout<ATTN_F32>(a, wide, s); break;
        case ATTN_BF16: err = dispatch_layout<ATTN_BF16>(a, wide, s); break;
        default: err = dispatch_layout<ATTN_F16>(a, wide, s); break;
    }
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
