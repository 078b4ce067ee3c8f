// gemm.hip -- tiled matrix product with a fused bias + activation epilogue for
// gfx950 (MI355X), and its C ABI.
//
// Method: "Triton: CUDA-level operators in Python", example 3, and "CS336
// Lecture 6", Level 3: a work-group computes one BM x BN tile of C, walking K
// in BK steps and accumulating in fp32; the element-wise epilogue (bias of
// "Triton core syntax" 4.4, then ReLU or tanh-GELU) is applied to the finished
// tile in registers before its single store, so the unactivated product never
// reaches HBM.  The grouped launch order of example 3 (GROUP_M tile rows
// share the B panels they load) decides which tile a work-group takes.
//
// gfx950 mapping (not taken from the pages, which target NVIDIA tensor cores):
//
//  * 256 x 256 tiles, BK = 64, eight waves (two per SIMD) in a 2 (n) x 4 (m)
//    grid, each wave 128 n x 64 m = 4 x 2 blocks of v_mfma_f32_32x32x16.
//  * The two waves of a SIMD belong to two groups that alternate between
//    reading a k tile's operands from LDS into registers and running its
//    MFMAs from registers (gemm_kernel_pp), so one issues MFMAs while the other
//    reads LDS; the next tile's loads are spread over both phases.
//  * The MFMA produces C^T: the A operand is a 32-row block of B^T (n, k) and
//    the B operand a 32-column block of A^T (k, m).  In the 32 x 32
//    accumulator layout a lane then owns one m and runs of 4 consecutive n,
//    so the epilogue stages each wave's block through LDS and stores whole
//    256-byte row segments (8 contiguous bytes per lane without 16-byte
//    aligned C).
//  * A and B tiles go from HBM straight into LDS (buffer loads with the LDS
//    destination), two stages of 64 KB; rows of 128 bytes, 16-byte chunks
//    XOR-swizzled by row so the operand reads are free of bank conflicts.
//    B stored K x N (rows of N) is read through the gfx950 transpose load.
//  * Edges: buffer range checks return zero past the last row of a panel;
//    16-byte chunks at or past K are redirected out of range, so they read
//    as zero in both operands; rows and columns past M, N are never stored.
//  * Work-group ids are dealt round-robin over the 8 XCDs; they are remapped
//    so that each XCD takes a contiguous run of the grouped order, keeping
//    the A and B panels its tiles share in its own L2.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "gemm.h"
#include "launch.h"
#include "lds_load.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

template <int DT> struct Elem;

template <> struct Elem<ATTN_F16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
    }
    // two floats rounded to nearest even, packed low/high
    static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
        f16x2_t p;
        p[0] = (_Float16)lo;
        p[1] = (_Float16)hi;
        return __builtin_bit_cast(unsigned, p);
    }
    static __device__ __forceinline__ float get(const unsigned char* p) {
        return (float)*reinterpret_cast<const _Float16*>(p);
    }
    static __device__ __forceinline__ void put(unsigned char* p, float v) { *reinterpret_cast<_Float16*>(p) = (_Float16)v; }
};

template <> struct Elem<ATTN_BF16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
        bf16x2_t p;
        p[0] = (__bf16)lo;
        p[1] = (__bf16)hi;
        return __builtin_bit_cast(unsigned, p);
    }
    static __device__ __forceinline__ float get(const unsigned char* p) {
        return __uint_as_float((unsigned)*reinterpret_cast<const unsigned short*>(p) << 16);
    }
    static __device__ __forceinline__ void put(unsigned char* p, float v) { *reinterpret_cast<__bf16*>(p) = (__bf16)v; }
};

// Tile configuration.
//
// LDS stage s (s = 0, 1) at s * STAGE holds the A tile (BM rows of m, BK values
// of k) at AOFF and the B tile at BOFF.  K-contiguous tiles are BM (or BN) rows
// of 128 bytes; chunk c (8 values of k) of row r sits at c ^ swz(r) with
// swz(r) = (r / 2) % 8: the 16 rows read by 16 lanes at one logical chunk then
// cover 16 distinct 16-byte slots of a 256-byte bank line.  B stored K x N is
// BK rows (k) of BN values of n (512 bytes); its 64-byte granule g of row r
// sits at g ^ (r % 8), so the transpose reads of 16 lanes (4 rows x 4 granule
// offsets) spread over the banks.
// C rows are stored with the non-temporal hint (written once, not read back).

// WAVES waves per work-group in a WAVES_N (along n) x WAVES / WAVES_N (along m)
// grid; K in steps of BK (64 or 32) through STAGES LDS stages
template <int WAVES_, int WAVES_N_, int BK_, int STAGES_>
struct Cfg {
    static constexpr int WAVES = WAVES_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BM = 256, BN = 256, BK = BK_;
    static constexpr int WN = BN / WAVES_N, WM = BM / (WAVES / WAVES_N);   // per wave
    static constexpr int MB = WM / 32, NB = WN / 32;
    static constexpr int KS = BK / 16;     // MFMA k-steps per stage
    static constexpr int ROWB = BK * 2;    // bytes per K-contiguous row
    static constexpr int CPRK = BK / 8;    // 16-byte chunks per K-contiguous row
    static constexpr int RPL = 256 / ROWB; // K-contiguous rows per 256-byte bank line
    static constexpr int AOFF = 0;
    static constexpr int BOFF = BM * ROWB;
    static constexpr int STAGE = BOFF + BN * BK * 2;
    static constexpr int LDS = STAGES * STAGE;
    static constexpr int ROUNDS = BM * ROWB / (16 * NT);   // direct-load rounds per tile (A and B alike)
    static constexpr int LOADS = 2 * ROUNDS;               // direct loads per tile and wave
    static constexpr int GROUP_M = 4;                // tile rows per group of the launch order
    static_assert(BK == 32 || BK == 64, "k step");
    static_assert(BN * BK * 2 == BM * ROWB, "both tiles take the same number of load rounds");
    static_assert(WAVES % WAVES_N == 0 && WM % 32 == 0 && WN % 32 == 0, "wave layouts");
    static_assert((NT / CPRK / RPL) % CPRK == 0 && (NT / 32) % 8 == 0, "load rounds keep every lane's swizzle");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(WAVES * WM * WN * 2 <= LDS && WN == 128, "the epilogue's per-wave C slices (rows of 256 bytes) fit in the stages");
};
using Shape = Cfg<4, 2, 64, 2>;   // the tile shape (BM, BN, GROUP_M) shared by every configuration

struct GemmArgs {
    const unsigned char* a;
    const unsigned char* b;
    const unsigned char* bias;   // may be null
    unsigned char* c;
    long long lda, ldb, ldc;     // in bytes
    int M, N, K;
    int act;
    int tm, tn;                  // tile rows (of M) and tile columns (of N)
    int c_vec;                   // 8-byte C stores allowed (c and ldc 8-byte aligned)
    int c_vec16;                 // 16-byte C stores allowed (c and ldc 16-byte aligned)
};

typedef __fp16 lds_v4h_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) lds_v4h_t* lds_v4h_ptr;
typedef __attribute__((address_space(3))) unsigned char* lds_bytes;

__device__ __forceinline__ u32x4_t lds_read16(unsigned addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((lds_bytes)(size_t)addr);
}

// 8 bytes through the gfx950 transpose read: within each 16-lane group, lane i
// receives element (i % 4) of the 8-byte rows addressed by lanes i/4, i/4 + 4,
// i/4 + 8, i/4 + 12.
__device__ __forceinline__ u32x2_t lds_read_tr(unsigned addr) {
    const lds_v4h_t t = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4h_ptr)(lds_bytes)(size_t)addr);
    return __builtin_bit_cast(u32x2_t, t);
}


#if defined(__HIP_DEVICE_COMPILE__)

// Work-group id -> (tile row, tile column).  Ids are dealt round-robin over the
// 8 XCDs; the remap gives XCD x a contiguous range of the grouped order, which
// walks GROUP_M tile rows column by column (example 3's L2 grouping).
__device__ __forceinline__ void map_tile(const GemmArgs& g, int& tile_m, int& tile_n) {
    const int T = g.tm * g.tn;
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int v = xcd * (T >> 3) + min(xcd, T & 7) + (L >> 3);
    const int per_group = Shape::GROUP_M * g.tn;
    const int first = (v / per_group) * Shape::GROUP_M;
    const int gs = min(g.tm - first, Shape::GROUP_M);
    const int w = v - (v / per_group) * per_group;
    tile_m = first + w % gs;
    tile_n = w / gs;
}

__device__ __forceinline__ float gelu_tanh(float z) {
    // tanh(u) = 1 - 2 / (1 + e^(2u)): +-1 at the extremes, no overflow trouble
    const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
    const float e = __builtin_amdgcn_exp2f(2.0f * kLog2e * u);
    const float t = 1.0f - 2.0f / (1.0f + e);
    return 0.5f * z * (1.0f + t);
}

template <int DT, bool BKN, class C>
struct Tile {
    using E = Elem<DT>;

    int lane, wave, wn, wm, hf, l32;
    int m0, n0, rows_a, rows_b;
    unsigned lds0;
    unsigned loff_a, loff_b;     // per-lane direct-load offsets of round 0 within a panel
    unsigned rstep_a, rstep_b;   // bytes between consecutive load rounds (uniform)
    int kc;                      // logical 16-byte chunk of k this lane loads (K-contiguous tiles)
    unsigned ra, rb;             // per-lane LDS offsets of the operand reads (row and chunk of k-step 0)
    unsigned cx;                 // per-lane swizzle term of the chunk index
    f32x16_t acc[C::NB][C::MB];

    __device__ __forceinline__ void init(const GemmArgs& g, unsigned lds_base, int tile_m, int tile_n) {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: keeps LDS bases scalar
        wn = wave % C::WAVES_N;
        wm = wave / C::WAVES_N;
        hf = lane >> 5;
        l32 = lane & 31;
        lds0 = lds_base;
        m0 = tile_m * C::BM;
        n0 = tile_n * C::BN;
        rows_a = min(C::BM, g.M - m0);
        rows_b = min(C::BN, g.N - n0);
        // K-contiguous tiles: load round it, thread tid fills slot it*NT + tid =
        // (row it*NT/CPRK + tid/CPRK, physical chunk tid%CPRK), i.e. logical chunk
        // (tid%CPRK) ^ swz(row) = (tid%CPRK) ^ ((tid/16)%CPRK), the same in every round
        kc = (tid % C::CPRK) ^ ((tid >> 4) % C::CPRK);
        loff_a = (unsigned)((tid / C::CPRK) * g.lda) + (unsigned)(kc * 16);
        rstep_a = (unsigned)((C::NT / C::CPRK) * g.lda);
        if constexpr (BKN) {
            // B stored K x N: row k of the tile is 512 bytes = 8 granules of 64
            // bytes; round it, thread tid fills slot it*NT + tid = (row it*NT/32 +
            // tid/32, physical 16-byte chunk tid%32), i.e. granule (tid%32)/4 ^
            // (row % 8) = (tid%32)/4 ^ ((tid/32)%8) and chunk tid%4 within it
            const int gran = ((tid & 31) >> 2) ^ ((tid >> 5) & 7);
            loff_b = (unsigned)((tid >> 5) * g.ldb) + (unsigned)(gran * 64 + (tid & 3) * 16);
            rstep_b = (unsigned)((C::NT / 32) * g.ldb);
        } else {
            loff_b = (unsigned)((tid / C::CPRK) * g.ldb) + (unsigned)(kc * 16);
            rstep_b = (unsigned)((C::NT / C::CPRK) * g.ldb);
        }
        cx = (unsigned)((l32 / C::RPL) % C::CPRK);
        ra = (unsigned)(C::AOFF + (wm * C::WM + l32) * C::ROWB);
        rb = (unsigned)(C::BOFF + (wn * C::WN + l32) * C::ROWB);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) acc[nb][mb] = f32x16_t{};
    }

    // tile j of A and B into the LDS stage at byte offset `stage`
    __device__ __forceinline__ void issue(const GemmArgs& g, int j, unsigned stage) const {
        const int k0 = j * C::BK;
        const int krem = g.K - k0;                      // > 0
        const unsigned region = lds0 + stage;
        {
            const unsigned char* base = g.a + (size_t)m0 * (size_t)g.lda + (size_t)k0 * 2;
            const int bytes = (int)((rows_a - 1) * g.lda + (long long)krem * 2);
            const eta_desc_t desc = buffer_desc(base, bytes);
            const unsigned vo = kc * 8 < krem ? loff_a : 0x80000000u;   // chunks past K read as zero
#pragma unroll
            for (int it = 0; it < C::ROUNDS; ++it) {
                load_lds16(desc, vo, (unsigned)(it * rstep_a), region + C::AOFF + (unsigned)((it * C::NT + wave * 64) * 16));
            }
        }
        if constexpr (BKN) {
            // rows k0 .. K-1 of B, columns n0 .. N-1: rows past K read as zero
            // through the range check, columns past N only feed unstored outputs.
            // The range ends on a whole 16-byte chunk, so a chunk that straddles
            // column N is read whole (it lies in one aligned 16-byte block of the
            // last row, so no byte outside a mapped page is touched)
            const unsigned char* base = g.b + (size_t)k0 * (size_t)g.ldb + (size_t)n0 * 2;
            const int kr = min(krem, C::BK);
            const int bytes = (int)((kr - 1) * g.ldb + (((long long)rows_b * 2 + 15) & ~15LL));
            const eta_desc_t desc = buffer_desc(base, bytes);
#pragma unroll
            for (int it = 0; it < C::ROUNDS; ++it) {
                load_lds16(desc, loff_b, (unsigned)(it * rstep_b), region + C::BOFF + (unsigned)((it * C::NT + wave * 64) * 16));
            }
        } else {
            const unsigned char* base = g.b + (size_t)n0 * (size_t)g.ldb + (size_t)k0 * 2;
            const int bytes = (int)((rows_b - 1) * g.ldb + (long long)krem * 2);
            const eta_desc_t desc = buffer_desc(base, bytes);
            const unsigned vo = kc * 8 < krem ? loff_b : 0x80000000u;
#pragma unroll
            for (int it = 0; it < C::ROUNDS; ++it) {
                load_lds16(desc, vo, (unsigned)(it * rstep_b), region + C::BOFF + (unsigned)((it * C::NT + wave * 64) * 16));
            }
        }
    }

    // load rounds r0 .. r1-1 of tile j (rounds 0 .. ROUNDS-1 of A, then those of B)
    __device__ __forceinline__ void issue_rounds(const GemmArgs& g, int j, unsigned stage, int r0, int r1) const {
        const int k0 = j * C::BK;
        const int krem = g.K - k0;
        const unsigned region = lds0 + stage;
        if (r0 < C::ROUNDS) {
            const unsigned char* base = g.a + (size_t)m0 * (size_t)g.lda + (size_t)k0 * 2;
            const eta_desc_t desc = buffer_desc(base, (int)((rows_a - 1) * g.lda + (long long)krem * 2));
            const unsigned vo = kc * 8 < krem ? loff_a : 0x80000000u;
#pragma unroll
            for (int it = 0; it < C::ROUNDS; ++it)
                if (it >= r0 && it < r1)
                    load_lds16(desc, vo, (unsigned)(it * rstep_a), region + C::AOFF + (unsigned)((it * C::NT + wave * 64) * 16));
        }
        if (r1 > C::ROUNDS) {
            if constexpr (BKN) {
                const unsigned char* base = g.b + (size_t)k0 * (size_t)g.ldb + (size_t)n0 * 2;
                const int kr = min(krem, C::BK);
                const eta_desc_t desc = buffer_desc(base, (int)((kr - 1) * g.ldb + (((long long)rows_b * 2 + 15) & ~15LL)));
#pragma unroll
                for (int it = 0; it < C::ROUNDS; ++it)
                    if (it + C::ROUNDS >= r0 && it + C::ROUNDS < r1)
                        load_lds16(desc, loff_b, (unsigned)(it * rstep_b), region + C::BOFF + (unsigned)((it * C::NT + wave * 64) * 16));
            } else {
                const unsigned char* base = g.b + (size_t)n0 * (size_t)g.ldb + (size_t)k0 * 2;
                const eta_desc_t desc = buffer_desc(base, (int)((rows_b - 1) * g.ldb + (long long)krem * 2));
                const unsigned vo = kc * 8 < krem ? loff_b : 0x80000000u;
#pragma unroll
                for (int it = 0; it < C::ROUNDS; ++it)
                    if (it + C::ROUNDS >= r0 && it + C::ROUNDS < r1)
                        load_lds16(desc, vo, (unsigned)(it * rstep_b), region + C::BOFF + (unsigned)((it * C::NT + wave * 64) * 16));
            }
        }
    }

    // operands of k-step s from the stage at `base` (= lds0 + stage offset):
    // av[nb] is the MFMA A operand (B^T block nb: 32 n x 16 k), bv[mb] the B
    // operand (A^T block mb: 16 k x 32 m)
    __device__ __forceinline__ void operands(unsigned base, int s, u32x4_t (&av)[C::NB], u32x4_t (&bv)[C::MB]) const {
        const unsigned ch = (unsigned)(((2 * s + hf) ^ cx) * 16);
        if constexpr (BKN) {
            // k-rows 16 s + 8 hf .. +7 of column n: two transpose reads of 4
            // k-rows each (lane j of a 16-lane group addresses k-row 16 s + 8 hf
            // + 4 h + j/4 at columns n .. n+3, n = block + 16 (group % 2) + 4 (j % 4));
            // the 64-byte granule of row r is swizzled by r % 8
            const int g16 = lane >> 4, s16 = lane & 15;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                u32x4_t v;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 16 * s + 8 * (g16 >> 1) + 4 * h + (s16 >> 2);
                    const int n = wn * C::WN + nb * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);
                    const int gran = (n >> 5) ^ (r & 7);
                    const u32x2_t t = lds_read_tr(base + C::BOFF + (unsigned)(r * (C::BN * 2) + gran * 64 + (n & 31) * 2));
                    v[2 * h] = t[0];
                    v[2 * h + 1] = t[1];
                }
                av[nb] = v;
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) av[nb] = lds_read16(base + rb + ch + nb * 32 * C::ROWB);
        }
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) bv[mb] = lds_read16(base + ra + ch + mb * 32 * C::ROWB);
    }

    // every operand of the tile in the stage at byte offset `stage`, all KS k-steps;
    // with j >= 0, tile j's load rounds are issued in between (LOADS / KS per k-step)
    __device__ __forceinline__ void load_step(const GemmArgs& g, unsigned stage, u32x4_t (&av)[C::KS][C::NB],
                                              u32x4_t (&bv)[C::KS][C::MB], int j, unsigned jstage) const {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            if (j >= 0) issue_rounds(g, j, jstage, s * C::LOADS / C::KS, (s + 1) * C::LOADS / C::KS);
            operands(lds0 + stage, s, av[s], bv[s]);
        }
    }

    // the tile's MFMAs from operands already in registers; with j >= 0, tile j's
    // load rounds are issued in between (LOADS / KS per k-step)
    __device__ __forceinline__ void mma_step(const GemmArgs& g, const u32x4_t (&av)[C::KS][C::NB],
                                             const u32x4_t (&bv)[C::KS][C::MB], int j, unsigned jstage) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) acc[nb][mb] = E::mfma(av[s][nb], bv[s][mb], acc[nb][mb]);
            if (j >= 0) issue_rounds(g, j, jstage, s * C::LOADS / C::KS, (s + 1) * C::LOADS / C::KS);
        }
    }

    // bias, activation, rounding and the store of this wave's 128 x 128 block
    // bias + activation of one accumulator quad: C[m][n .. n+3] for this lane
    __device__ __forceinline__ void epilogue_values(const GemmArgs& g, int nb, int gq, int mb, const float (&bias)[4],
                                                    float (&v)[4]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float z = acc[nb][mb][4 * gq + j] + bias[j];
            if (g.act == GEMM_ACT_RELU) z = fmaxf(z, 0.f);
            else if (g.act == GEMM_ACT_GELU_TANH) z = gelu_tanh(z);
            v[j] = z;
        }
    }

    __device__ __forceinline__ void load_bias(const GemmArgs& g, int n, float (&bias)[4]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) bias[j] = 0.f;
        if (g.bias) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n + j < g.N) bias[j] = E::get(g.bias + (size_t)(n + j) * 2);
        }
    }

    // Bias, activation, rounding and the stores of C.  With 16-byte aligned C
    // the wave's WM x WN block first goes to its own slice of the (then unused)
    // LDS stages, 256-byte rows with the 16-byte chunk c of row r at c ^ (r % 16),
    // and is stored as whole row segments: each store instruction writes 256
    // contiguous bytes of four rows instead of 16 bytes of 32 rows.
    __device__ __forceinline__ void finish(const GemmArgs& g) const {
        if (!g.c_vec16) {
            finish_direct(g);
            return;
        }
        __syncthreads();                                  // every wave has read its last operands
        const unsigned slice = lds0 + (unsigned)(wave * C::WM * C::WN * 2);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int n = n0 + wn * C::WN + nb * 32 + 8 * gq + 4 * hf;
                float bias[4];
                load_bias(g, n, bias);
                const int c = nb * 4 + gq;                // 16-byte chunk of the slice row
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) {
                    float v[4];
                    epilogue_values(g, nb, gq, mb, bias, v);
                    const int r = mb * 32 + l32;
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                        (lds_bytes)(size_t)(slice + r * 256 + ((c ^ (r % 16)) * 16) + 8 * hf)) =
                        u32x2_t{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
                }
            }
        const int c = lane % 16, rq = lane / 16;
        const int n = n0 + wn * C::WN + 8 * c;
#pragma unroll
        for (int k = 0; k < C::WM / 4; ++k) {
            const int r = 4 * k + rq;
            const int m = m0 + wm * C::WM + r;
            const u32x4_t v = lds_read16(slice + r * 256 + ((c ^ (r % 16)) * 16));
            if (m >= g.M || n >= g.N) continue;
            unsigned char* dst = g.c + (size_t)m * (size_t)g.ldc + (size_t)n * 2;
            if (n + 7 < g.N) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (n + j < g.N) reinterpret_cast<uint16_t*>(dst)[j] = (uint16_t)(v[j / 2] >> (16 * (j % 2)));
            }
        }
    }

    // the same values stored straight from the accumulator layout (any C alignment)
    __device__ __forceinline__ void finish_direct(const GemmArgs& g) const {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                // accumulator registers 4 gq .. 4 gq + 3 of a lane hold rows
                // n = nb*32 + 8 gq + 4 hf + (0..3) of C^T, i.e. columns of C
                const int n = n0 + wn * C::WN + nb * 32 + 8 * gq + 4 * hf;
                float bias[4];
                load_bias(g, n, bias);
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) {
                    const int m = m0 + wm * C::WM + mb * 32 + l32;
                    if (m >= g.M || n >= g.N) continue;
                    float v[4];
                    epilogue_values(g, nb, gq, mb, bias, v);
                    unsigned char* dst = g.c + (size_t)m * (size_t)g.ldc + (size_t)n * 2;
                    if (g.c_vec && n + 3 < g.N) {
                        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (n + j < g.N) E::put(dst + 2 * j, v[j]);
                    }
                }
            }
        }
    }
};

#endif  // __HIP_DEVICE_COMPILE__


// Two wave groups in alternation (8 waves, 2 LDS stages): waves 0-3 and 4-7,
// one of each on every SIMD, run the same sequence per k tile i,
//     M(i)  barrier  X(i)  barrier
// with M(i) = every operand of tile i read from LDS into registers and X(i) =
// tile i's MFMAs from those registers.  Group 1 passes one extra barrier
// before its first M and group 0 one after its last X, so between two
// barriers one wave of a SIMD issues MFMAs while the other reads LDS:
//     slot 2i:   group 0 M(i),  group 1 X(i-1)
//     slot 2i+1: group 0 X(i),  group 1 M(i)
// Tile i+1 is issued at the start of slot 2i (group 0 at the start of M(i),
// group 1 at the start of X(i-1); its stage last held tile i-1, read in slots
// 2i-2 and 2i-1) and waited for at the end of slot 2i+1, before its first read
// in slot 2i+2.
template <int DT, bool BKN, int WAVES, int WAVES_N, int BK, int STAGES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void gemm_kernel_pp(GemmArgs g) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Cfg<WAVES, WAVES_N, BK, STAGES>;
    static_assert(WAVES == 8 && STAGES == 2, "two groups of four waves, two stages");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS];
    Tile<DT, BKN, C> t;
    int tile_m, tile_n;
    map_tile(g, tile_m, tile_n);
    t.init(g, (unsigned)(size_t)(lds_bytes)lds, tile_m, tile_n);
    const int nk = (g.K + C::BK - 1) / C::BK;
    const bool g0 = t.wave < 4;                      // wave-uniform
    u32x4_t av[C::KS][C::NB], bv[C::KS][C::MB];
    // tile 0 from everyone; group 1's share of tile 1 too (group 0 issues its
    // share at the start of its first M)
    if (nk > 0) t.issue(g, 0, 0);
    if (!g0 && nk > 1) {
        t.issue(g, 1, C::STAGE);
        wait_vmcnt<C::LOADS>();
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();
    if (!g0) __syncthreads();
    for (int i = 0; i < nk; ++i) {
        const unsigned st = (unsigned)(i & 1) * C::STAGE;
        const int j0 = g0 && i + 1 < nk ? i + 1 : -1;   // group 0: tile i+1 during M(i)
        const int j1 = !g0 && i + 2 < nk ? i + 2 : -1;  // group 1: tile i+2 during X(i)
        t.load_step(g, st, av, bv, j0, C::STAGE - st);
        if (!g0) wait_vmcnt<0>();                    // slot 2i+1 ends (group 1): tile i+1 landed
        __syncthreads();
        __builtin_amdgcn_s_setprio(2);
        t.mma_step(g, av, bv, j1, st);
        __builtin_amdgcn_s_setprio(0);
        if (g0) wait_vmcnt<0>();                     // slot 2i+1 ends (group 0): tile i+1 landed
        __syncthreads();
    }
    if (g0) __syncthreads();
    t.finish(g);
#endif
}

// --- host side ---------------------------------------------------------------

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

// The launched configuration: 8 waves (two groups of four, see gemm_kernel_pp),
// two of them along n, k steps of 64 through two LDS stages.
using Launch = Cfg<8, 2, 64, 2>;

hipError_t launch(const GemmArgs& g, int dtype, bool bkn, hipStream_t s) {
    const dim3 grid((unsigned)(g.tm * g.tn)), block(Launch::NT);
    if (dtype == ATTN_BF16)
        return bkn ? launch_kernel(gemm_kernel_pp<ATTN_BF16, true, 8, 2, 64, 2>, grid, block, s, g)
                   : launch_kernel(gemm_kernel_pp<ATTN_BF16, false, 8, 2, 64, 2>, grid, block, s, g);
    return bkn ? launch_kernel(gemm_kernel_pp<ATTN_F16, true, 8, 2, 64, 2>, grid, block, s, g)
               : launch_kernel(gemm_kernel_pp<ATTN_F16, false, 8, 2, 64, 2>, grid, block, s, g);
}

}  // namespace

extern "C" int gemm_bias_act(const void* a, long long lda, const void* b, long long ldb, int b_layout, const void* bias,
                             void* c, long long ldc, int M, int N, int K, int act, int dtype, void* stream) {
    if (!c || (K > 0 && (!a || !b))) return ATTN_ERR_NULL;
    if (M < 1 || N < 1 || K < 0 || K % 8 != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (b_layout != GEMM_B_KN && b_layout != GEMM_B_NK) return ATTN_ERR_LAYOUT;
    if (act != GEMM_ACT_NONE && act != GEMM_ACT_RELU && act != GEMM_ACT_GELU_TANH) return ATTN_ERR_LAYOUT;
    const bool bkn = b_layout == GEMM_B_KN;
    if (ldc < N) return ATTN_ERR_SHAPE;
    if (K > 0) {
        if (lda < K || ldb < (bkn ? N : K)) return ATTN_ERR_SHAPE;
        // 32-bit buffer offsets: one panel of A (and of B) must span < 2^31 bytes
        constexpr long long kSpan = 1LL << 31;
        if (lda > kSpan / (2 * Shape::BM) || ldb > kSpan / (2 * (bkn ? Shape::BK : Shape::BN))) return ATTN_ERR_SHAPE;
        if (((uintptr_t)a | (uintptr_t)b) % 16 || lda % 8 || ldb % 8) return ATTN_ERR_ALIGN;
    }
    if (ldc > (1LL << 40)) return ATTN_ERR_SHAPE;
    if (((uintptr_t)c | (uintptr_t)bias) % 2) return ATTN_ERR_ALIGN;
    // c's span must not meet an input's span
    const uintptr_t c0 = (uintptr_t)c, c1 = c0 + (uintptr_t)(((long long)M - 1) * ldc + N) * 2;
    if (K > 0) {
        const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)(((long long)M - 1) * lda + K) * 2;
        const long long brows = bkn ? K : N, bcols = bkn ? N : K;
        const uintptr_t b0 = (uintptr_t)b, b1 = b0 + (uintptr_t)((brows - 1) * ldb + bcols) * 2;
        if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return ATTN_ERR_ALIAS;
    }
    if (bias && overlaps(c0, c1, (uintptr_t)bias, (uintptr_t)bias + (uintptr_t)N * 2)) return ATTN_ERR_ALIAS;
    const long long tm = ((long long)M + Shape::BM - 1) / Shape::BM, tn = ((long long)N + Shape::BN - 1) / Shape::BN;
    if (tm * tn > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    const int dev_status = check_device();
    if (dev_status != ATTN_OK) return dev_status;

    GemmArgs g;
    g.a = static_cast<const unsigned char*>(a);
    g.b = static_cast<const unsigned char*>(b);
    g.bias = static_cast<const unsigned char*>(bias);
    g.c = static_cast<unsigned char*>(c);
    g.lda = lda * 2;
    g.ldb = ldb * 2;
    g.ldc = ldc * 2;
    g.M = M;
    g.N = N;
    g.K = K;
    g.act = act;
    g.tm = (int)tm;
    g.tn = (int)tn;
    g.c_vec = ((uintptr_t)c % 8 == 0) && (ldc % 4 == 0);
    g.c_vec16 = ((uintptr_t)c % 16 == 0) && (ldc % 8 == 0);
    return launch(g, dtype, bkn, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
