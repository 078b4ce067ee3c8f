// attn_fwd.hip -- fused exact-attention forward for gfx950 (MI355X) and its C ABI.
//
// Method: "Triton in depth: from matmul to Flash Attention" (ybb.press),
// sections 3.2-3.3.  A work-group owns query tiles of one (batch, head) and
// walks the key/value tiles once, keeping for every query row the running max
// m and running sum l of the exponentials; the fp32 output accumulator is
// rescaled by exp(m_old - m_new) when the max grows and divided by l once after
// the loop.  Keys with index > query index are excluded when causal.  The
// N x N score matrix never leaves registers.  The sliding-window variant (a
// variant "Triton: CUDA-level operators in Python" names without defining; read
// as the local band i - W < j, and j < i + W when not causal) only narrows the
// range of key tiles a query tile visits and adds a lower mask limit on the
// tiles that straddle the band's edge; it is a compile-time kernel parameter.
//
// gfx950 mapping (not taken from the pages, which target NVIDIA tensor cores):
//
//  * Scores are produced transposed, S^T = K Q^T, with v_mfma_f32_32x32x16.
//    In the 32x32 accumulator layout a lane owns one column, so each lane
//    holds 16 scores of ONE query.  The row max is 15 lane-local max ops plus
//    one exchange with lane^32 (the other half of the same column); the row
//    sum needs no exchange until the epilogue.
//  * The K rows fed to the A operand are permuted (kperm) so that the 16
//    accumulator registers of a lane map to two runs of 8 consecutive keys.
//    Those runs are exactly the B operand layout of O^T += V^T P^T, so P goes
//    from the score accumulator to the P.V operand without leaving the lane.
//  * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//    destination, issued from inline assembly), rows XOR-swizzled for
//    conflict-free reads: two stages for 4-wave work-groups, a three-stage
//    ring for 8-wave ones.  V stays row-major; its P.V operand is read with
//    the gfx950 transpose load.
//  * Work-groups are remapped so that each XCD (ids are dealt round-robin over
//    the 8 XCDs) gets a contiguous run of heads, keeping a head's K/V in one
//    L2.  A causal work-group takes the query-tile pair (i, nqt-1-i), so all
//    work-groups do the same amount of work.
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA; lse is
//    returned in natural-log units.
//
// Small problems use 4-wave work-groups (128 queries) whose waves run free:
// two work-groups share a CU, so on each SIMD one wave's exponentials overlap
// the other's MFMAs, and the grid still fills the 256 CUs.  Large problems use
// 8-wave work-groups (256 queries, halving the K/V loads per query), resident
// one per CU, whose two groups of four waves alternate between the softmax
// half and the matrix half of a key tile (see the kernel).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "attn.h"
#include "attn_bwd.h"
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
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// log2 headroom before the reference max is raised (see Wave::prepare)
constexpr float kRescaleTh = 8.0f;

// --- element type ------------------------------------------------------------
template <int DT> struct Elem;

template <> struct Elem<ATTN_F16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                     __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    // l may be the sum of the probabilities as rounded to this type: its
    // relative rounding (2^-11) keeps lse within the tolerance (see Wave)
    static constexpr bool kRoundedSum = true;
    static constexpr unsigned kOne = 0x3c00u;
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
    static constexpr bool kRoundedSum = false;   // 2^-8 would show in lse
    static constexpr unsigned kOne = 0x3f80u;
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
    int ngroups;       // work-groups per head: causal without a window pairs tiles (i, nqt-1-i), else nqt
    float c;           // |scale| * log2(e), > 0
    unsigned qsign;    // 0x80008000 when scale < 0 (Q negated exactly), else 0
    int window;        // 0: none; W in [1, N): key j kept for query i only if i - W < j (and j < i + W if not causal)
    // Key-range parts (the PARTS kernel only): work units 0 .. nwhole-1 are whole
    // query tiles; the other nleft tiles (the last ones in (head, tile) order,
    // whose rows row0 .. row0+rows-1 of the [BH*N] row space are contiguous)
    // are each cut into nparts key ranges, part p of them written to
    // o_parts[p][row - row0][:] (normalised by its own sum) and lse_parts[p][row - row0].
    int nwhole;        // whole work units (ngroups * BH without parts)
    int nleft;
    int nparts;
    long long row0;
    long long rows;
    uint16_t* o_parts;
    float* lse_parts;
    int unpaired;      // causal 4-wave grid: one query tile per unit, longest first (see the kernel), instead of pairs
};

// x combined with the value in the lane 32 positions away (the other half of
// the same accumulator column), through v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of the K tile that feeds A-operand row m of the score MFMA.  With this
// permutation, accumulator register i of a lane in half h holds key
// 16*(i/8) + 8*h + (i%8) of the 32-key block.
__device__ __forceinline__ int kperm(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Tile configuration shared by the kernels and the host launcher.
//
// LDS holds STAGES stages of K and V, each a BN x ROWB byte array written by
// direct global->LDS loads: one load instruction of a wave fills 1 KB of
// consecutive 16-byte slots, so rows are unpadded (ROWB = CPRP * 16 with CPRP
// the chunk count rounded up to a power of two) and bank conflicts are avoided
// by XOR-swizzling the 16-byte chunk index with a function of the row:
//  * K is read by the score MFMA as 16-byte chunks of 16 different rows at the
//    same logical chunk: chunk c of row r sits at c ^ kswz(r), kswz(r) =
//    (r / RPB) % CPRP with RPB rows per 256-byte bank line.
//  * V is read by 8-byte transpose loads, 4 consecutive rows x one 64-byte
//    granule per 32 lanes: the granule index g of row r sits at g ^ vswz(r),
//    vswz(r) = (r / RPB) % GPR with GPR granules per row.  It only moves whole
//    granules, so rows 4 apart differ by a fixed offset for every lane.
template <int D, int WAVES_, int STAGES_ = 2, int SUBS_ = 1> struct Cfg {
    static constexpr int WAVES = WAVES_;
    static constexpr int STAGES = STAGES_;            // K/V tile stages in LDS
    static constexpr int SUBS = SUBS_;                // tiles per stage (2: the key-split schedule)
    static constexpr int NT = 64 * WAVES;             // threads per work-group
    static constexpr int BM = 32 * WAVES;             // queries per work-group (32 per wave)
    static constexpr int BN = 64;                     // keys per tile
    static constexpr int SB = BN / 32;                // 32-key score blocks per tile
    static constexpr int KK = BN / 16;                // 16-key P.V k-steps per tile
    static constexpr int KSTEPS = D / 16;             // MFMA k-steps over the head dim
    static constexpr int DBLK = (D + 31) / 32;        // 32-row blocks of O^T
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row in HBM
    static constexpr int CPRP = CPR <= 8 ? 8 : 16;    // chunks per row in LDS
    static constexpr int ROWB = CPRP * 16;            // bytes per row in LDS
    static constexpr int RPB = 256 / ROWB;            // rows per 256-byte bank line
    static constexpr int GPR = CPRP / 4;              // 64-byte granules per row
    static constexpr int TILEB = BN * ROWB;           // bytes of one K or V tile
    static constexpr int SSTR = SUBS * TILEB;         // bytes of one K (or V) stage
    static constexpr int KOFF = 0;                    // K stage s at KOFF + s * SSTR (+ sub * TILEB)
    static constexpr int VOFF = STAGES * SSTR;        // V stage s at VOFF + s * SSTR (+ sub * TILEB)
    static constexpr int LDS = 2 * STAGES * SSTR;
    static constexpr int IT = TILEB / (16 * NT);      // direct-load instructions per tile and thread
    static __device__ __forceinline__ int kswz(int r) { return (r / RPB) % CPRP; }
    static __device__ __forceinline__ int vswz(int r) { return (r / RPB) % GPR; }
    static_assert(D % 16 == 0 && CPR <= CPRP, "head dim");
    static_assert(IT >= 1 && TILEB % (16 * NT) == 0, "a tile is a whole number of load rounds");
    static_assert(DBLK <= GPR, "transpose reads of the padded head dim stay inside a row");
    static_assert(STAGES == 3 || VOFF + 2 * SSTR <= 65536, "LDS offsets fit the 16-bit immediate");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(WAVES * 32 * ROWB <= LDS, "the epilogue's per-wave O slices fit in the stages");
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

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

#if defined(__HIP_DEVICE_COMPILE__)

// Work-group id -> (head, group): ids are dealt round-robin over the 8 XCDs,
// so XCD x runs ids x, x+8, ...; the remap gives each XCD a contiguous range
// of (head, group) indices.
__device__ __forceinline__ void map_workgroup(const FwdArgs& a, int L, int T, int& bh, int& grp) {
    const int xcd = L & 7;
    const int vidx = xcd * (T >> 3) + min(xcd, T & 7) + (L >> 3);
    bh = vidx / a.ngroups;
    grp = vidx - bh * a.ngroups;
}

// State and arithmetic of one wave: 32 query rows (one per accumulator column;
// the two lanes of a column each hold half of the keys of a tile).
template <int D, int DT, bool CAUSAL, int WAVES, bool WIN, int STAGES = 2, int SUBS = 1>
struct Wave {
    using C = Cfg<D, WAVES, STAGES, SUBS>;
    using E = Elem<DT>;
    static constexpr int SB = C::SB, KK = C::KK, KSTEPS = C::KSTEPS, DBLK = C::DBLK, CPR = C::CPR;
    // ONES: the head dim leaves padding in the last 32-row block of O^T (d = 80:
    // rows 80..95).  Column D of every V row in LDS is set to 1, so O^T row D
    // accumulates the row sum l of the rounded probabilities with the P.V
    // MFMAs that run anyway, rescaled with O, instead of one add per score.
    // Used where it measured faster: the unmasked 8-wave schedule (+2-3% at
    // d = 80 fp16; -0.9% causal and -4.6% with 4 waves, whose extra LDS writes
    // and registers cost more than the adds).
    static constexpr bool ONES = D % 32 != 0 && E::kRoundedSum && WAVES == 8 && !CAUSAL;
    static constexpr int LDB = D / 32, LREG = 4 * ((D % 32) / 8);   // O^T row D: o[LDB][LREG] of the lanes with hf = 0

    int lane, wave, hf, n, N, qw0, qi, W;
    unsigned onesm;                    // bit it: this lane's slot of load round it holds V column D
    float c;
    unsigned lds0;
    const unsigned char* kbase;
    const unsigned char* vbase;
    unsigned kvo[C::IT], vvo[C::IT];   // per-lane offsets of the direct loads
    unsigned ka[KSTEPS];               // per-lane LDS addresses of the score A operand
    unsigned va[DBLK];                 // per-lane LDS addresses of the P.V A operand
    u32x4_t qf[KSTEPS];                // Q^T fragments (score B operand)
    f32x16_t o[DBLK];                  // O^T accumulator
    float m, l;                        // reference max (log2 units) and this half's sum (not kept with ONES)

    // sub: the tile of each stage this wave reads (the key-split schedule's second
    // pair of waves reads the second tile)
    __device__ __forceinline__ void init(const FwdArgs& a, unsigned lds_base, int tid, int wave_, int sub = 0) {
        lane = tid & 63;
        wave = wave_;
        hf = lane >> 5;
        n = lane & 31;
        N = a.N;
        W = WIN ? a.window : 0;          // a compile-time 0 without a window: its tests fold away
        c = a.c;
        lds0 = lds_base;
        // direct-load slot (it, wave, lane) of a tile holds row r = slot / CPRP,
        // physical chunk p = slot % CPRP, i.e. logical chunk p ^ swizzle(r); chunks
        // past the head dim get an out-of-range offset and read as zero, as do rows
        // past N (the buffer ends at row N)
#pragma unroll
        for (int it = 0; it < C::IT; ++it) {
            const int slot = slot_base(it) + lane;
            const int r = slot / C::CPRP, p = slot % C::CPRP;
            const int kc = p ^ C::kswz(r);
            const int vc = p ^ (4 * C::vswz(r));
            kvo[it] = kc < CPR ? (unsigned)(r * D * 2 + kc * 16) : 0x80000000u;
            vvo[it] = vc < CPR ? (unsigned)(r * D * 2 + vc * 16) : 0x80000000u;
        }
        onesm = 0;
#pragma unroll
        for (int it = 0; it < C::IT; ++it) {
            const int slot = slot_base(it) + lane;
            if (((slot % C::CPRP) ^ (4 * C::vswz(slot / C::CPRP))) == CPR) onesm |= 1u << it;
        }
        {
            const int r = kperm(n);
            const int x = C::kswz(r);                              // rows r and r + 32 share it
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                ka[ks] = lds0 + C::KOFF + sub * C::TILEB + r * C::ROWB + (((2 * ks + hf) ^ x) * 16);
        }
        {
            const int g16 = lane >> 4, s16 = lane & 15;
            const int r = 8 * (g16 >> 1) + (s16 >> 2);           // + 16*kk + 4*half: multiples of 4 rows
            const int x = C::vswz(r);                             // the same for r + 16*kk + 4*half
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                va[db] = lds0 + C::VOFF + sub * C::TILEB + r * C::ROWB + (4 * (db ^ x) + 2 * (g16 & 1) + ((s16 & 3) >> 1)) * 16 +
                         8 * (s16 & 1);
        }
    }

    // start a query tile: this wave's rows begin at qw0_ (the Q fragments come
    // later, from q_issue / q_read)
    __device__ __forceinline__ void begin(const FwdArgs& a, int bh, int qw0_) {
        qw0 = qw0_;
        qi = qw0 + n;
        const size_t hoff = (size_t)bh * (size_t)N * CPR;   // head offset in 16-byte chunks
        kbase = reinterpret_cast<const unsigned char*>(a.k + hoff);
        vbase = reinterpret_cast<const unsigned char*>(a.v + hoff);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
        m = kNegInf;
        l = 0.f;
    }

    // this wave's share of tile j of K (is_v false) or V into LDS stage `stage`
    // (its tile `sub` in the key-split schedule)
    __device__ __forceinline__ void issue(bool is_v, int j, int stage, int sub = 0) const {
        const int kt0 = j * C::BN;
        const int bytes = (N - kt0) * D * 2;            // rows kt0 .. N-1 are in range
        const unsigned char* base = (is_v ? vbase : kbase) + (size_t)kt0 * D * 2;
        const eta_desc_t desc = buffer_desc(base, bytes);
        const unsigned region = lds0 + (is_v ? C::VOFF : C::KOFF) + stage * C::SSTR + sub * C::TILEB;
#pragma unroll
        for (int it = 0; it < C::IT; ++it)
            load_lds16(desc, is_v ? vvo[it] : kvo[it], 0, region + (unsigned)(slot_base(it) * 16));
    }

    // ONES: V column D = 1 (and D+1 .. D+7 = 0) in the rows this wave's loads of
    // stage ST just filled; the loads write zeros there (the chunk is past the
    // head dim), so this runs after they have landed, before the barrier that
    // publishes the tile.
    template <int ST>
    __device__ __forceinline__ void ones() const {
        if constexpr (ONES) {
            const unsigned region = lds0 + C::VOFF + ST * C::SSTR;
#pragma unroll
            for (int it = 0; it < C::IT; ++it)
                if (onesm & (1u << it))
                    *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(
                        (lds_bytes)(size_t)(region + (unsigned)((slot_base(it) + lane) * 16))) = u32x4_t{E::kOne, 0u, 0u, 0u};
        }
    }

    // This wave's 32 Q rows (qw0 ..) into its LDS slice by direct loads: 32 rows of
    // ROWB bytes, logical 16-byte chunk c of row r at physical c ^ (r % CPRP); rows
    // at or past N and chunks past the head dim read as zero.  Each load
    // instruction moves 1 KB of consecutive rows (a register load of the
    // fragments touches 32 rows per instruction).
    __device__ __forceinline__ void q_issue(const FwdArgs& a, int bh, unsigned slice) const {
        const unsigned char* base = reinterpret_cast<const unsigned char*>(a.q + ((size_t)bh * N + qw0) * CPR);
        const eta_desc_t desc = buffer_desc(base, max(0, (N - qw0) * D * 2));
#pragma unroll
        for (int it = 0; it < 32 * C::CPRP / 64; ++it) {
            const int slot = it * 64 + lane, r = slot / C::CPRP, c = (slot % C::CPRP) ^ (r % C::CPRP);
            load_lds16(desc, c < CPR ? (unsigned)(r * D * 2 + c * 16) : 0x80000000u, 0, slice + (unsigned)(it * 1024));
        }
    }

    // the Q^T fragments (score B operands) from the slice, once q_issue's loads have landed
    __device__ __forceinline__ void q_read(const FwdArgs& a, unsigned slice) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qf[ks] = lds_read16(slice + n * C::ROWB + (((2 * ks + hf) ^ (n % C::CPRP)) * 16));
        if (a.qsign) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] ^= a.qsign;
        }
    }

    // first slot of load round `it` for this wave
    __device__ __forceinline__ int slot_base(int it) const { return (it * C::WAVES + wave) * 64; }

    // does this wave have keys to process in tile j?
    // (the rows qw0 .. qw0+31 keep keys up to qw0+31 when causal, and within the
    // window band [qi-W+1, qi+W-1] otherwise)
    __device__ __forceinline__ bool active(int j) const {
        if (qw0 >= N) return false;
        const int klo = j * C::BN, khi = klo + C::BN - 1;
        if (CAUSAL && klo > qw0 + 31) return false;
        if (W > 0 && (khi < qw0 - W + 1 || (!CAUSAL && klo > qw0 + 31 + W - 1))) return false;
        return true;
    }

    // S^T = K Q^T for the tile in K stage ST: two independent 32-key accumulators
    template <int ST>
    __device__ __forceinline__ void score(f32x16_t (&s)[SB]) const {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) s[sb] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
                s[sb] = E::mfma(lds_read16(ka[ks] + ST * C::SSTR + sb * 32 * C::ROWB), qf[ks], s[sb]);
    }

    // Mask tile j's scores where needed and update the reference max.  m is
    // raised only when a tile's max exceeds it by more than kRescaleTh (log2
    // units), so p <= 2^TH and the O rescale is rare; m, l and O always refer to
    // the same m, so the result is unchanged.
    __device__ __forceinline__ void prepare(f32x16_t (&s)[SB], int j) {
        const int kt0 = j * C::BN;
        const bool window_edge = W > 0 && (kt0 < qw0 + 32 - W || (!CAUSAL && kt0 + C::BN - 1 > qw0 + W - 1));
        if ((CAUSAL && kt0 + C::BN - 1 > qw0) || kt0 + C::BN > N || window_edge) {
            // key index of register i is kt0 + 8*hf + 32*sb + 16*(i/8) + i%8; it is
            // kept iff lo <= that <= hi: hi is the query for causal (else the band's
            // upper end, else N-1), capped at N-1; lo is the band's lower end
            const int base = kt0 + 8 * hf;
            const int hi = (CAUSAL ? min(qi, N - 1) : (W > 0 ? min(qi + W - 1, N - 1) : N - 1)) - base;
            const int lo = (W > 0 ? qi - W + 1 : 0) - base;
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 32 * sb + 16 * (i >> 3) + (i & 7);
                    if (key > hi || (WIN && key < lo)) s[sb][i] = kNegInf;
                }
        }
        float mc[4] = {kNegInf, kNegInf, kNegInf, kNegInf};   // four independent chains
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mc[i & 3] = fmaxf(mc[i & 3], s[sb][i]);
        const float mx = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
        const float mt = pair_max(mx) * c;           // c > 0, so -inf stays -inf
        const bool grow = mt > m + kRescaleTh;
        if (__any(grow)) {
            const float mnew = grow ? mt : m;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;   // 0 when m was -inf
            m = mnew;
            if constexpr (!ONES) l *= alpha;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
        }
    }

    // P = exp2(c*s - m), rounded to the input type and packed as the B operands
    // of the P.V k-steps; the fp32 probabilities are added to l (with ONES the
    // P.V MFMAs sum the rounded ones instead)
    __device__ __forceinline__ void probs(const f32x16_t (&s)[SB], u32x4_t (&pf)[KK]) {
        const float nm = m > kNegInf ? -m : 0.f;
        float part[4];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            float p[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + i], c, nm));
                // the chains start at their first probability (p >= 0, so 0 + p = p exactly)
                if constexpr (!ONES) part[i & 3] = kk == 0 && i < 4 ? p[i] : part[i & 3] + p[i];
            }
            pf[kk] = u32x4_t{E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]), E::pack2(p[6], p[7])};
        }
        if constexpr (!ONES) l += (part[0] + part[1]) + (part[2] + part[3]);
    }

    // O^T += V^T P^T for the tile in V stage ST; V^T operand = two transpose
    // reads of 4 keys each
    template <int ST>
    __device__ __forceinline__ void pv(const u32x4_t (&pf)[KK]) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const u32x2_t lo = lds_read_tr(va[db] + ST * C::SSTR + 16 * kk * C::ROWB);
                const u32x2_t hi = lds_read_tr(va[db] + ST * C::SSTR + (16 * kk + 4) * C::ROWB);
                o[db] = E::mfma(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf[kk], o[db]);
            }
    }

    // The matrix half of a step: O^T += V^T P^T for the tile in V stage ST and
    // S^T = K Q^T for the tile in K stage ST1, in rounds of one P.V and one
    // score MFMA.  The LDS operands of round r+1 are read before round r's
    // MFMAs (scheduling fences keep the compiler from sinking the reads next to
    // their MFMAs), so two rounds of operands are live at a time.
    template <int ST, int ST1>
    __device__ __forceinline__ void pv_score(const u32x4_t (&pf)[KK], f32x16_t (&s)[SB]) {
        constexpr int NPV = KK * DBLK, NSC = KSTEPS * SB;
        constexpr int R = NPV > NSC ? NPV : NSC;
        u32x4_t vo[2], ko[2];
        auto rd = [&](int r) {
            if (r < NPV) {
                const int kk = r / DBLK, db = r % DBLK;
                const u32x2_t lo = lds_read_tr(va[db] + ST * C::SSTR + 16 * kk * C::ROWB);
                const u32x2_t hi = lds_read_tr(va[db] + ST * C::SSTR + (16 * kk + 4) * C::ROWB);
                vo[r & 1] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            }
            if (r < NSC) ko[r & 1] = lds_read16(ka[r / SB] + ST1 * C::SSTR + (r % SB) * 32 * C::ROWB);
        };
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) s[sb] = f32x16_t{};
        rd(0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r + 1 < R) rd(r + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (r < NPV) o[r % DBLK] = E::mfma(vo[r & 1], pf[r / DBLK], o[r % DBLK]);
            if (r < NSC) s[r % SB] = E::mfma(ko[r & 1], qf[r / SB], s[r % SB]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // O = acc / l rounded to the input type; lse = ln2 * (m + log2 l), written
    // to out / lse (may be null) as rows row .. row+31 of a [rows, D] array.  The
    // wave's 32 x D block goes through its own slice of LDS (32 rows of ROWB
    // bytes, the 16-byte chunk c of row r at c ^ (r % CPRP)) so that the global
    // stores are whole rows: each store instruction writes 64/CPRP consecutive
    // rows.  Only called when no wave reads the K/V stages and no tile load is
    // in flight (after the last barrier of a query tile, before the next one's
    // first).
    __device__ __forceinline__ void finish(const FwdArgs& a, int bh) { store(a.o, a.lse, (size_t)bh * N + qw0); }

    // the result of key-range part `part` of a query tile: rows past row0 in
    // the part's slice of the workspace
    __device__ __forceinline__ void finish_part(const FwdArgs& a, int bh, int part) {
        store(a.o_parts + (size_t)part * (size_t)a.rows * D, a.lse_parts + (size_t)part * (size_t)a.rows,
              (size_t)bh * N + qw0 - (size_t)a.row0);
    }

    __device__ __forceinline__ void store(uint16_t* out, float* lse, size_t row) {
        if (qw0 >= N) return;
        float ltot;
        if constexpr (ONES) ltot = pair_sum(hf == 0 ? o[LDB][LREG] : 0.f);
        else ltot = pair_sum(l);
        const float inv = 1.0f / ltot;   // rows past N are never stored
        const unsigned slice = lds0 + (unsigned)(wave * 32 * C::ROWB);
        // the lane's addresses are derived here from an opaque copy of the lane
        // index: computed once before the tile loop they would stay live across
        // it, and the registers they take get spilled
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int nn = ln & 31, hh = ln >> 5;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = 4 * db + g;                      // 16-byte chunk: d = 8c .. 8c+7, this lane's half hf
                if (c < CPR) {
                    const u32x2_t w = {E::pack2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                                       E::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                        (lds_bytes)(size_t)(slice + nn * C::ROWB + ((c ^ (nn & (C::CPRP - 1))) * 16) + 8 * hh)) = w;
                }
            }
        constexpr int RPR = 64 / C::CPRP;                     // rows per store round
        const int rr = ln / C::CPRP, c = ln % C::CPRP;
        uint16_t* obase = out + row * D;
        // every round's row read first, then the stores back to back
        u32x4_t v[32 / RPR];
#pragma unroll
        for (int k = 0; k < 32 / RPR; ++k) {
            const int r = k * RPR + rr;
            v[k] = lds_read16(slice + r * C::ROWB + ((c ^ (r & (C::CPRP - 1))) * 16));
        }
#pragma unroll
        for (int k = 0; k < 32 / RPR; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
        for (int k = 0; k < 32 / RPR; ++k) {
            const int r = k * RPR + rr;
            if (c < CPR && qw0 + r < N) {
                // O is written once and not read back here: the stores bypass L2 allocation
                __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4_t*>(obase + (unsigned)(r * D + 8 * c)));
            }
        }
        if (lse != nullptr && hf == 0 && qi < N) lse[row + n] = (m + __builtin_amdgcn_logf(ltot)) * kLn2;
    }
};

#endif  // __HIP_DEVICE_COMPILE__

// ---- the kernel ---------------------------------------------------------------
// 4 waves: free-running waves, two K/V stages.  8 waves: two wave groups in
// alternation over a three-stage K/V ring (see the kernel).
template <int WAVES> constexpr bool fwd_ping() { return WAVES == 8; }
template <int WAVES> constexpr int fwd_stages() { return fwd_ping<WAVES>() ? 3 : 2; }

// SPLIT (8 waves, no window): the key-split form of the two-group schedule.
// A work-group owns 128 query rows; wave w and wave w+4 hold the same 32 rows,
// group 0 over the first half of the item's key tiles and group 1 over the
// second half, each LDS stage holding one tile of each half; the two partial
// results of a row are merged through LDS at the end of the item.  Used for
// short problems where one 256-query work-group per CU would leave CUs idle
// and the 4-wave grid would leave them with one wave per SIMD.
//
// PARTS (8 waves, no mask, no window, no SPLIT): besides whole query tiles the
// work units include key-range parts of the last query tiles (see FwdArgs),
// so that an incomplete last round of the resident work-groups is spread over
// all of them; attn_lse_merge combines the parts afterwards.
template <int D, int DT, bool CAUSAL, int WAVES, bool WIN, bool SPLIT = false, bool PARTS = false>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    static_assert(!SPLIT || (WAVES == 8 && !WIN), "the key split is a form of the 8-wave schedule without a window");
    static_assert(!PARTS || (WAVES == 8 && !WIN && !SPLIT && !CAUSAL), "key-range parts: 8-wave unmasked schedule");
    static_assert(!SPLIT || !Wave<D, DT, CAUSAL, WAVES, WIN>::ONES, "the key split merges l, which ONES does not keep");
    constexpr int STAGES = fwd_stages<WAVES>();
    constexpr int SUBS = SPLIT ? 2 : 1;
    using C = Cfg<D, WAVES, STAGES, SUBS>;
    constexpr int BMQ = SPLIT ? 128 : C::BM;                // query rows per work item
    // the two-group schedule adds room for the Q slices of waves 4-7 (waves 0-3
    // use the K and V areas of stage 2, free while a query tile's loads start)
    constexpr int QEXTRA = fwd_ping<WAVES>() ? 4 * 32 * C::ROWB : 0;
    static_assert(C::LDS + QEXTRA <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS + QEXTRA];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    Wave<D, DT, CAUSAL, WAVES, WIN, STAGES, SUBS> w;
    const int half = SPLIT ? wave >> 2 : 0;                       // key half of this wave (key split)
    w.init(a, (unsigned)(size_t)(lds_bytes)smem, tid, wave, half);

    // Work units (a query tile, or a causal pair of them) blockIdx.x,
    // blockIdx.x + gridDim.x, ...: the grid is either one work-group per unit
    // or, for the 8-wave kernel, a multiple of 8 work-groups that stay resident
    // (a unit keeps its XCD since gridDim.x % 8 == 0).  With PARTS, units past
    // the whole ones are the parts of the remaining tiles, tile by tile.
    bool first = true;
    const int nunits = PARTS ? a.nwhole + a.nleft * a.nparts : a.nwhole;
    for (int unit = blockIdx.x; unit < nunits; unit += gridDim.x) {
    int bh, grp, part = -1;
    if (!PARTS || unit < a.nwhole) {
        map_workgroup(a, unit, a.nwhole, bh, grp);
    } else {
        const int u = unit - a.nwhole, left = u / a.nparts;
        part = u - left * a.nparts;
        const int g = a.nwhole + left;
        bh = g / a.ngroups;
        grp = g - bh * a.ngroups;
    }
    // a causal tile's keys grow with its index, so tiles i and nqt-1-i share a
    // unit; with a window every tile has about W keys and runs alone (a pair
    // would only put two tiles in sequence on one work-group)
    int nitems = CAUSAL && !WIN && grp != a.nqt - 1 - grp ? 2 : 1;
    int qt_one = -1;
    if (CAUSAL && WAVES == 4 && !WIN && a.unpaired) {
        // All U tiles in one round of two work-groups per CU.  With the tiles listed
        // longest first (tile index descending, heads within a tile index), units
        // 0 .. U/2-1 take the list from its head and units U/2 .. U-1 from its
        // tail, so the work-groups dispatched second, which fill the second slot of
        // each CU in the order the first ones took the first slot, pair a long tile
        // with a short one on every CU.
        const int U = a.nqt * a.BH, half = U / 2;
        const int d = unit < half ? unit : U - 1 - (unit - half);
        qt_one = a.nqt - 1 - d / a.BH;
        bh = d % a.BH;
        nitems = 1;
    }
    for (int item = 0; item < nitems; ++item, first = false) {
        const int qt = qt_one >= 0 ? qt_one : (CAUSAL && !WIN ? (item == 0 ? a.nqt - 1 - grp : grp) : grp);
        const int q0 = qt * BMQ;
        // Q rows come through LDS (q_issue / q_read) in every schedule
        w.begin(a, bh, q0 + 32 * (SPLIT ? wave & 3 : wave));
        // key tiles jlo .. nt-1: up to the last query (causal) or its band's end,
        // from the first query's band start
        const int win = WIN ? a.window : 0;
        const int kend = CAUSAL ? min(a.N, q0 + BMQ) : (win > 0 ? min(a.N, q0 + BMQ - 1 + win) : a.N);
        int nt = (kend + C::BN - 1) / C::BN;
        int jlo = win > 0 ? max(0, q0 - win + 1) / C::BN : 0;
        if (PARTS && part >= 0) {                          // key tiles of this part: an even share
            const int ti = nt - jlo;
            nt = jlo + ti * (part + 1) / a.nparts;
            jlo = jlo + ti * part / a.nparts;
        }

        if constexpr (fwd_ping<WAVES>()) {
            // Two groups of four waves, one wave of each on every SIMD.  Every
            // wave runs the same sequence per key tile u (u = 0 .. T-1 from jlo):
            //     Y(u)  barrier  X(u)  barrier
            // with Y(u) = the softmax half (mask, max, rescale, exponentials of
            // tile u's scores into P) and X(u) = the matrix half (O^T += V^T P^T
            // of tile u, then S^T = K Q^T of tile u+1).  Group 1 passes one
            // extra barrier before its first Y and group 0 one after its last
            // X, so between two barriers one wave of a SIMD issues MFMAs while
            // the other works through its exponentials:
            //     slot 2u+1: group 0 X(u),   group 1 Y(u)
            //     slot 2u+2: group 0 Y(u+1), group 1 X(u)
            // K/V tile u lives in LDS stage u % 3.  Tile u+2 is issued at the
            // start of slot 2u+1 into the stage of tile u-1, whose V was last
            // read in slot 2u, and every wave waits for its share at the end of
            // slot 2u+2, before that tile's K is first read in slot 2u+3.
            // With the key split, step u of group g works on key tile jlo + g H + u
            // (H = the first half's tile count) and stage u % 3 holds both groups'
            // tiles of step u.
            if (!first) __syncthreads();                   // every wave has left the previous item's tiles
            const bool g0 = wave < 4;                      // wave-uniform
            const int TI = nt - jlo;                       // key tiles of the item
            const int H = SPLIT ? (TI + 1) / 2 : TI;       // steps (the first half's tiles)
            const int T = H;
            const int j0 = jlo + half * H;                 // this wave's first tile
            const int jend = SPLIT && half == 0 ? jlo + H : nt;
            // keys for this wave in step u (without the split every step has a tile: testing it spills registers)
            auto has = [&](int u) { return (!SPLIT || j0 + u < jend) && w.active(j0 + u); };
            f32x16_t s[C::SB];                             // scores of the tile whose softmax is next
            u32x4_t pf[C::KK];                             // P of the tile whose P.V is next
            // One code path for the matrix half keeps register use low: a wave
            // with no P.V for tile u multiplies a zero P, and a score computed
            // past the wave's last tile is not used.
            auto X = [&](auto stage_tag, int u) {
                constexpr int ST = decltype(stage_tag)::value, ST1 = (ST + 1) % 3;
                const bool do_pv = has(u), do_s = u + 1 < T && has(u + 1);
                if (do_pv || do_s) {
                    if (!do_pv) {
#pragma unroll
                        for (int kk = 0; kk < C::KK; ++kk) pf[kk] = u32x4_t{0, 0, 0, 0};
                    }
                    __builtin_amdgcn_s_setprio(2);
                    w.template pv_score<ST, ST1>(pf, s);
                    __builtin_amdgcn_s_setprio(0);
                }
            };
            // the tiles of step t into stage `stage`: K (is_v false) or V
            auto issue_step = [&](bool is_v, int t, int stage) {
                if (t < H) w.issue(is_v, jlo + t, stage, 0);
                if (SPLIT && H + t < TI) w.issue(is_v, jlo + H + t, stage, 1);
            };
            auto issue_tile = [&](auto stage_tag, int u) {
                constexpr int ST2 = (decltype(stage_tag)::value + 2) % 3;
                issue_step(false, u + 2, ST2);
                issue_step(true, u + 2, ST2);
            };
            auto tile = [&](auto stage_tag, int u) {
                constexpr int ST = decltype(stage_tag)::value;
                if (!g0) issue_tile(stage_tag, u);          // slot 2u+1 starts (group 1)
                if (has(u)) {
                    w.prepare(s, j0 + u);
                    w.probs(s, pf);
                }
                if (g0) {
                    wait_loads();                           // slot 2u ends (group 0): tile u+1 landed
                    if (u == 0) w.template ones<0>();       // (and tile 0, from the prologue)
                    if (u + 1 < T) w.template ones<(ST + 1) % 3>();
                }
                __syncthreads();
                if (g0) issue_tile(stage_tag, u);           // slot 2u+1 starts (group 0)
                X(stage_tag, u);
                if (!g0) {
                    wait_loads();                           // slot 2u+2 ends (group 1): tile u+2 landed
                    if (u + 2 < T) w.template ones<(ST + 2) % 3>();
                }
                __syncthreads();
            };
            // this wave's Q slice: stage 2's K area (waves 0, 1), its V area (2, 3) or
            // the extra room past the stages (4-7); stage 2 first receives a tile
            // after the barrier below
            const unsigned lds_base = (unsigned)(size_t)(lds_bytes)smem;
            const unsigned qslice = lds_base + (unsigned)((wave < 2   ? C::KOFF + 2 * C::SSTR + wave * 32 * C::ROWB
                                                           : wave < 4 ? C::VOFF + 2 * C::SSTR + (wave - 2) * 32 * C::ROWB
                                                                      : C::LDS + (wave - 4) * 32 * C::ROWB));
            if (w.qw0 < a.N) w.q_issue(a, bh, qslice);
            issue_step(false, 0, 0);
            issue_step(true, 0, 0);
            issue_step(false, 1, 1);
            issue_step(true, 1, 1);
            // only Q and step 0's K are needed for the first scores: step 0's V and
            // step 1's tiles (issued after them) are waited for before the barrier
            // that ends slot 0 (group 0 in its first tile step, group 1 just below)
            {
                const int tiles0 = SPLIT && H < TI ? 2 : 1;                  // tiles in step 0
                const int tiles1 = (1 < H ? 1 : 0) + (SPLIT && H + 1 < TI ? 1 : 0);
                const int after = (SPLIT ? tiles0 : 1) + 2 * tiles1;          // K/V loads issued after step 0's K
                if (!SPLIT) {
                    if (T > 1) wait_vmcnt<3 * C::IT>();
                    else wait_vmcnt<C::IT>();
                } else if (tiles0 == 2) {
                    // order: K0a, K0b, V0a, V0b, K1a, K1b, V1a, V1b; wait for Q, K0a, K0b
                    // (each wave's loads complete in order: K0b is the second K)
                    if (after >= 6) wait_vmcnt<6 * C::IT>();
                    else if (after >= 4) wait_vmcnt<4 * C::IT>();
                    else if (after >= 3) wait_vmcnt<3 * C::IT>();
                    else wait_vmcnt<2 * C::IT>();
                } else {
                    if (after >= 3) wait_vmcnt<3 * C::IT>();
                    else wait_vmcnt<C::IT>();
                }
            }
            w.q_read(a, qslice);                           // this wave's own loads: no barrier needed
            __syncthreads();
            if (has(0)) w.template score<0>(s);
            if (!g0) {
                wait_loads();
                w.template ones<0>();
                if (T > 1) w.template ones<1>();
                __syncthreads();
            }
            for (int u = 0; u < T; u += 3) {
                tile(std::integral_constant<int, 0>{}, u);
                if (u + 1 < T) tile(std::integral_constant<int, 1>{}, u + 1);
                if (u + 2 < T) tile(std::integral_constant<int, 2>{}, u + 2);
            }
            if (g0) __syncthreads();
            if constexpr (SPLIT) {
                // group 1 hands its partial (m, l, O^T) to the group-0 wave with the same
                // rows through the V stages (idle now; the epilogue's slices lie in the K
                // stages): register i of lane L at float i * 64 + L of the wave's area
                constexpr int NV = 16 * C::DBLK + 2;       // floats per lane
                static_assert(4 * NV * 64 * 4 <= C::STAGES * C::SSTR, "merge areas fit the V stages");
                float* area = reinterpret_cast<float*>(smem + C::VOFF) + (wave & 3) * NV * 64;
                const int ln = tid & 63;
                if (!g0) {
#pragma unroll
                    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) area[(16 * db + i) * 64 + ln] = w.o[db][i];
                    area[(NV - 2) * 64 + ln] = w.m;
                    area[(NV - 1) * 64 + ln] = w.l;
                }
                __syncthreads();
                if (g0) {
                    // m in log2 units; a half with no kept key has m = -inf, l = 0, O = 0
                    const float mb = area[(NV - 2) * 64 + ln], lb = area[(NV - 1) * 64 + ln];
                    const float mm = fmaxf(w.m, mb);
                    const float fa = mm > kNegInf ? __builtin_amdgcn_exp2f(w.m - mm) : 0.f;
                    const float fb = mm > kNegInf ? __builtin_amdgcn_exp2f(mb - mm) : 0.f;
#pragma unroll
                    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) w.o[db][i] = w.o[db][i] * fa + area[(16 * db + i) * 64 + ln] * fb;
                    w.l = w.l * fa + lb * fb;
                    w.m = mm;
                    w.finish(a, bh);
                }
            } else if (PARTS && part >= 0) {
                w.finish_part(a, bh, part);
            } else {
                w.finish(a, bh);
            }
            continue;
        }

        if (!first) __syncthreads();                       // every wave has left the previous item's epilogue
        // one step: prefetch tile j+1 into the other stage, compute tile j, sync.
        // The wave raises its priority while it issues the score MFMAs, so the
        // matrix pipe is fed as soon as it frees up while the other wave on the
        // SIMD works through its exponentials.
        auto step = [&](auto stage_tag, int j) {
            constexpr int ST = decltype(stage_tag)::value;
            if (j + 1 < nt) {
                w.issue(false, j + 1, ST ^ 1);
                w.issue(true, j + 1, ST ^ 1);
            }
            if (w.active(j)) {
                f32x16_t s[C::SB];
                u32x4_t pf[C::KK];
                __builtin_amdgcn_s_setprio(2);
                w.template score<ST>(s);
                __builtin_amdgcn_s_setprio(0);
                w.prepare(s, j);
                w.probs(s, pf);
                w.template pv<ST>(pf);
            }
            wait_loads();
            if (j + 1 < nt) w.template ones<ST ^ 1>();
            __syncthreads();
        };
        // the Q slices of the 4-wave kernel: stage 1's K area (waves 0, 1) and V
        // area (2, 3); stage 1 first receives a tile after the barrier below
        const unsigned qslice = (unsigned)(size_t)(lds_bytes)smem +
                                (unsigned)(wave < 2 ? C::KOFF + C::SSTR + wave * 32 * C::ROWB
                                                    : C::VOFF + C::SSTR + (wave - 2) * 32 * C::ROWB);
        if (w.qw0 < a.N) w.q_issue(a, bh, qslice);           // four Q slices fill stage 1
        w.issue(false, jlo, 0);
        w.issue(true, jlo, 0);
        wait_loads();
        w.template ones<0>();
        w.q_read(a, qslice);                               // this wave's own loads: no barrier needed
        __syncthreads();
        for (int j = jlo; j < nt; j += 2) {                 // tile j in stage (j - jlo) & 1
            step(std::integral_constant<int, 0>{}, j);
            if (j + 1 < nt) step(std::integral_constant<int, 1>{}, j + 1);
        }
        w.finish(a, bh);
    }
    }
#endif
}

// --- host side ---------------------------------------------------------------

// Work-groups of 256 queries needed before the 8-wave kernel is used: below
// about two rounds of the 256 CUs (one such work-group fits per CU) the
// 128-query work-groups fill the chip better.
constexpr long long kWideMinGroups = 512;

bool use_wide(long long bh, long long N, int causal) {
    const long long nqt = (N + 255) / 256;
    return (causal ? (nqt + 1) / 2 : nqt) * bh >= kWideMinGroups;
}

// The key-split form of the 8-wave schedule (d = 64: its stages of two tiles
// fit the LDS; no window) where the 4-wave grid would leave CUs with one
// work-group, i.e. one wave per SIMD (fewer than two work-groups per CU of a
// 256-CU MI355X), and the query tiles are long: measured against the 4-wave
// schedule, +6.6% at B=1 H=16 N=4096 causal and +3.2% at B=2 H=16 N=2048
// causal, but -4% at N=1024 and -18% at N=128, where the fixed cost of each
// query tile (first loads, merge, epilogue) outweighs the overlap it gains.
// Causal problems below 4096 keys whose single query tiles fit one round of
// two 4-wave work-groups per CU run those unpaired instead (use_unpaired, with
// the 256 CUs of an MI355X): +1.6 to +8.4% over the key split at N = 2048,
// -5.9% at N = 4096.
constexpr long long kSplitBelowGroups = 512;
constexpr long long kSplitMinN = 2048;
constexpr long long kUnpairedOverSplitBelowN = 4096;
constexpr long long kUnpairedMaxTiles = 512;

bool use_split(long long bh, long long N, int d, int causal, int window) {
    if (d != 64 || window > 0 || N < kSplitMinN || use_wide(bh, N, causal)) return false;
    if (causal && N < kUnpairedOverSplitBelowN && ((N + 127) / 128) * bh <= kUnpairedMaxTiles) return false;
    const long long nqt = (N + 127) / 128;
    return (causal ? (nqt + 1) / 2 : nqt) * bh < kSplitBelowGroups;
}

// Resident work-groups for the 8-wave schedule: one per CU (its LDS stages
// leave room for no second one), each looping over work units, so that the
// grid runs as one round instead of several.

// Causal 4-wave grids whose single query tiles fit one round of two work-groups
// per CU run them unpaired, longest first (see the kernel): measured +13% at
// B=4 H=16 N=1024 d=64 and +13-35% on other such shapes, but -11% at twice that
// many tiles, where the pairs keep every round balanced.
bool use_unpaired(long long bh, long long N, int causal, int window, int cus) {
    return causal && window == 0 && cus > 0 && ((N + 127) / 128) * bh <= 2LL * cus;
}

template <int D, int DT, bool CAUSAL, int WAVES, bool WIN, bool SPLIT = false>
hipError_t launch_waves(FwdArgs a, hipStream_t stream, int cus) {
    constexpr int BM = SPLIT ? 128 : Cfg<D, WAVES>::BM;
    const long long nqt = ((long long)a.N + BM - 1) / BM;
    a.nqt = (int)nqt;
    a.unpaired = WAVES == 4 && !WIN && use_unpaired(a.BH, a.N, CAUSAL, a.window, cus) ? 1 : 0;
    a.ngroups = CAUSAL && !WIN && !a.unpaired ? (int)((nqt + 1) / 2) : (int)nqt;
    const unsigned units = (unsigned)a.ngroups * (unsigned)a.BH;
    a.nwhole = (int)units;
    unsigned grid = units;
    if (fwd_ping<WAVES>() && cus >= 8 && units > (unsigned)cus) grid = (unsigned)cus & ~7u;
    return launch_kernel(attn_fwd_kernel<D, DT, CAUSAL, WAVES, WIN, SPLIT>, dim3(grid), dim3(64 * WAVES), stream, a);
}

// Key-range parts (attn_fwd_ws).  With I query tiles of 256 rows over S
// resident 8-wave work-groups, a last round of r = I mod S tiles would leave
// S - r CUs idle for a whole tile's time.  Instead the last r tiles (in
// (head, tile) order, so their rows are one contiguous range) are each cut
// into P = min(S / r, key tiles / 2) key ranges that run as one short round on
// all work-groups, and attn_lse_merge combines the P partial results.  Only
// without a mask: a causal problem already pairs its tiles to equal work.
struct PartPlan {
    int nwhole = 0, nleft = 0, nparts = 0;
    long long row0 = 0, rows = 0;
    size_t o_bytes = 0, lse_bytes = 0, tmp_bytes = 0;   // workspace: O parts, lse parts, merged lse
    size_t total() const { return o_bytes + lse_bytes + tmp_bytes; }
};

constexpr long long kPartMinTiles = 2;   // key tiles per part at least

PartPlan plan_parts(long long bh, long long N, int d, int causal, int cus) {
    PartPlan p;
    if (causal || cus < 8) return p;
    const long long S = cus & ~7, nqt = (N + 255) / 256, items = nqt * bh;
    const long long r = items % S;
    if (r == 0) return p;
    const long long P = std::min(S / r, ((N + 63) / 64) / kPartMinTiles);
    if (P < 2) return p;
    p.nparts = (int)P;
    p.nleft = (int)r;
    p.nwhole = (int)(items - r);
    p.row0 = (p.nwhole / nqt) * N + (p.nwhole % nqt) * 256;
    p.rows = bh * N - p.row0;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p.o_bytes = up((size_t)P * (size_t)p.rows * (size_t)d * 2u);
    p.lse_bytes = up((size_t)P * (size_t)p.rows * 4u);
    p.tmp_bytes = up((size_t)p.rows * 4u);
    return p;
}

template <int D, int DT>
hipError_t launch_parts(FwdArgs a, const PartPlan& p, hipStream_t stream, int cus) {
    a.nqt = (a.N + 255) / 256;
    a.ngroups = a.nqt;
    a.nwhole = p.nwhole;
    a.nleft = p.nleft;
    a.nparts = p.nparts;
    a.row0 = p.row0;
    a.rows = p.rows;
    const unsigned grid = (unsigned)cus & ~7u;
    return launch_kernel(attn_fwd_kernel<D, DT, false, 8, false, false, true>, dim3(grid), dim3(512), stream, a);
}

template <int D, int DT, bool CAUSAL>
hipError_t launch(FwdArgs a, hipStream_t stream, int cus) {
    if constexpr (D == 64) {
        if (use_split(a.BH, a.N, D, CAUSAL, a.window)) return launch_waves<D, DT, CAUSAL, 8, false, true>(a, stream, cus);
    }
    const bool wide = use_wide(a.BH, a.N, CAUSAL);
    if (a.window > 0)
        return wide ? launch_waves<D, DT, CAUSAL, 8, true>(a, stream, cus)
                    : launch_waves<D, DT, CAUSAL, 4, true>(a, stream, cus);
    return wide ? launch_waves<D, DT, CAUSAL, 8, false>(a, stream, cus)
                : launch_waves<D, DT, CAUSAL, 4, false>(a, stream, cus);
}

template <int D, int DT>
hipError_t dispatch_causal(const FwdArgs& a, int causal, hipStream_t s, int cus) {
    return causal ? launch<D, DT, true>(a, s, cus) : launch<D, DT, false>(a, s, cus);
}

template <int D>
hipError_t dispatch_dtype(const FwdArgs& a, int dtype, int causal, hipStream_t s, int cus) {
    return dtype == ATTN_BF16 ? dispatch_causal<D, ATTN_BF16>(a, causal, s, cus)
                              : dispatch_causal<D, ATTN_F16>(a, causal, s, cus);
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];       // compute units, once known

// ATTN_OK when the current device is a gfx950; *cus receives its compute-unit count
int check_device(int* cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int st = g_arch_ok[dev].load(std::memory_order_acquire);
        if (st == 1) {
            *cus = g_cus[dev].load(std::memory_order_relaxed);
            return ATTN_OK;
        }
        if (st == 2) return ATTN_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    *cus = prop.multiProcessorCount;
    if (dev < kMaxDevices) {
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_release);
    }
    return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

// shape checks shared by attn_fwd and attn_fwd_schedule
int check_shape(int B, int H, int N, int d, int causal) {
    if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 80 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
    const long long bh = (long long)B * H;
    const long long nqt = ((long long)N + 127) / 128;   // the smaller query tile bounds the grid
    if (bh > INT32_MAX || nqt * bh > INT32_MAX) return ATTN_ERR_SHAPE;
    if ((long long)N * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;   // one head must fit a 32-bit buffer range
    return ATTN_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

namespace {

// Argument checks of every forward entry point (nothing touches the device
// before they pass) and the kernel arguments they imply.
int prepare(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
            int causal, int window, float scale, int dtype, FwdArgs& a, int& cus) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 80 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return ATTN_ERR_CAUSAL;
    if (window < 0) return ATTN_ERR_WINDOW;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return ATTN_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;
    const int shape_status = check_shape(B, H, N, d, causal);
    if (shape_status != ATTN_OK) return shape_status;

    const long long bh = (long long)B * H;
    const size_t tensor_bytes = (size_t)bh * (size_t)N * (size_t)d * 2u;
    const size_t lse_bytes = (size_t)bh * (size_t)N * 4u;
    if (overlaps(out, tensor_bytes, q, tensor_bytes) || overlaps(out, tensor_bytes, k, tensor_bytes) ||
        overlaps(out, tensor_bytes, v, tensor_bytes))
        return ATTN_ERR_ALIAS;
    if (lse && (overlaps(lse, lse_bytes, q, tensor_bytes) || overlaps(lse, lse_bytes, k, tensor_bytes) ||
                overlaps(lse, lse_bytes, v, tensor_bytes) || overlaps(lse, lse_bytes, out, tensor_bytes)))
        return ATTN_ERR_ALIAS;

    const int dev_status = check_device(&cus);
    if (dev_status != ATTN_OK) return dev_status;

    a = FwdArgs{};
    a.q = static_cast<const u32x4_t*>(q);
    a.k = static_cast<const u32x4_t*>(k);
    a.v = static_cast<const u32x4_t*>(v);
    a.o = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.N = N;
    a.BH = (int)bh;
    a.nqt = 0;       // set per kernel by the launcher
    a.ngroups = 0;
    // c must be > 0 so that masked scores (-inf) map to -inf; scale == 0 uses the
    // smallest normal float, which makes every exponent round to exactly 0
    a.c = scale == 0.f ? FLT_MIN : std::fabs(scale) * kLog2e;
    a.qsign = std::signbit(scale) && scale != 0.f ? 0x80008000u : 0u;
    a.window = window >= N ? 0 : window;   // a band of N or more keeps every key the mask allows
    return ATTN_OK;
}

int fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d, int causal,
        int window, float scale, int dtype, void* stream) {
    FwdArgs a;
    int cus = 0;
    const int st = prepare(q, k, v, out, lse, B, H, N, d, causal, window, scale, dtype, a, cus);
    if (st != ATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (d) {
        case 64: err = dispatch_dtype<64>(a, dtype, causal, s, cus); break;
        case 80: err = dispatch_dtype<80>(a, dtype, causal, s, cus); break;
        default: err = dispatch_dtype<128>(a, dtype, causal, s, cus); break;
    }
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <int D>
hipError_t dispatch_parts(const FwdArgs& a, const PartPlan& p, int dtype, hipStream_t s, int cus) {
    return dtype == ATTN_BF16 ? launch_parts<D, ATTN_BF16>(a, p, s, cus) : launch_parts<D, ATTN_F16>(a, p, s, cus);
}

int fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
           int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    FwdArgs a;
    int cus = 0;
    const int st = prepare(q, k, v, out, lse, B, H, N, d, causal, 0, scale, dtype, a, cus);
    if (st != ATTN_OK) return st;
    const PartPlan p = plan_parts(a.BH, N, d, causal, cus);
    if (workspace == nullptr || p.nparts == 0) return fwd(q, k, v, out, lse, B, H, N, d, causal, 0, scale, dtype, stream);
    if (workspace_bytes < p.total()) return ATTN_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return ATTN_ERR_ALIGN;
    const size_t tensor_bytes = (size_t)a.BH * (size_t)N * (size_t)d * 2u;
    const size_t lse_bytes = (size_t)a.BH * (size_t)N * 4u;
    if (overlaps(workspace, p.total(), q, tensor_bytes) || overlaps(workspace, p.total(), k, tensor_bytes) ||
        overlaps(workspace, p.total(), v, tensor_bytes) || overlaps(workspace, p.total(), out, tensor_bytes) ||
        (lse && overlaps(workspace, p.total(), lse, lse_bytes)))
        return ATTN_ERR_ALIAS;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    a.o_parts = reinterpret_cast<uint16_t*>(ws);
    a.lse_parts = reinterpret_cast<float*>(ws + p.o_bytes);
    float* lse_merged = lse ? lse + p.row0 : reinterpret_cast<float*>(ws + p.o_bytes + p.lse_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (d) {
        case 64: err = dispatch_parts<64>(a, p, dtype, s, cus); break;
        case 80: err = dispatch_parts<80>(a, p, dtype, s, cus); break;
        default: err = dispatch_parts<128>(a, p, dtype, s, cus); break;
    }
    if (err != hipSuccess) return ATTN_ERR_LAUNCH;
    // the rows of the cut tiles: O and lse from their parts, on the same stream
    const int mst = attn_lse_merge(a.o_parts, a.lse_parts, p.nparts, static_cast<uint16_t*>(out) + p.row0 * d,
                                   lse_merged, p.rows, d, dtype, stream);
    return mst == ATTN_OK ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int N, int d, int causal, float scale, int dtype, void* stream) {
    return fwd(q, k, v, out, lse, B, H, N, d, causal, 0, scale, dtype, stream);
}

extern "C" int attn_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse,
                               int B, int H, int N, int d, int causal, int window, float scale, int dtype,
                               void* stream) {
    return fwd(q, k, v, out, lse, B, H, N, d, causal, window, scale, dtype, stream);
}

extern "C" int attn_fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N,
                           int d, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return fwd_ws(q, k, v, out, lse, B, H, N, d, causal, scale, dtype, workspace, workspace_bytes, stream);
}

extern "C" long long attn_fwd_workspace_bytes(int B, int H, int N, int d, int causal) {
    const int st = check_shape(B, H, N, d, causal);
    if (st != ATTN_OK) return -st;
    int cus = 0;
    const int dev_status = check_device(&cus);
    if (dev_status != ATTN_OK) return -dev_status;
    return (long long)plan_parts((long long)B * H, N, d, causal, cus).total();
}

extern "C" int attn_fwd_schedule(int B, int H, int N, int d, int causal) {
    const int st = check_shape(B, H, N, d, causal);
    if (st != ATTN_OK) return -st;
    const long long bh = (long long)B * H;
    if (use_split(bh, N, d, causal, 0)) return ATTN_SCHEDULE_SPLIT;
    return use_wide(bh, N, causal) ? ATTN_SCHEDULE_WIDE : ATTN_SCHEDULE_SMALL;
}
