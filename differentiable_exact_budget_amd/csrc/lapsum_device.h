// Device-side definitions shared by the HIP kernels of the Fast LapSum solver
// (gfx950, wave64).  Host code includes it for the control-block layout only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace lapsum {

// ---------------------------------------------------------------------------
// sizes
// ---------------------------------------------------------------------------
constexpr int kStreamThreads = 256;      // streaming kernels (filter, p, VJP)
constexpr int kMaxStreamBlocks = 2048;   // 256 CUs x 8 resident blocks
constexpr int kMaxStreamParts = 131072;  // workgroups of a tiled streaming pass that leave partials
constexpr int kMaxBuckets = 1024;        // band buckets
constexpr int kBucketCapMax = 16384;     // band scores per bucket (LDS sort capacity)
constexpr int kSortThreads = 1024;       // single-workgroup LDS sort / solve
constexpr int kSortItems = 16;           // keys per thread in the LDS sort
constexpr int kSmallMax = kSortThreads * kSortItems;  // 16384
constexpr int kRadixThreads = 256;       // multi-workgroup radix pass
constexpr int kRadixItems = 16;
constexpr int kRadixTile = kRadixThreads * kRadixItems;  // 4096 keys
constexpr int kRadixHistBlocks = 512;
constexpr int kHistStride = 1028;        // 4 x 256 digit counts + a non-finite flag, per workgroup
constexpr int kHistGlobalCopies = 8;     // copies of the radix sort's global digit totals
constexpr int kHistGlobalWords = kHistGlobalCopies * 1024 + 1;  // the copies, then a non-finite flag
// the split radix passes' digit totals (eight per-XCD copies of 256 uint32
// words, for the pass under way) and their non-finite flag (uint64 word
// 4 * 256), inside the same region
constexpr int kSplitTotOffset = ((kHistGlobalWords + 63) / 64) * 64;  // uint32 words
constexpr int kSplitTotWords = 4 * 256 + 1;                            // uint64 words
constexpr int kHistRegionWords = kSplitTotOffset + 2 * kSplitTotWords;  // uint32 words, zero on entry and exit
constexpr int kCurveThreads = 256;
constexpr int kCurveTile = kRadixTile;   // sorted keys per curve segment
constexpr int kCurveRootThreads = 1024;  // the full-sort root's workgroup
constexpr int kSplitThreads = 512;       // split radix passes: threads per workgroup (>= 256)
constexpr int kSplitItems = 8;           // split radix passes: keys per thread
constexpr int kSplitTileKeys = kSplitThreads * kSplitItems;
constexpr int kSampleMax = 40960;        // sample size cap (select holds it in registers)
constexpr int kSelectThreads = 1024;
constexpr int kSelectItems = kSampleMax / kSelectThreads;  // 40
constexpr int kCandMax = 2048;           // sample values kept for the splitters
constexpr int kSelHistShift = 20;        // sample histogram bin of a key: its leading 12 bits
constexpr int kSelHistBins = 1 << (32 - kSelHistShift);  // 4096
constexpr int kWinMax = 4096;            // sample keys the select sorts around ranks l..h
constexpr int kWinHdr = 4;               // window buffer header: fill count, ok, size, keys below

// control-block flags
constexpr int kFlagNonFinite = 1;
constexpr int kFlagOverflow = 2;
constexpr int kFlagInternal = 4;
constexpr int kFlagBigRoot = 8;   // the root lies in a bucket too large for LDS (host sorts it)
constexpr int kFlagCertified = 16;  // G(a_L) >= k > G(a_R) from the filter's sums
constexpr int kFlagHeavy = 32;      // certified with overflowed buckets, and slots for them laid out
constexpr uint32_t kNotHeavy = 0xFFFFFFFFu;  // bucket slot offset marker: not an overflowed bucket
constexpr int kHeavyChunk = 2048;   // scores of an overflowed bucket per aggregation workgroup

// ---------------------------------------------------------------------------
// control block: one per workspace, in device memory
// ---------------------------------------------------------------------------
struct Ctl {
    // bracket and bucket layout (written by the select kernel)
    float aL, aR;
    int32_t ng;       // gaps between consecutive splitters
    int32_t J;        // equal-width sub-buckets per finite gap
    int32_t nb;       // ng * J buckets
    int32_t flags;    // kFlag*
    int32_t cap;      // bucket capacity in use
    int32_t pad0;
    // streaming filter results (written by the filter's last workgroup)
    unsigned long long c_L, m, c_R;
    double S_L, S_R, B_L, B_R;
    // solve
    double b;
    long long jstar;  // 0-based sorted index of the interval's lower end (-1: below the first)
    // p pass
    double sum_p;
    // VJP
    double sumfg, sumf, c;
    // last-workgroup tickets (each returns to 0 after use)
    unsigned int done[8];
    // radix sort: tile counters of the look-back passes, and 1 when this sort
    // holds the device's resident-pass lock (set by the histogram kernel)
    unsigned int tile_ctr[4];
    int resident;
    unsigned int pad1[3];
    // 1 when the filter certified the bracket with every band score stored:
    // the band solve and p pass launched right behind it then do their work
    int32_t gate;
    int32_t pad2;
    // overflowed buckets: aggregation chunks, and the slot offset of a root
    // bucket too large for LDS (for the host's sort)
    uint32_t hchunks;
    uint32_t pad3;
    unsigned long long root_off;
    // G at the bracket ends from the filter's sums (kept for the summary the
    // certification pass writes when it decides instead)
    double gL_alg, gR_alg;
    unsigned long long max_bucket, heavy_total;  // largest bucket count; scores in overflowed buckets
};

// Slots of the overflowed ("heavy") buckets, laid out by the filter's
// finalize kernel: per bucket its slot offset (kNotHeavy for the others),
// fill count, smallest and largest score key, and first aggregation chunk;
// per chunk its four 64-bit fixed-point partial sums.
struct HeavyArrays {
    uint32_t* hoff;
    uint32_t* hfill;
    uint32_t* hmin;
    uint32_t* hmax;
    uint32_t* hch0;
    unsigned long long* hpart;
    unsigned long long base_off;   // slot offsets start here (elements past bucket_vals)
    unsigned long long cap_total;  // scores the slot region holds
};

// host-pinned summary written by the filter's last workgroup; the host polls seq
struct HostSummary {
    unsigned long long c_L, m, c_R;
    double S_L, S_R, B_L, B_R;
    double g_aL, g_aR;  // G at the bracket ends from the filter's sums
    double g_aL_direct, g_aR_direct;  // the same summed directly by the certification pass (when it ran)
    float aL, aR;
    int32_t flags;
    int32_t nb;
    unsigned long long max_bucket;
    unsigned long long heavy_total;  // scores in overflowed buckets (kFlagHeavy)
    uint32_t hchunks;                // their aggregation chunks
    volatile unsigned int seq;
    // written by the band solve of overflowed buckets when asked to
    unsigned long long root_off;  // slot of a root bucket too large for LDS
    unsigned long long root_m;    // its score count
    int32_t root_flags;
    volatile unsigned int root_seq;
};

enum DoneSlot { kDoneFilter = 0, kDoneHist = 1, kDoneCurve = 2, kDoneBucket = 3, kDoneProbs = 4, kDoneVjp = 5 };

#ifdef __HIP_DEVICE_COMPILE__
#define LS_DEV __device__ __forceinline__
#else
#define LS_DEV __device__ __forceinline__
#endif

// ---------------------------------------------------------------------------
// order-preserving fp32 <-> u32 keys (-0.0 is read as +0.0)
// ---------------------------------------------------------------------------
LS_DEV uint32_t f2key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
LS_DEV float key2f(uint32_t k) {
    uint32_t u = k ^ ((k >> 31) ? 0x80000000u : 0xFFFFFFFFu);
    return __uint_as_float(u);
}
LS_DEV bool finite_f(float v) { return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u; }

// e^y for y <= 0 with the hardware exp2 (1 ulp); argument pre-scaled by log2(e)
LS_DEV float exp_neg(float y) { return __builtin_amdgcn_exp2f(y * 1.4426950408889634f); }

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
LS_DEV int lane_id() { return __lane_id(); }
LS_DEV unsigned long long ballot(bool p) { return __ballot(p); }
// number of set bits of mask below this lane
LS_DEV int mbcnt(unsigned long long mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}
LS_DEV int popc64(unsigned long long m) { return __popcll(m); }

// lanes of `active` whose 8-bit digit equals this lane's digit
LS_DEV unsigned long long match_digit8(uint32_t d, unsigned long long active) {
    unsigned long long m = active;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const unsigned long long bal = ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// The value of lane (lane XOR D) for D = 1 .. 32 with data-parallel
// primitives instead of an LDS permute: DPP quad permutations (D = 1, 2),
// row shifts into alternate 4-lane banks (D = 4), a row rotation (D = 8),
// and the gfx950 row-pair / half-wave swaps (D = 16, 32).  All 64 lanes must
// be active.
template <int D>
LS_DEV uint32_t xor_lane(uint32_t x) {
    static_assert(D == 1 || D == 2 || D == 4 || D == 8 || D == 16 || D == 32, "lane distance");
    if constexpr (D == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (D == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (D == 4) {
        const int y = __builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xA, false);  // row_shr:4 -> banks 1, 3
        return (uint32_t)__builtin_amdgcn_update_dpp(y, (int)x, 0x104, 0xF, 0x5, false);  // row_shl:4 -> banks 0, 2
    } else if constexpr (D == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return ((__lane_id() >> 4) & 1) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return ((__lane_id() >> 5) & 1) ? r[0] : r[1];
    }
}
template <int D>
LS_DEV unsigned long long xor_lane64(unsigned long long x) {
    return ((unsigned long long)xor_lane<D>((uint32_t)(x >> 32)) << 32) | xor_lane<D>((uint32_t)x);
}
template <int D>
LS_DEV double xor_lane_f64(double x) {
    return __longlong_as_double((long long)xor_lane64<D>((unsigned long long)__double_as_longlong(x)));
}
// run-time lane distance (a power of two, 1 .. 32, wave-uniform)
LS_DEV uint32_t xor_lane_rt(uint32_t x, int d) {
    switch (d) {
        case 1: return xor_lane<1>(x);
        case 2: return xor_lane<2>(x);
        case 4: return xor_lane<4>(x);
        case 8: return xor_lane<8>(x);
        case 16: return xor_lane<16>(x);
        default: return xor_lane<32>(x);
    }
}

// fixed-order butterfly sums over the wave
LS_DEV double wave_sum(double v) {
    v += xor_lane_f64<32>(v);
    v += xor_lane_f64<16>(v);
    v += xor_lane_f64<8>(v);
    v += xor_lane_f64<4>(v);
    v += xor_lane_f64<2>(v);
    v += xor_lane_f64<1>(v);
    return v;
}
LS_DEV unsigned long long wave_sum_u64(unsigned long long v) {
    v += xor_lane64<32>(v);
    v += xor_lane64<16>(v);
    v += xor_lane64<8>(v);
    v += xor_lane64<4>(v);
    v += xor_lane64<2>(v);
    v += xor_lane64<1>(v);
    return v;
}
LS_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, xor_lane<32>(v));
    v = max(v, xor_lane<16>(v));
    v = max(v, xor_lane<8>(v));
    v = max(v, xor_lane<4>(v));
    v = max(v, xor_lane<2>(v));
    v = max(v, xor_lane<1>(v));
    return v;
}

// Inclusive scans over the wave as a butterfly of lane exchanges: at
// distance D each lane takes the total of its partner's aligned D-block and
// adds it when that block lies before it (after it, for a reverse scan).
// The exchanges are DPP / lane swaps, not LDS permutes; the order of the
// additions is fixed.  All 64 lanes must be active.
template <int D>
LS_DEV void scan_step_u32(uint32_t& v, uint32_t& tot, int l) {
    const uint32_t o = xor_lane<D>(tot);
    if (l & D) v += o;
    tot += o;
}
template <int D>
LS_DEV void scan_step_max_f32(float& v, float& tot, int l) {
    const float o = __uint_as_float(xor_lane<D>(__float_as_uint(tot)));
    if (l & D) v = fmaxf(v, o);
    tot = fmaxf(tot, o);
}
template <int D>
LS_DEV void rscan_step_min_f32(float& v, float& tot, int l) {
    const float o = __uint_as_float(xor_lane<D>(__float_as_uint(tot)));
    if (!(l & D)) v = fminf(v, o);
    tot = fminf(tot, o);
}
// running maximum over lanes <= l; running minimum over lanes >= l
LS_DEV float wave_scan_max_f32(float v) {
    const int l = lane_id();
    float tot = v;
    scan_step_max_f32<1>(v, tot, l);
    scan_step_max_f32<2>(v, tot, l);
    scan_step_max_f32<4>(v, tot, l);
    scan_step_max_f32<8>(v, tot, l);
    scan_step_max_f32<16>(v, tot, l);
    scan_step_max_f32<32>(v, tot, l);
    return v;
}
LS_DEV float wave_rscan_min_f32(float v) {
    const int l = lane_id();
    float tot = v;
    rscan_step_min_f32<1>(v, tot, l);
    rscan_step_min_f32<2>(v, tot, l);
    rscan_step_min_f32<4>(v, tot, l);
    rscan_step_min_f32<8>(v, tot, l);
    rscan_step_min_f32<16>(v, tot, l);
    rscan_step_min_f32<32>(v, tot, l);
    return v;
}
LS_DEV uint32_t wave_inclusive_scan(uint32_t v) {
    const int l = lane_id();
    uint32_t tot = v;
    scan_step_u32<1>(v, tot, l);
    scan_step_u32<2>(v, tot, l);
    scan_step_u32<4>(v, tot, l);
    scan_step_u32<8>(v, tot, l);
    scan_step_u32<16>(v, tot, l);
    scan_step_u32<32>(v, tot, l);
    return v;
}

// block exclusive scan of uint32 (NT threads); returns the block total in *total
template <int NT>
LS_DEV uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* scratch /* >= NT/64 + 1 */) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, w = tid >> 6, l = lane_id();
    uint32_t inc = wave_inclusive_scan(v);
    if (l == 63) scratch[w] = inc;
    __syncthreads();
    if (w == 0) {
        uint32_t x = (l < NW) ? scratch[l] : 0u;
        uint32_t xi = wave_inclusive_scan(x);
        if (l < NW) scratch[l] = xi - x;
        if (l == NW - 1) scratch[NW] = xi;
    }
    __syncthreads();
    uint32_t res = scratch[w] + inc - v;
    if (total) *total = scratch[NW];
    __syncthreads();
    return res;
}

// Several workgroup reductions behind one barrier: ND double sums, NU uint64
// sums and NM uint32 maxima.  Wave butterflies first, then every thread adds
// the waves' results in wave order, so all threads get the same totals in a
// fixed order.  Scratch: sd >= ND*NT/64, su >= NU*NT/64, sm >= NM*NT/64; it
// must not be written again before another barrier.
template <int NT, int ND, int NU, int NM>
LS_DEV void block_reduce_multi(double (&d)[ND], unsigned long long (&u)[NU], uint32_t (&m)[NM], double* sd,
                               unsigned long long* su, uint32_t* sm) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
#pragma unroll
    for (int i = 0; i < ND; ++i) d[i] = wave_sum(d[i]);
#pragma unroll
    for (int i = 0; i < NU; ++i) u[i] = wave_sum_u64(u[i]);
#pragma unroll
    for (int i = 0; i < NM; ++i) m[i] = wave_max_u32(m[i]);
    if (l == 0) {
#pragma unroll
        for (int i = 0; i < ND; ++i) sd[i * NW + w] = d[i];
#pragma unroll
        for (int i = 0; i < NU; ++i) su[i * NW + w] = u[i];
#pragma unroll
        for (int i = 0; i < NM; ++i) sm[i * NW + w] = m[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ND; ++i) {
        double a = sd[i * NW];
#pragma unroll
        for (int x = 1; x < NW; ++x) a += sd[i * NW + x];
        d[i] = a;
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        unsigned long long a = su[i * NW];
#pragma unroll
        for (int x = 1; x < NW; ++x) a += su[i * NW + x];
        u[i] = a;
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        uint32_t a = sm[i * NW];
#pragma unroll
        for (int x = 1; x < NW; ++x) a = max(a, sm[i * NW + x]);
        m[i] = a;
    }
}

// block sum of double in a fixed order (wave butterflies, then wave 0); the
// result is valid in wave 0 only (broadcast it through LDS where others need it)
template <int NT>
LS_DEV double block_sum(double v, double* scratch /* >= NT/64 */) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    v = wave_sum(v);
    if (l == 0) scratch[w] = v;
    __syncthreads();
    double r = 0.0;
    if (w == 0) {
        double x = (l < NW) ? scratch[l] : 0.0;
        r = wave_sum(x);
    }
    __syncthreads();
    return r;  // valid in wave 0
}


// ascending bitonic sort of N (a power of two) keys in LDS by NT threads
template <int NT>
LS_DEV void bitonic_sort_lds(uint32_t* a, int N) {
    for (int size = 2; size <= N; size <<= 1) {
        for (int half = size >> 1; half > 0; half >>= 1) {
            for (int t = threadIdx.x; t < (N >> 1); t += NT) {
                const int i = ((t & ~(half - 1)) << 1) | (t & (half - 1));  // half is a power of two
                const int j = i + half;
                const bool up = (i & size) == 0;
                const uint32_t x = a[i], y = a[j];
                if ((x > y) == up) { a[i] = y; a[j] = x; }
            }
            __syncthreads();
        }
    }
}

constexpr int ilog2_c(int v) { return v <= 1 ? 0 : 1 + ilog2_c(v >> 1); }

// Ascending bitonic sort of N = NA * IPT keys (a power of two) held in LDS,
// called by all NT threads of the workgroup; the first NA (whole waves) sort.
// Thread t keeps keys t*IPT .. t*IPT + IPT - 1 in registers: compare-exchanges
// at strides < IPT stay in registers, strides < 64 * IPT go through lane
// exchanges inside the wave (DPP and lane swaps), and only wider strides go
// through LDS (consecutive LDS stages are done between one store and one
// reload).  With NT = 64 one wave sorts alone (no barrier).  The caller
// synchronises before reading the result.
template <int NT, int NA, int IPT>
LS_DEV void bitonic_sort_hybrid(uint32_t* lds) {
    constexpr int N = NA * IPT;
    constexpr int LOGN = ilog2_c(N), LOGI = ilog2_c(IPT), LOGW = ilog2_c(64 * IPT);
    static_assert((1 << LOGN) == N && (1 << LOGI) == IPT, "powers of two");
    static_assert(NA % 64 == 0 && NA <= NT, "whole waves");
    const int tid = threadIdx.x;
    const bool act = tid < NA;  // wave-uniform
    uint32_t x[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) x[q] = act ? lds[tid * IPT + q] : 0u;
    // every loop below has a compile-time trip count and is unrolled, so each
    // stage's lane distance is a constant and picks its exchange statically
#pragma unroll
    for (int ls = 1; ls <= LOGN; ++ls) {
        const int size = 1 << ls;
        int lh = ls - 1;
        if (lh >= LOGW) {
            if (act) {
#pragma unroll
                for (int q = 0; q < IPT; ++q) lds[tid * IPT + q] = x[q];
            }
            __syncthreads();
#pragma unroll
            for (; lh >= LOGW; --lh) {
                const int half = 1 << lh;
                for (int t = tid; t < (N >> 1); t += NT) {
                    const int i = ((t & ~(half - 1)) << 1) | (t & (half - 1));
                    const int j = i + half;
                    const bool up = (i & size) == 0;
                    const uint32_t a = lds[i], b = lds[j];
                    if ((a > b) == up) { lds[i] = b; lds[j] = a; }
                }
                __syncthreads();
            }
            if (act) {
#pragma unroll
                for (int q = 0; q < IPT; ++q) x[q] = lds[tid * IPT + q];
            }
            __syncthreads();
        }
        if (!act) continue;  // idle waves only take part in the barriers
#pragma unroll
        for (; lh >= LOGI; --lh) {
            const int half = 1 << lh;
            const int lx = 1 << (lh - LOGI);  // partner lane distance
#pragma unroll
            for (int q = 0; q < IPT; ++q) {
                const int i = tid * IPT + q;
                const uint32_t y = xor_lane_rt(x[q], lx);
                const bool up = (i & size) == 0;
                const bool lower = (i & half) == 0;
                const uint32_t mn = x[q] < y ? x[q] : y, mx = x[q] < y ? y : x[q];
                x[q] = (lower == up) ? mn : mx;
            }
        }
#pragma unroll
        for (; lh >= 0; --lh) {
            const int half = 1 << lh;
#pragma unroll
            for (int q = 0; q < IPT; ++q) {
                if ((q & half) == 0 && (q | half) < IPT) {
                    const int i = tid * IPT + q;
                    const bool up = (i & size) == 0;
                    const uint32_t a = x[q], b = x[q | half];
                    if ((a > b) == up) { x[q] = b; x[q | half] = a; }
                }
            }
        }
    }
    if (act) {
#pragma unroll
        for (int q = 0; q < IPT; ++q) lds[tid * IPT + q] = x[q];
    }
}

// Ascending sort of the first N keys of lds (N a power of two, N >= 64) by
// all NT threads; ends with a barrier.  Up to 4 NT keys: the hybrid sort on
// min(N, NT) threads (measured on gfx950 with NT = 1024: more threads beat
// more keys per thread, and the hybrid beats the plain LDS sort at every
// size); larger N: the plain LDS bitonic sort.
template <int NT, int NA>
LS_DEV bool sort_pow2_hybrid(uint32_t* lds, int N) {
    if (N == NA) {
        bitonic_sort_hybrid<NT, NA, 1>(lds);
        return true;
    }
    if constexpr (NA < NT) return sort_pow2_hybrid<NT, 2 * NA>(lds, N);
    return false;
}
template <int NT>
LS_DEV void sort_pow2_lds(uint32_t* lds, int N) {
    if (N == 2 * NT) bitonic_sort_hybrid<NT, NT, 2>(lds);
    else if (N == 4 * NT) bitonic_sort_hybrid<NT, NT, 4>(lds);
    else if (!sort_pow2_hybrid<NT, 64>(lds, N)) {
        bitonic_sort_lds<NT>(lds, N);
        return;
    }
    __syncthreads();
}

LS_DEV int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// fp64 sums over the wave, forward or reverse: the butterfly scan of
// wave_inclusive_scan (all 64 lanes active)
template <int D>
LS_DEV void scan_step_f64(double& v, double& tot, int l, bool reverse) {
    const double o = xor_lane_f64<D>(tot);
    if (((l & D) != 0) != reverse) v += o;
    tot += o;  // the partner forms o + tot: the same value
}
LS_DEV double wave_scan_add_incl(double v, bool reverse) {
    const int l = lane_id();
    double tot = v;
    scan_step_f64<1>(v, tot, l, reverse);
    scan_step_f64<2>(v, tot, l, reverse);
    scan_step_f64<4>(v, tot, l, reverse);
    scan_step_f64<8>(v, tot, l, reverse);
    scan_step_f64<16>(v, tot, l, reverse);
    scan_step_f64<32>(v, tot, l, reverse);
    return v;
}
LS_DEV double wave_excl_from_incl(double inc, bool reverse) {
    const int lane = lane_id();
    const double e = reverse ? __shfl_down(inc, 1, 64) : __shfl_up(inc, 1, 64);
    return (reverse ? lane == 63 : lane == 0) ? 0.0 : e;
}
// additive exclusive scan of double over the workgroup.  reverse = false:
// sum over lower thread indices; true: over higher ones.  Butterfly scans inside
// each wave, then the wave totals scanned by wave 0 (s: >= NT/64 entries).
// The exclusive value is read from the neighbour's inclusive sum, never
// formed as (inclusive - own).
template <int NT>
LS_DEV double block_scan_add_excl(double v, double* s, bool reverse) {
    constexpr int NW = NT / 64;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const double inc = wave_scan_add_incl(v, reverse);
    double ex = wave_excl_from_incl(inc, reverse);
    if (NW > 1) {
        if (lane == (reverse ? 0 : 63)) s[w] = inc;
        __syncthreads();
        if (w == 0) {
            const double x = lane < NW ? s[lane] : 0.0;
            const double xe = wave_excl_from_incl(wave_scan_add_incl(x, reverse), reverse);
            if (lane < NW) s[lane] = xe;
        }
        __syncthreads();
        ex = s[w] + ex;
        __syncthreads();
    }
    return ex;
}

// a forward exclusive scan of a and a backward one of b behind the barriers
// of one (the same arithmetic as two block_scan_add_excl calls); s: >= 2 NT/64
template <int NT>
LS_DEV void block_scan_add_excl2(double a, double b, double& ea, double& eb, double* s) {
    constexpr int NW = NT / 64;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const double ia = wave_scan_add_incl(a, false);
    const double ib = wave_scan_add_incl(b, true);
    ea = wave_excl_from_incl(ia, false);
    eb = wave_excl_from_incl(ib, true);
    if (NW > 1) {
        if (lane == 63) s[w] = ia;
        if (lane == 0) s[NW + w] = ib;
        __syncthreads();
        if (w == 0) {
            const double x = lane < NW ? s[lane] : 0.0;
            const double y = lane < NW ? s[NW + lane] : 0.0;
            const double xe = wave_excl_from_incl(wave_scan_add_incl(x, false), false);
            const double ye = wave_excl_from_incl(wave_scan_add_incl(y, true), true);
            if (lane < NW) { s[lane] = xe; s[NW + lane] = ye; }
        }
        __syncthreads();
        ea = s[w] + ea;
        eb = s[NW + w] + eb;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 128-bit fixed-point sums of terms in [0, 1] (62 fractional bits): integer
// addition is associative, so a sum over scores in any order (e.g. the order
// atomics appended them) is bit-reproducible.  Each term is truncated to
// 2^-62 (below fp64 summation error).
// ---------------------------------------------------------------------------
struct Fx128 { unsigned long long lo, hi; };
LS_DEV Fx128 fx_zero() { Fx128 r; r.lo = 0ull; r.hi = 0ull; return r; }
LS_DEV void fx_add_term(Fx128& a, double e) {
    const unsigned long long x = (unsigned long long)(e * 0x1p62);
    const unsigned long long lo = a.lo + x;
    a.hi += (lo < a.lo) ? 1ull : 0ull;
    a.lo = lo;
}
LS_DEV Fx128 fx_add(Fx128 a, Fx128 b) {
    Fx128 r;
    r.lo = a.lo + b.lo;
    r.hi = a.hi + b.hi + ((r.lo < a.lo) ? 1ull : 0ull);
    return r;
}
LS_DEV double fx_to_double(Fx128 a) { return (double)a.hi * 0x1p2 + (double)a.lo * 0x1p-62; }
// a - 1 (the own term of one score), exact
LS_DEV Fx128 fx_minus_one(Fx128 a) {
    Fx128 r;
    r.lo = a.lo - (1ull << 62);
    r.hi = a.hi - ((a.lo < (1ull << 62)) ? 1ull : 0ull);
    return r;
}
template <int NT>
LS_DEV Fx128 block_sum_fx(Fx128 v, unsigned long long* s /* >= 2 * NT/64 */) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    auto step = [&](auto d_tag) {
        constexpr int D = decltype(d_tag)::value;
        Fx128 y;
        y.lo = xor_lane64<D>(v.lo);
        y.hi = xor_lane64<D>(v.hi);
        v = fx_add(v, y);
    };
    step(std::integral_constant<int, 32>());
    step(std::integral_constant<int, 16>());
    step(std::integral_constant<int, 8>());
    step(std::integral_constant<int, 4>());
    step(std::integral_constant<int, 2>());
    step(std::integral_constant<int, 1>());
    if (l == 0) { s[2 * w] = v.lo; s[2 * w + 1] = v.hi; }
    __syncthreads();
    Fx128 r = fx_zero();
    if (w == 0) {
        for (int q = 0; q < NW; ++q) { Fx128 y; y.lo = s[2 * q]; y.hi = s[2 * q + 1]; r = fx_add(r, y); }
    }
    __syncthreads();
    return r;  // valid in wave 0
}

// two fixed-point block sums behind one barrier pair (results valid in wave 0)
template <int NT>
LS_DEV void block_sum_fx2(Fx128& a, Fx128& b, unsigned long long* s /* >= 4 * NT/64 */) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    auto step = [&](auto d_tag) {
        constexpr int D = decltype(d_tag)::value;
        Fx128 y, z;
        y.lo = xor_lane64<D>(a.lo);
        y.hi = xor_lane64<D>(a.hi);
        z.lo = xor_lane64<D>(b.lo);
        z.hi = xor_lane64<D>(b.hi);
        a = fx_add(a, y);
        b = fx_add(b, z);
    };
    step(std::integral_constant<int, 32>());
    step(std::integral_constant<int, 16>());
    step(std::integral_constant<int, 8>());
    step(std::integral_constant<int, 4>());
    step(std::integral_constant<int, 2>());
    step(std::integral_constant<int, 1>());
    if (l == 0) { s[4 * w] = a.lo; s[4 * w + 1] = a.hi; s[4 * w + 2] = b.lo; s[4 * w + 3] = b.hi; }
    __syncthreads();
    Fx128 ra = fx_zero(), rb = fx_zero();
    if (w == 0) {
        for (int q = 0; q < NW; ++q) {
            Fx128 y, z;
            y.lo = s[4 * q]; y.hi = s[4 * q + 1];
            z.lo = s[4 * q + 2]; z.hi = s[4 * q + 3];
            ra = fx_add(ra, y);
            rb = fx_add(rb, z);
        }
    }
    __syncthreads();
    a = ra;
    b = rb;
}

// wave minimum / maximum of a float, returned as its bits (NaN-free inputs)
LS_DEV uint32_t wave_min_f32_bits(float x) {
    uint32_t v = __float_as_uint(x);
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(xor_lane<32>(v))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(xor_lane<16>(v))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(xor_lane<8>(v))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(xor_lane<4>(v))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(xor_lane<2>(v))));
    v = __float_as_uint(fminf(__uint_as_float(v), __uint_as_float(xor_lane<1>(v))));
    return v;
}
LS_DEV uint32_t wave_max_f32_bits(float x) {
    uint32_t v = __float_as_uint(x);
    v = __float_as_uint(fmaxf(__uint_as_float(v), __uint_as_float(xor_lane<32>(v))));
    v = __float_as_uint(fmaxf(__uint_as_float(v), __uint_as_float(xor_lane<16>(v))));
    v = __float_as_uint(fmaxf(__uint_as_float(v), __uint_as_float(xor_lane<8>(v))));
    v = __float_as_uint(fmaxf(__uint_as_float(v), __uint_as_float(xor_lane<4>(v))));
    v = __float_as_uint(fmaxf(__uint_as_float(v), __uint_as_float(xor_lane<2>(v))));
    v = __float_as_uint(fmaxf(__uint_as_float(v), __uint_as_float(xor_lane<1>(v))));
    return v;
}

LS_DEV uint32_t wave_min_u32(uint32_t v) {
    v = min(v, xor_lane<32>(v));
    v = min(v, xor_lane<16>(v));
    v = min(v, xor_lane<8>(v));
    v = min(v, xor_lane<4>(v));
    v = min(v, xor_lane<2>(v));
    v = min(v, xor_lane<1>(v));
    return v;
}

// wave minimum of a non-negative double (+inf allowed): the bit patterns of
// non-negative doubles order like the values (all 64 lanes active)
LS_DEV double wave_min_nonneg_f64(double x) {
    unsigned long long v = (unsigned long long)__double_as_longlong(x);
    auto step = [&](unsigned long long o) { v = o < v ? o : v; };
    step(xor_lane64<32>(v));
    step(xor_lane64<16>(v));
    step(xor_lane64<8>(v));
    step(xor_lane64<4>(v));
    step(xor_lane64<2>(v));
    step(xor_lane64<1>(v));
    return __longlong_as_double((long long)v);
}

// minimum of a non-negative double over the workgroup, in every thread
// (s: >= NT/64 doubles; every thread calls it)
template <int NT>
LS_DEV double block_min_nonneg_f64(double x, double* s) {
    constexpr int NW = NT / 64;
    const double wm = wave_min_nonneg_f64(x);
    if (lane_id() == 0) s[threadIdx.x >> 6] = wm;
    __syncthreads();
    double r = s[0];
#pragma unroll
    for (int q = 1; q < NW; ++q) r = fmin(r, s[q]);
    __syncthreads();
    return r;
}


}  // namespace lapsum
