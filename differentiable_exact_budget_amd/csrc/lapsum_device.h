// Device-side definitions shared by the HIP kernels of the Fast LapSum solver
// (gfx950, wave64).  Host code includes it for the control-block layout only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kCurveThreads = 256;
constexpr int kCurveTile = kRadixTile;   // sorted keys per curve segment
constexpr int kSampleMax = 40960;        // sample size cap (select holds it in registers)
constexpr int kSelectThreads = 1024;
constexpr int kSelectItems = kSampleMax / kSelectThreads;  // 40
constexpr int kCandMax = 2048;           // sample values kept for the splitters

// control-block flags
constexpr int kFlagNonFinite = 1;
constexpr int kFlagOverflow = 2;
constexpr int kFlagInternal = 4;
constexpr int kFlagBigRoot = 8;   // the root lies in a bucket too large for LDS (host sorts it)
constexpr int kFlagCertified = 16;  // G(a_L) >= k > G(a_R) from the filter's sums
constexpr uint32_t kNotHeavy = 0xFFFFFFFFu;  // bucket slot offset marker: not an overflowed bucket

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
    // last-workgroup tickets (each returns to 0 after use) and tile counters
    unsigned int done[8];
    unsigned int tile_ctr[4];
    unsigned int pad1[4];
    // 1 when the filter certified the bracket with every band score stored:
    // the band solve and p pass launched right behind it then do their work
    int32_t gate;
    int32_t pad2;
};

// host-pinned summary written by the filter's last workgroup; the host polls seq
struct HostSummary {
    unsigned long long c_L, m, c_R;
    double S_L, S_R, B_L, B_R;
    double g_aL, g_aR;  // G at the bracket ends (the certification quantities)
    float aL, aR;
    int32_t flags;
    int32_t nb;
    unsigned long long max_bucket;
    volatile unsigned int seq;
    unsigned int pad;
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

// fixed-order butterfly sums over the wave
LS_DEV double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
LS_DEV unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// inclusive scan of uint32 over the wave (Hillis-Steele with shuffles)
LS_DEV uint32_t wave_inclusive_scan(uint32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(v, o, 64);
        if (l >= o) v += y;
    }
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
    for (int i = 0; i < NM; ++i) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m[i] = max(m[i], (uint32_t)__shfl_xor((int)m[i], o, 64));
    }
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

template <int NT>
LS_DEV unsigned long long block_sum_u64(unsigned long long v, unsigned long long* scratch) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    v = wave_sum_u64(v);
    if (l == 0) scratch[w] = v;
    __syncthreads();
    unsigned long long r = 0;
    if (w == 0) {
        unsigned long long x = (l < NW) ? scratch[l] : 0ull;
        r = wave_sum_u64(x);
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

// Ascending bitonic sort of N = NT * IPT keys (a power of two) held in LDS.
// Thread t keeps keys t*IPT .. t*IPT + IPT - 1 in registers: compare-exchanges
// at strides < IPT stay in registers, strides < 64 * IPT go through wave
// shuffles, and only wider strides go through LDS (consecutive LDS stages
// are done between one store and one reload).  With NT = 64 one wave sorts
// alone (no barrier).  The caller synchronises before reading the result.
template <int NT, int IPT>
LS_DEV void bitonic_sort_hybrid(uint32_t* lds) {
    constexpr int N = NT * IPT;
    const int tid = threadIdx.x;
    uint32_t x[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) x[q] = lds[tid * IPT + q];
    for (int size = 2; size <= N; size <<= 1) {
        int half = size >> 1;
        if (half >= 64 * IPT) {
#pragma unroll
            for (int q = 0; q < IPT; ++q) lds[tid * IPT + q] = x[q];
            __syncthreads();
            for (; half >= 64 * IPT; half >>= 1) {
                for (int t = tid; t < (N >> 1); t += NT) {
                    const int i = ((t & ~(half - 1)) << 1) | (t & (half - 1));
                    const int j = i + half;
                    const bool up = (i & size) == 0;
                    const uint32_t a = lds[i], b = lds[j];
                    if ((a > b) == up) { lds[i] = b; lds[j] = a; }
                }
                __syncthreads();
            }
#pragma unroll
            for (int q = 0; q < IPT; ++q) x[q] = lds[tid * IPT + q];
            __syncthreads();
        }
        for (; half >= IPT; half >>= 1) {
            const int lx = half / IPT;  // partner lane distance
#pragma unroll
            for (int q = 0; q < IPT; ++q) {
                const int i = tid * IPT + q;
                const uint32_t y = (uint32_t)__shfl_xor((int)x[q], lx, 64);
                const bool up = (i & size) == 0;
                const bool lower = (i & half) == 0;
                const uint32_t mn = x[q] < y ? x[q] : y, mx = x[q] < y ? y : x[q];
                x[q] = (lower == up) ? mn : mx;
            }
        }
        for (; half >= 1; half >>= 1) {
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
#pragma unroll
    for (int q = 0; q < IPT; ++q) lds[tid * IPT + q] = x[q];
}

// Ascending sort of the first N keys of lds (N a power of two, N >= 64) by
// all NT threads; ends with a barrier.  The choice follows measurements on
// gfx950 with NT = 1024: the hybrid sort wins for NT <= N <= 4 NT, the plain
// LDS bitonic sort below that (one wave alone is slower: its shuffle stages
// run back to back) and above it (the hybrid's register blocks then
// conflict in LDS).
template <int NT>
LS_DEV void sort_pow2_lds(uint32_t* lds, int N) {
    if (N == NT) { bitonic_sort_hybrid<NT, 1>(lds); __syncthreads(); }
    else if (N == 2 * NT) { bitonic_sort_hybrid<NT, 2>(lds); __syncthreads(); }
    else if (N == 4 * NT) { bitonic_sort_hybrid<NT, 4>(lds); __syncthreads(); }
    else bitonic_sort_lds<NT>(lds, N);
}

LS_DEV int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// additive exclusive scan of double over the workgroup.  reverse = false:
// sum over lower thread indices; true: over higher ones.  Shuffles inside
// each wave, then the wave totals scanned by wave 0 (s: >= NT/64 entries).
// The exclusive value is read from the neighbour's inclusive sum, never
// formed as (inclusive - own).
LS_DEV double wave_scan_add_incl(double v, bool reverse) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = reverse ? __shfl_down(v, o, 64) : __shfl_up(v, o, 64);
        if (reverse ? (lane + o < 64) : (lane >= o)) v += y;
    }
    return v;
}
LS_DEV double wave_excl_from_incl(double inc, bool reverse) {
    const int lane = lane_id();
    const double e = reverse ? __shfl_down(inc, 1, 64) : __shfl_up(inc, 1, 64);
    return (reverse ? lane == 63 : lane == 0) ? 0.0 : e;
}
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
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Fx128 y;
        y.lo = __shfl_xor(v.lo, o, 64);
        y.hi = __shfl_xor(v.hi, o, 64);
        v = fx_add(v, y);
    }
    if (l == 0) { s[2 * w] = v.lo; s[2 * w + 1] = v.hi; }
    __syncthreads();
    Fx128 r = fx_zero();
    if (w == 0) {
        for (int q = 0; q < NW; ++q) { Fx128 y; y.lo = s[2 * q]; y.hi = s[2 * q + 1]; r = fx_add(r, y); }
    }
    __syncthreads();
    return r;  // valid in wave 0
}

// device-scope ticket for the last-workgroup pattern: release this
// workgroup's global writes, take a ticket, and tell every thread whether it
// is in the last workgroup to finish (which then sees all earlier writes).
LS_DEV bool last_block_ticket(unsigned int* counter, int* s_flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        unsigned int prev = atomicAdd(counter, 1u);
        *s_flag = (prev == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    bool last = *s_flag != 0;
    if (last) __threadfence();
    return last;
}

}  // namespace lapsum
