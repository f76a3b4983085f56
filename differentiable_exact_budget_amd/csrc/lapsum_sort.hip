// Sorting and threshold-solve kernels of the Fast LapSum solver (gfx950).
//
// Full-sort solver (Fast LapSum paper, gist.science section 2.2): sort all
// scores, build the threshold curve with one stable prefix/suffix scan,
// search the interval where the budget balances and take the closed-form
// root there.  Band solve (same section, bracketing step 3): the same on the
// middle band only, with the out-of-band scores entering as tail sums.
//
// Kernels
//   k_small_solve   n <= 16384: one workgroup sorts in LDS and solves.
//   k_bucket_agg    one workgroup per band bucket: count, min, max and the
//                   two order-free exp-sums of its (unsorted) scores.
//   k_band_root     one workgroup: the curve across buckets, the root bucket
//                   sorted in LDS, the root.
//   k_radix_hist    all four 8-bit digit histograms in one read; the last
//                   workgroup turns them into the passes' digit offsets.
//   k_radix_pass    one LSD digit pass in one kernel (up to 512 tiles).
//   k_radix_count / k_radix_scan / k_radix_scatter  the same pass in three
//                   kernels (more tiles).
//   k_curve_tiles   per-tile curve aggregates of the sorted scores.
//   k_curve_root    one workgroup: the curve across the tiles, the root
//                   tile's per-score curve, the root.
#include "lapsum_blocksolve.h"
#include "lapsum_launch.h"
#include <algorithm>
#include <atomic>

namespace lapsum {

// ---------------------------------------------------------------------------
// n <= 16384: everything in one workgroup
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void k_small_solve(const float* __restrict__ r, int n, double k,
                                                               double t, double inv_t, Ctl* ctl, SolveScratch sc,
                                                               double* b_out, uint32_t* keys_out) {
    __shared__ uint32_t keys[kSmallMax];
    __shared__ uint32_t cnt[256 * (kSortThreads / 64)];
    __shared__ uint32_t scr[32];
    __shared__ float s_k[kSortThreads];
    __shared__ double s_v[kSortThreads];
    __shared__ int s_int[32];
    __shared__ uint32_t sg_cnt, sg_off;
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    // up to 4 keys per thread the bitonic sort (padded with the largest key,
    // which sorts to the end) is the faster of the two LDS sorts
    const int np = n <= 4 * kSortThreads ? max(next_pow2(n), 64) : n;
    for (int i = tid; i < np; i += kSortThreads) {
        if (i < n) {
            const float v = r[i];
            bad |= !finite_f(v);
            keys[i] = f2key(v);
        } else {
            keys[i] = 0xFFFFFFFFu;
        }
    }
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    if (n <= 4 * kSortThreads) sort_pow2_lds<kSortThreads>(keys, np);
    else block_sort_lds<kSortThreads, kSortItems>(keys, n, cnt, scr);
    if (keys_out)
        for (int i = tid; i < n; i += kSortThreads) keys_out[i] = keys[i];
    if (tid == 0) { sg_cnt = (uint32_t)n; sg_off = 0u; }
    __syncthreads();
    // the whole sorted array as one segment, no aggregates: the solve tests G
    // at every score
    SegView sv{1, nullptr, nullptr, nullptr, nullptr, &sg_cnt, &sg_off, keys, nullptr};
    Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t, -INFINITY, INFINITY};
    SolveOut o = segment_solve<kSortThreads, kSortItems>(sv, tl, sc, s_k, s_v, s_int);
    if (tid == 0) {
        double b = o.b;
        int flags = 0;
        if (s_bad) { b = __longlong_as_double(0x7ff8000000000000ll); flags = kFlagNonFinite; }
        else if (!o.ok) flags = kFlagInternal;
        ctl->flags = flags;
        ctl->b = b;
        ctl->jstar = o.jstar;
        if (b_out) *b_out = b;
    }
}

// ---------------------------------------------------------------------------
// band buckets: the buckets are value-ordered (every score of bucket i is <=
// every score of bucket i+1), so the curve across buckets only needs, per
// bucket, its count, minimum, maximum and the two sums
//   P = sum e^{(v - max)/t},  Bx = sum e^{(min - v)/t} - 1,
// which do not depend on the order of the scores inside it.  k_bucket_agg
// forms them (fixed-point sums: bit-reproducible whatever order the filter
// appended the scores in); k_band_root finds the bucket holding the root,
// sorts only that one and solves.
// ---------------------------------------------------------------------------
constexpr int kAggThreads = 256;

// hoff (may be null): per bucket, kNotHeavy, or the element offset from
// bucket_vals of the slot holding all of an overflowed bucket's scores
__global__ __launch_bounds__(kAggThreads) void k_bucket_agg(const uint32_t* __restrict__ bucket_vals,
                                                             const uint32_t* bucket_cnt, int cap, SegArrays seg,
                                                             double inv_t, HeavyArrays ha, int heavy,
                                                             const int* gate) {
    constexpr int NW = kAggThreads / 64;
    constexpr int R = 4;  // scores a thread keeps in registers; a larger bucket is read twice
    __shared__ uint32_t s_mm[2 * NW];
    __shared__ unsigned long long s_fx[4 * NW];
    if (gate && *gate == 0) return;  // launched ahead of a certification that failed
    const int tid = threadIdx.x, w = tid >> 6;
    const int bkt = blockIdx.x;
    const uint32_t ho = heavy ? ha.hoff[bkt] : kNotHeavy;
    const int c = ho != kNotHeavy ? (int)bucket_cnt[bkt] : (int)min(bucket_cnt[bkt], (uint32_t)cap);
    const size_t off = ho != kNotHeavy ? (size_t)ho : (size_t)bkt * (size_t)cap;
    if (tid == 0) { seg.cnt[bkt] = (uint32_t)c; seg.off[bkt] = (uint32_t)off; }
    if (c == 0) return;
    if (ho != kNotHeavy) {
        // an overflowed bucket: its range from the collect pass, its sums from
        // the chunk partials (integer sums, any order)
        const uint32_t j0 = ha.hch0[bkt];
        const uint32_t nj = ((uint32_t)c + kHeavyChunk - 1) / kHeavyChunk;
        Fx128 P = fx_zero(), Q = fx_zero();
        for (uint32_t j = (uint32_t)tid; j < nj; j += kAggThreads) {
            const unsigned long long* h = ha.hpart + 4ull * (j0 + j);
            Fx128 y, z;
            y.lo = h[0]; y.hi = h[1]; z.lo = h[2]; z.hi = h[3];
            P = fx_add(P, y);
            Q = fx_add(Q, z);
        }
        block_sum_fx2<kAggThreads>(P, Q, s_fx);
        if (tid == 0) {
            seg.first[bkt] = key2f(ha.hmin[bkt]);
            seg.last[bkt] = key2f(ha.hmax[bkt]);
            seg.P[bkt] = fx_to_double(P);
            seg.Bx[bkt] = fx_to_double(fx_minus_one(Q));
        }
        return;
    }
    const uint32_t* vals = bucket_vals + off;
    uint32_t kk[R];
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int i = tid + q * kAggThreads;
        kk[q] = i < c ? f2key(__uint_as_float(vals[i])) : 0u;
        if (i < c) { kmn = min(kmn, kk[q]); kmx = max(kmx, kk[q]); }
    }
    for (int i = tid + R * kAggThreads; i < c; i += kAggThreads) {
        const uint32_t k = f2key(__uint_as_float(vals[i]));
        kmn = min(kmn, k);
        kmx = max(kmx, k);
    }
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane_id() == 0) { s_mm[w] = kmn; s_mm[NW + w] = kmx; }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NW; ++x) { kmn = min(kmn, s_mm[x]); kmx = max(kmx, s_mm[NW + x]); }
    const double vmin = (double)key2f(kmn), vmax = (double)key2f(kmx);
    Fx128 P = fx_zero(), Q = fx_zero();
    auto add = [&](uint32_t k) {
        const double v = (double)key2f(k);
        fx_add_term(P, exp((v - vmax) * inv_t));
        fx_add_term(Q, exp((vmin - v) * inv_t));
    };
#pragma unroll
    for (int q = 0; q < R; ++q)
        if (tid + q * kAggThreads < c) add(kk[q]);
    for (int i = tid + R * kAggThreads; i < c; i += kAggThreads) add(f2key(__uint_as_float(vals[i])));
    block_sum_fx2<kAggThreads>(P, Q, s_fx);
    if (tid == 0) {
        seg.first[bkt] = (float)vmin;
        seg.last[bkt] = (float)vmax;
        seg.P[bkt] = fx_to_double(P);
        seg.Bx[bkt] = fx_to_double(fx_minus_one(Q));
    }
}

__global__ __launch_bounds__(kSortThreads) void k_band_root(const uint32_t* bucket_vals, int nb, Ctl* ctl,
                                                             SegArrays seg, SolveScratch sc, double k, double t,
                                                             double inv_t, double* b_out, const int* gate,
                                                             HostSummary* hs, unsigned int seq) {
    if (gate && *gate == 0) return;  // launched ahead of a certification that failed
    __shared__ uint32_t sortbuf[kBucketCapMax];
    __shared__ float s_k[kSortThreads];
    __shared__ double s_v[kSortThreads];
    __shared__ int s_int[32];
    SegView sv{nb, seg.first, seg.last, seg.P, seg.Bx, seg.cnt, seg.off, bucket_vals, sortbuf};
    Tails tl{ctl->aL, ctl->aR, ctl->S_L, ctl->S_R, (double)ctl->m, (double)ctl->c_R, k, t, inv_t, ctl->aL, ctl->aR};
    SolveOut o = segment_solve<kSortThreads, kSortItems>(sv, tl, sc, s_k, s_v, s_int);
    if (threadIdx.x == 0) {
        if (o.big) {
            // hand the root bucket over to a multi-workgroup sort: everything
            // below it becomes the lower tail (its carry), everything above it
            // the upper tail, and the bucket itself the scores to solve over
            const int s = (int)o.jstar;
            const unsigned long long cnt = seg.cnt[s], rank = sc.rank[s];
            ctl->c_R = ctl->c_R + (ctl->m - rank - cnt);
            ctl->m = cnt;
            ctl->aL = sc.pk[s]; ctl->S_L = sc.pv[s];
            ctl->aR = sc.bk[s]; ctl->S_R = sc.bv[s];
            ctl->jstar = s;
            ctl->root_off = seg.off[s];
            atomicOr(&ctl->flags, kFlagBigRoot);
        } else {
            if (!o.ok) atomicOr(&ctl->flags, kFlagInternal);
            ctl->b = o.b;
            ctl->jstar = o.jstar;
            if (b_out) *b_out = o.b;
        }
        if (hs) {  // the host waits for this one (a root bucket too large for LDS is its job)
            hs->root_off = ctl->root_off;
            hs->root_m = ctl->m;
            hs->root_flags = ctl->flags;
            __threadfence_system();
            hs->root_seq = seq;
            __threadfence_system();
        }
    }
}

// ---------------------------------------------------------------------------
// multi-workgroup LSD radix sort: one histogram pass, then one pass per
// 8-bit digit (after Adinets & Merrill, "Onesweep", 2022; the look-back form
// follows Merrill & Garland, "Single-pass parallel prefix scan with
// decoupled look-back", 2016)
// ---------------------------------------------------------------------------
// Digit histograms of all four LSD passes in one read.  Per workgroup in LDS,
// one atomic add per key and digit into one of four copies picked by the
// lane, so that a digit shared by a whole wave (skewed or equal scores)
// costs a 16-way conflict, not 64-way (measured on gfx950 at 10^6 keys:
// 8.8 us for N(0,1) scores, 11.5 us for equal ones; grouping equal digits
// with ballots first, or a one-digit-wave test, costs more).  The workgroup
// totals then go into the global totals with integer atomics (order-free:
// deterministic), into one of kHistGlobalCopies copies picked by the
// workgroup, so that each global word takes a few dozen adds rather than one
// from every workgroup (the adds are done at device scope, one after another
// per word).
// The last workgroup to finish sums the copies, turns the totals into the
// four passes' exclusive digit offsets (goff), sets the control flags for the
// sort and re-zeroes the copies and its ticket.
// hist: global uint32[kHistGlobalCopies * 1024 + 1] (per copy four 256-bin
// histograms; then a non-finite flag), all zero on entry and on exit.
constexpr int kHistCopies = 4;  // LDS histogram copies, by lane & 3
constexpr int kHistLoads = 4;   // quads a histogram thread has in flight

// the device's resident-pass lock: 0 when free, else the holder's token
static __device__ unsigned int g_resident_owner;

__global__ __launch_bounds__(kRadixThreads) void k_radix_hist(const float* __restrict__ r, long long n,
                                                               uint32_t* __restrict__ hist, uint32_t* goff,
                                                               Ctl* ctl, int want_resident, unsigned int token) {
    __shared__ uint32_t h[kHistCopies * 1024];
    __shared__ uint32_t scr[kRadixThreads / 64 + 2];
    __shared__ int s_bad, s_last;
    const int tid = threadIdx.x, lane = lane_id();
    for (int i = tid; i < kHistCopies * 1024; i += kRadixThreads) h[i] = 0u;
    uint32_t* hl = h + (lane & (kHistCopies - 1)) * 1024;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    // whole-wave call: valid marks the lanes that hold a key
    auto add = [&](float v, bool valid) {
        bad |= valid && !finite_f(v);
        const uint32_t key = f2key(v);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            if (valid) atomicAdd(&hl[p * 256 + ((key >> (8 * p)) & 0xFFu)], 1u);
    };
    const long long stride = (long long)gridDim.x * kRadixThreads;
    if ((reinterpret_cast<uintptr_t>(r) & 15u) == 0u) {
        const long long n4 = n >> 2;
        const float4* r4 = reinterpret_cast<const float4*>(r);
        // kHistLoads quads per thread requested at once, then counted
        for (long long base = (long long)blockIdx.x * (kRadixThreads * kHistLoads); base < n4;
             base += stride * kHistLoads) {
            float4 v[kHistLoads];
#pragma unroll
            for (int u = 0; u < kHistLoads; ++u) {
                const long long i = base + u * kRadixThreads + tid;
                v[u] = i < n4 ? r4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < kHistLoads; ++u) {
                const bool valid = base + u * kRadixThreads + tid < n4;
                add(v[u].x, valid); add(v[u].y, valid); add(v[u].z, valid); add(v[u].w, valid);
            }
        }
        if (blockIdx.x == 0 && tid < 64) {  // the last n % 4 keys, one wave
            const long long j = (n4 << 2) + tid;
            const bool valid = tid < 4 && j < n;
            add(valid ? r[j] : 0.0f, valid);
        }
    } else {
        for (long long base = (long long)blockIdx.x * kRadixThreads; base < n; base += stride) {
            const long long i = base + tid;
            const bool valid = i < n;
            add(valid ? r[i] : 0.0f, valid);
        }
    }
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    // the adds return their old values and the wave waits for them, so that
    // every add is done (device scope) before the ticket is taken; a fence
    // here would also write back and invalidate the L2 in every workgroup
    constexpr int NB = 1024 / kRadixThreads;
    uint32_t old[NB + 1];
#pragma unroll
    for (int b = 0; b < NB; ++b) {  // all adds in flight, then one wait
        const int i = tid + b * kRadixThreads;
        uint32_t c = 0u;
#pragma unroll
        for (int q = 0; q < kHistCopies; ++q) c += h[q * 1024 + i];
        old[b] = c ? atomicAdd(&hist[(blockIdx.x % kHistGlobalCopies) * 1024 + i], c) : 0u;
    }
    old[NB] = (tid == 0 && s_bad) ? atomicOr(&hist[kHistGlobalCopies * 1024], 1u) : 0u;
    uint32_t acc = 0u;
#pragma unroll
    for (int b = 0; b <= NB; ++b) acc |= old[b];
    asm volatile("" ::"v"(acc));
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&ctl->done[0], 1u) == gridDim.x - 1u;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    uint32_t y[kHistGlobalCopies][4];  // every load in flight, then the sums
#pragma unroll
    for (int q = 0; q < kHistGlobalCopies; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            y[q][p] = __hip_atomic_load(&hist[q * 1024 + p * 256 + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t any_bad =
        __hip_atomic_load(&hist[kHistGlobalCopies * 1024], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t x[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < kHistGlobalCopies; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            x[p] += y[q][p];
            hist[q * 1024 + p * 256 + tid] = 0u;
        }
#pragma unroll
    for (int p = 0; p < 4; ++p)
        goff[p * 256 + tid] = block_exclusive_scan<kRadixThreads>(x[p], nullptr, scr);  // thread = digit
    if (tid == 0) {
        hist[kHistGlobalCopies * 1024] = 0u;
        ctl->done[0] = 0u;
        ctl->flags = any_bad ? kFlagNonFinite : 0;
        // the one-kernel passes: resident when the lock is free (the sort's
        // last pass frees it), else look-back
        for (int p = 0; p < 4; ++p) ctl->tile_ctr[p] = 0u;
        ctl->resident = want_resident && atomicCAS(&g_resident_owner, 0u, token) == 0u ? 1 : 0;
    }
}

// a published word: the pass's epoch, a kind, a 32-bit value
LS_DEV unsigned long long st_pack(uint32_t epoch, unsigned long long flag, uint32_t v) {
    return ((unsigned long long)epoch << 34) | (flag << 32) | (unsigned long long)v;
}

// One LSD pass in one kernel, 1024 threads per 4096-key tile (four rows of
// 64 keys per wave, so that a wave's chain of rank-counter updates is four
// long).  Two designs; the histogram kernel picks one per sort.
//
// Resident (when the sort holds the device's resident-pass lock; every tile
// of the pass is then on the device at once, T <= one workgroup per CU):
//   1. each tile counts its digits (LDS atomics) and publishes the 256 counts
//      as soon as its keys are in;
//   2. digit d's scan over the tiles runs in one wave of tile d mod T (wave
//      d div T), so that the column reads, one line per word, spread over
//      the CUs; it publishes every tile's global offset for d;
//   3. meanwhile each tile ranks its keys stably (per wave and digit, in row
//      order) and scatters them into LDS in digit order; it then takes its
//      256 offsets and writes runs out.
// Every published word carries the pass's epoch, so a reader waits on the
// word itself: no grid barrier, and each word is read about once.  Each
// array is laid out so that its writer writes whole lines (partial-line
// writes of coherent words stall): counts tile-major, written by the tile;
// offsets digit-major, written by the digit's wave.  A tile waits on every
// other tile, so all of them must be resident: two such sorts at once could
// each hold part of the CUs, hence the lock (a sort that finds it taken uses
// the look-back), and a bounded wait as the last guard.
//
// Look-back (decoupled look-back): tiles take numbers in arrival order and
// a tile adds up its predecessors' published counts until it meets an
// inclusive prefix; a tile waits only on tiles that started before it.
//
// Measured on gfx950 at 10^6 keys: 11.5 us a pass resident, 20 us look-back
// (all tiles run at once there, so the look-back chain and its polling of
// status words that cross the XCDs' L2 caches set the time).
constexpr int kPassThreads = 1024;
constexpr int kPassItems = 4;
constexpr int kPassTile = kPassThreads * kPassItems;
static_assert(kHistCopies * 256 == kPassThreads, "one histogram word per thread");
constexpr unsigned long long kStCount = 1ull, kStBase = 2ull;  // resident: count / offset words
constexpr unsigned long long kStAgg = 1ull, kStInc = 2ull;     // look-back: aggregate / inclusive prefix
constexpr long long kOnesweepMaxTiles = 512;  // up to ~2M keys: one kernel per pass
constexpr int kLookWindow = 8;  // look-back: predecessors' status words read per round trip


struct PassLds {
    uint32_t* cnt;    // 256 * 16: per-wave digit counters
    uint32_t* stage;  // kPassTile: the tile in digit order
    uint32_t* hist;   // kHistCopies * 256
    uint32_t* loc;    // 256
    uint32_t* gbase;  // 256
    uint32_t* scr;    // 18
};

// waits for the word at p to carry this pass's epoch (bounded: a broken
// invariant becomes a reported error, not a hang)
LS_DEV uint32_t wait_word(const unsigned long long* p, uint32_t epoch, Ctl* ctl) {
    unsigned int spins = 0u;
    while (true) {
        const unsigned long long x =
            __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(x >> 34) == epoch) return (uint32_t)x;
        if (++spins > (1u << 24)) { atomicOr(&ctl->flags, kFlagInternal); return 0u; }
        __builtin_amdgcn_s_sleep(1);
    }
}

LS_DEV void pass_resident(const uint32_t* __restrict__ in, int in_is_float, uint32_t* __restrict__ out, long long n,
                          int pass, unsigned long long* status, uint32_t epoch, const uint32_t* goff, Ctl* ctl,
                          const PassLds& sm) {
    constexpr int NW = kPassThreads / 64;
    uint32_t* cnt = sm.cnt;
    uint32_t* stage = sm.stage;
    uint32_t* hist = sm.hist;
    uint32_t* loc = sm.loc;
    uint32_t* gbase = sm.gbase;
    uint32_t* scr = sm.scr;
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const int shift = 8 * pass;
    const uint32_t T = gridDim.x;
    const uint32_t tile = blockIdx.x;
    unsigned long long* cnt_words = status;                      // [tile][digit]
    unsigned long long* base_words = status + (size_t)256 * T;   // [digit][tile]
    const long long base = (long long)tile * kPassTile;
    uint32_t kr[kPassItems];
    // a whole tile: one 16-byte load per thread, turned into the ranking's
    // rows (wave w, row i: keys (w * kPassItems + i) * 64 + lane) through the
    // stage buffer, which is written again only after the ranking's barrier
    static_assert(kPassItems == 4, "one 16-byte load per thread");
    const bool whole = base + kPassTile <= n && (reinterpret_cast<uintptr_t>(in) & 15u) == 0u;
    if (whole) {
        reinterpret_cast<uint4*>(stage)[tid] = reinterpret_cast<const uint4*>(in + base)[tid];
    } else {
#pragma unroll
        for (int i = 0; i < kPassItems; ++i) {
            const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
            uint32_t key = 0u;
            if (idx < n) key = in_is_float ? f2key(__uint_as_float(in[idx])) : in[idx];
            kr[i] = key;
        }
    }
    for (int e = tid; e < 256 * NW; e += kPassThreads) cnt[e] = 0u;
    hist[tid] = 0u;  // kHistCopies * 256 == kPassThreads
    __syncthreads();
    if (whole) {
#pragma unroll
        for (int i = 0; i < kPassItems; ++i) {
            const uint32_t raw = stage[(w * kPassItems + i) * 64 + lane];
            kr[i] = in_is_float ? f2key(__uint_as_float(raw)) : raw;
        }
    }
    // 1. the tile's digit counts, published as soon as the keys are in: one
    // LDS atomic add per key into the copy of its lane group (as in
    // k_radix_hist); the stable ranking below runs while the counts travel
#pragma unroll
    for (int i = 0; i < kPassItems; ++i) {
        const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
        if (idx < n) atomicAdd(&hist[(lane & (kHistCopies - 1)) * 256 + ((kr[i] >> shift) & 0xFFu)], 1u);
    }
    __syncthreads();
    uint32_t dinc = 0u;
    if (tid < 256) {  // waves 0-3, thread = digit
        uint32_t tot = 0u;
#pragma unroll
        for (int q = 0; q < kHistCopies; ++q) tot += hist[q * 256 + tid];
        __hip_atomic_store(cnt_words + (size_t)tile * 256 + tid, st_pack(epoch, kStCount, tot), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        dinc = wave_inclusive_scan(tot);
        if (lane == 63) scr[w] = dinc;
        dinc -= tot;
    }
    // 2. wave w of tile g scans the digits g + T w (+ 16 T ...): every count
    // word of the digit is requested at once (lane l holds the tiles l,
    // l + 64, ...; T <= kOnesweepMaxTiles), the scan runs in registers, then
    // every offset word is written (a load waits for the stores issued
    // before it, so no store goes out before the last load)
    for (int d = (int)tile + (int)T * w; d < 256; d += (int)(T * NW)) {
        constexpr int R = (int)((kOnesweepMaxTiles + 63) / 64);
        unsigned long long x[R];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const uint32_t i = (uint32_t)(m * 64 + lane);
            x[m] = i < T ? __hip_atomic_load(cnt_words + (size_t)i * 256 + d, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : 0ull;
        }
        uint32_t v[R];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const uint32_t i = (uint32_t)(m * 64 + lane);
            v[m] = 0u;
            if (i < T) v[m] = (uint32_t)(x[m] >> 34) == epoch ? (uint32_t)x[m]
                                                              : wait_word(cnt_words + (size_t)i * 256 + d, epoch, ctl);
        }
        uint32_t carry = goff[pass * 256 + d];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            if (m * 64 < (int)T) {  // wave-uniform
                const uint32_t inc = wave_inclusive_scan(v[m]);
                const uint32_t ex = carry + inc - v[m];
                carry += __shfl(inc, 63, 64);
                v[m] = ex;
            }
        }
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const uint32_t i = (uint32_t)(m * 64 + lane);
            if (i < T)
                __hip_atomic_store(base_words + (size_t)d * T + i, st_pack(epoch, kStBase, v[m]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // stable ranks: per wave and digit, in row order
    uint32_t rk[kPassItems];
    volatile uint32_t* vc = cnt;
#pragma unroll
    for (int i = 0; i < kPassItems; ++i) {
        const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
        const bool valid = idx < n;
        const unsigned long long act = ballot(valid);
        rk[i] = 0u;
        if (act != 0ull) {
            const uint32_t d = (kr[i] >> shift) & 0xFFu;
            const unsigned long long peers = match_digit8(d, act);
            const uint32_t b0 = vc[d * NW + w];
            rk[i] = b0 + (uint32_t)mbcnt(peers);
            if (valid && lane == 63 - __clzll(peers)) vc[d * NW + w] = b0 + (uint32_t)popc64(peers);
        }
    }
    __syncthreads();
    // per-wave exclusive offsets of each digit, and its offset in the tile
    if (tid < 256) {
        uint32_t c[NW];  // all reads first: one LDS round trip, not NW
#pragma unroll
        for (int q = 0; q < NW; ++q) c[q] = cnt[tid * NW + q];
        uint32_t tot = 0u;
#pragma unroll
        for (int q = 0; q < NW; ++q) { cnt[tid * NW + q] = tot; tot += c[q]; }
        for (int x = 0; x < w; ++x) dinc += scr[x];
        loc[tid] = dinc;
    }
    __syncthreads();
    // local scatter into LDS in digit order (before the offsets arrive)
#pragma unroll
    for (int i = 0; i < kPassItems; ++i) {
        const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
        if (idx < n) {
            const uint32_t dd = (kr[i] >> shift) & 0xFFu;
            stage[loc[dd] + cnt[dd * NW + w] + rk[i]] = kr[i];
        }
    }
    // 3. this tile's global offsets
    if (tid < 256) gbase[tid] = wait_word(base_words + (size_t)tid * T + tile, epoch, ctl);
    __syncthreads();
    if (pass == 3 && tid == 0) {
        // the sort's last pass: once every tile has its offsets nothing waits
        // any more, and the last tile here frees the lock
        if (atomicAdd(&ctl->done[1], 1u) == T - 1u) {
            ctl->done[1] = 0u;
            atomicExch(&g_resident_owner, 0u);
        }
    }
    const long long rem = n - base;
    const int tcount = rem < kPassTile ? (int)rem : kPassTile;
    for (int jj = tid; jj < tcount; jj += kPassThreads) {
        const uint32_t key = stage[jj];
        const uint32_t dd = (key >> shift) & 0xFFu;
        out[(size_t)gbase[dd] + (size_t)(jj - (int)loc[dd])] = key;
    }
}

LS_DEV void pass_lookback(const uint32_t* __restrict__ in, int in_is_float, uint32_t* __restrict__ out, long long n,
                          int pass, unsigned long long* status, uint32_t epoch, const uint32_t* goff, Ctl* ctl,
                          const PassLds& sm) {
    constexpr int NW = kPassThreads / 64;
    uint32_t* cnt = sm.cnt;
    uint32_t* stage = sm.stage;
    uint32_t* loc = sm.loc;
    uint32_t* gbase = sm.gbase;
    uint32_t* scr = sm.scr;
    uint32_t& s_tile = sm.hist[0];
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const int shift = 8 * pass;
    if (tid == 0) s_tile = atomicAdd(&ctl->tile_ctr[pass], 1u);
    for (int e = tid; e < 256 * NW; e += kPassThreads) cnt[e] = 0u;
    __syncthreads();
    const uint32_t tile = s_tile;
    const long long base = (long long)tile * kPassTile;
    uint32_t kr[kPassItems];
    uint32_t rk[kPassItems];
#pragma unroll
    for (int i = 0; i < kPassItems; ++i) {
        const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
        uint32_t key = 0u;
        if (idx < n) key = in_is_float ? f2key(__uint_as_float(in[idx])) : in[idx];
        kr[i] = key;
    }
    volatile uint32_t* vc = cnt;
#pragma unroll
    for (int i = 0; i < kPassItems; ++i) {
        const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
        const bool valid = idx < n;
        const unsigned long long act = ballot(valid);
        rk[i] = 0u;
        if (act != 0ull) {
            const uint32_t d = (kr[i] >> shift) & 0xFFu;
            const unsigned long long peers = match_digit8(d, act);
            const uint32_t b0 = vc[d * NW + w];
            rk[i] = b0 + (uint32_t)mbcnt(peers);
            if (valid && lane == 63 - __clzll(peers)) vc[d * NW + w] = b0 + (uint32_t)popc64(peers);
        }
    }
    __syncthreads();
    // thread d < 256: per-wave exclusive offsets and the tile total of digit d
    const int d = tid;
    uint32_t tot = 0u;
    if (d < 256) {
#pragma unroll
        for (int q = 0; q < NW; ++q) { const uint32_t x = cnt[d * NW + q]; cnt[d * NW + q] = tot; tot += x; }
    }
    const uint32_t dex = block_exclusive_scan<kPassThreads>(tot, nullptr, scr);
    if (d < 256) {
        loc[d] = dex;
        // decoupled look-back on digit d, up to kLookWindow predecessors per
        // round trip: aggregates are added until an inclusive prefix ends it
        unsigned long long* st = status + (size_t)tile * 256 + d;
        if (tile == 0) {
            __hip_atomic_store(st, st_pack(epoch, kStInc, tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            gbase[d] = goff[pass * 256 + d];
        } else {
            __hip_atomic_store(st, st_pack(epoch, kStAgg, tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t excl = 0u;
            long long j = (long long)tile - 1;
            unsigned int spins = 0u;
            bool done = false;
            while (!done && j >= 0) {
                unsigned long long sw[kLookWindow];
#pragma unroll
                for (int q = 0; q < kLookWindow; ++q)
                    sw[q] = (j - q >= 0) ? __hip_atomic_load(status + (size_t)(j - q) * 256 + d, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)
                                         : 0ull;
                int used = 0;
#pragma unroll
                for (int q = 0; q < kLookWindow; ++q) {
                    if (done || used < q || j - q < 0) continue;  // stop at the first word not yet usable
                    const unsigned long long sq = sw[q];
                    const uint32_t ep = (uint32_t)(sq >> 34);
                    const unsigned long long fl = (sq >> 32) & 3ull;
                    if (ep != epoch || fl == 0ull) continue;
                    excl += (uint32_t)sq;
                    used = q + 1;
                    if (fl == kStInc) done = true;
                }
                j -= used;
                if (!done && used == 0) {
                    // tiles are handed out in order, so the predecessor is
                    // resident and publishes within microseconds; a bounded
                    // wait turns a broken invariant into a reported error
                    if (++spins > (1u << 24)) { atomicOr(&ctl->flags, kFlagInternal); break; }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            __hip_atomic_store(st, st_pack(epoch, kStInc, excl + tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            gbase[d] = goff[pass * 256 + d] + excl;
        }
    }
    __syncthreads();
    // local scatter into LDS in digit order, then coalesced runs to global
#pragma unroll
    for (int i = 0; i < kPassItems; ++i) {
        const long long idx = base + (long long)((w * kPassItems + i) * 64 + lane);
        if (idx < n) {
            const uint32_t dd = (kr[i] >> shift) & 0xFFu;
            stage[loc[dd] + cnt[dd * NW + w] + rk[i]] = kr[i];
        }
    }
    __syncthreads();
    const long long rem = n - base;
    const int tcount = rem < kPassTile ? (int)rem : kPassTile;
    for (int jj = tid; jj < tcount; jj += kPassThreads) {
        const uint32_t key = stage[jj];
        const uint32_t dd = (key >> shift) & 0xFFu;
        out[(size_t)gbase[dd] + (size_t)(jj - (int)loc[dd])] = key;
    }
}

__global__ __launch_bounds__(kPassThreads) void k_radix_pass(const uint32_t* __restrict__ in, int in_is_float,
                                                              uint32_t* __restrict__ out, long long n, int pass,
                                                              unsigned long long* status, uint32_t epoch,
                                                              const uint32_t* goff, Ctl* ctl) {
    __shared__ uint32_t cnt[256 * (kPassThreads / 64)];
    __shared__ uint32_t stage[kPassTile];
    __shared__ uint32_t hist[kHistCopies * 256];
    __shared__ uint32_t loc[256];
    __shared__ uint32_t gbase[256];
    __shared__ uint32_t scr[kPassThreads / 64 + 2];
    const PassLds sm{cnt, stage, hist, loc, gbase, scr};
    if (ctl->resident) pass_resident(in, in_is_float, out, n, pass, status, epoch, goff, ctl, sm);
    else pass_lookback(in, in_is_float, out, n, pass, status, epoch, goff, ctl, sm);
}

// One LSD pass as count, scan, scatter, for more tiles than fit on the
// device at once (no tile waits on another; the keys are read twice).
//   k_radix_count    per tile (2048 keys): its 256 digit counts, written
//                    digit-major: counts[d * T + tile]
//   k_radix_scan     per digit, over the tiles: tile_base[d * T + tile] =
//                    the digit's global offset + the counts of earlier tiles
//   k_radix_scatter  per tile: stable ranks (wave-level multisplit), a local
//                    scatter into LDS in digit order, coalesced runs to global
LS_DEV uint32_t radix_key(const uint32_t* in, int in_is_float, long long idx) {
    return in_is_float ? f2key(__uint_as_float(in[idx])) : in[idx];
}

// Workgroups are dealt to the 8 XCDs in turn; the tile of workgroup b gives
// each XCD a contiguous range of tiles, so that neighbouring tiles' writes
// (count columns, runs of one digit) meet in one L2 and leave it as whole
// lines.  The grid is 8 * ceil(T / 8); workgroups past the last tile return.
constexpr int kXcds = 8;
LS_DEV long long xcd_tile(long long T) {
    const long long per = (T + kXcds - 1) / kXcds;
    return (long long)(blockIdx.x % kXcds) * per + (long long)(blockIdx.x / kXcds);
}
inline unsigned xcd_grid(long long T) { return (unsigned)(kXcds * ((T + kXcds - 1) / kXcds)); }

// kSplitThreads, kSplitItems: measured on gfx950 at 10^7 and 10^8 keys,
// 512 threads x 8 keys (4096-key tiles) beat 256 x 8 (313 against 293 us at
// 10^7, 2664 against 2524 us at 10^8), 256 x 16, 384 x 8, 512 x 4, 6 and 12,
// 768 x 8 and 1024 x 4 and 8.
constexpr int kSplitTile = kSplitTileKeys;
static_assert(kSplitTile == kSplitThreads * kSplitItems, "tile = threads x keys per thread");
static_assert(kSplitThreads >= 256 && kSplitThreads % 64 == 0, "a thread per digit, whole waves");

__global__ __launch_bounds__(kSplitThreads) void k_radix_count(const uint32_t* __restrict__ in, int in_is_float,
                                                                long long n, int pass, uint32_t* __restrict__ counts,
                                                                long long T, unsigned long long* totw) {
    __shared__ uint32_t cnt[kHistCopies * 256];
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const int shift = 8 * pass;
    const long long tile = xcd_tile(T);
    if (tile >= T) return;
    const long long base = tile * kSplitTile;
    for (int e = tid; e < kHistCopies * 256; e += kSplitThreads) cnt[e] = 0u;
    __syncthreads();
    uint32_t kr[kSplitItems];
    // counts only: one LDS atomic add per key into the copy of its lane
    // group (as in k_radix_hist)
    uint32_t* cl = cnt + (lane & (kHistCopies - 1)) * 256;
    if (base + kSplitTile <= n && (reinterpret_cast<uintptr_t>(in) & 15u) == 0u) {
        // a whole tile (the order of counting is free): four consecutive
        // keys per 16-byte load, every load of the thread in flight at once
        constexpr int Q = kSplitItems / 4;
        static_assert(Q * 4 == kSplitItems, "");
        const uint4* in4 = reinterpret_cast<const uint4*>(in + base);
        uint4 q[Q];
#pragma unroll
        for (int j = 0; j < Q; ++j) q[j] = in4[j * kSplitThreads + tid];
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            kr[4 * j] = q[j].x; kr[4 * j + 1] = q[j].y; kr[4 * j + 2] = q[j].z; kr[4 * j + 3] = q[j].w;
        }
        bool bad = false;
#pragma unroll
        for (int i = 0; i < kSplitItems; ++i) {
            if (in_is_float) bad |= !finite_f(__uint_as_float(kr[i]));
            const uint32_t key = in_is_float ? f2key(__uint_as_float(kr[i])) : kr[i];
            atomicAdd(&cl[(key >> shift) & 0xFFu], 1u);
        }
        if (ballot(bad) != 0ull && lane == 0) atomicOr(&totw[4 * 256], 1ull);
    } else {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < kSplitItems; ++i) {
            const long long idx = base + (long long)((w * kSplitItems + i) * 64 + lane);
            kr[i] = 0u;
            if (idx < n) {
                const uint32_t raw = in[idx];
                if (in_is_float) bad |= !finite_f(__uint_as_float(raw));
                kr[i] = in_is_float ? f2key(__uint_as_float(raw)) : raw;
            }
        }
#pragma unroll
        for (int i = 0; i < kSplitItems; ++i) {
            const long long idx = base + (long long)((w * kSplitItems + i) * 64 + lane);
            if (idx < n) atomicAdd(&cl[(kr[i] >> shift) & 0xFFu], 1u);
        }
        if (ballot(bad) != 0ull && lane == 0) atomicOr(&totw[4 * 256], 1ull);
    }
    __syncthreads();
    if (tid < 256) {  // thread = digit
        uint32_t c = 0u;
#pragma unroll
        for (int q = 0; q < kHistCopies; ++q) c += cnt[q * 256 + tid];
        counts[(size_t)tid * (size_t)T + (size_t)tile] = c;
        // the pass's digit totals: eight copies, one per XCD (workgroups are
        // dealt to the XCDs in turn), so that each word takes the adds of
        // one XCD's tiles only
        if (c) atomicAdd(reinterpret_cast<uint32_t*>(totw) + (blockIdx.x % kXcds) * 256 + tid, c);
    }
}

// One workgroup per digit: exclusive scan of its counts over the tiles,
// starting at the digit's global offset, which the scan forms itself (no
// histogram pass before the split sort) from the digit totals the count
// pass added up: eight copies of 256 words (one per XCD), uint32 words at
// totw; totw[4 * 256] (uint64) is the non-finite flag.  The workgroup of
// digit 0 of pass 0 also sets the status flags from that flag.
__global__ __launch_bounds__(1024) void k_radix_scan(const uint32_t* __restrict__ counts, long long T, int pass,
                                                      uint32_t* __restrict__ tile_base, unsigned long long* totw,
                                                      Ctl* ctl) {
    constexpr int IT = 8, NT = 1024;
    __shared__ uint32_t scr[NT / 64 + 2];
    const int tid = threadIdx.x;
    const int d = blockIdx.x;
    const uint32_t* col = counts + (size_t)d * (size_t)T;
    uint32_t* out = tile_base + (size_t)d * (size_t)T;
    uint32_t below = 0u;
    if (tid < d) {
        const uint32_t* t32 = reinterpret_cast<const uint32_t*>(totw);
#pragma unroll
        for (int q = 0; q < kXcds; ++q) below += t32[q * 256 + tid];
    }
    uint32_t carry = 0u;
    (void)block_exclusive_scan<NT>(below, &carry, scr);
    if (pass == 0 && d == 0 && tid == 0)  // the sort starts the flags afresh, as the histogram kernel does
        ctl->flags = totw[4 * 256] ? kFlagNonFinite : 0;
    for (long long c0 = 0; c0 < T; c0 += (long long)NT * IT) {
        uint32_t v[IT];
        uint32_t sum = 0u;
#pragma unroll
        for (int q = 0; q < IT; ++q) {
            const long long t = c0 + (long long)tid * IT + q;
            v[q] = t < T ? col[t] : 0u;
            sum += v[q];
        }
        uint32_t ctotal = 0u;
        uint32_t ex = block_exclusive_scan<NT>(sum, &ctotal, scr) + carry;
#pragma unroll
        for (int q = 0; q < IT; ++q) {
            const long long t = c0 + (long long)tid * IT + q;
            if (t < T) out[t] = ex;
            ex += v[q];
        }
        carry += ctotal;
    }
}

__global__ __launch_bounds__(kSplitThreads) void k_radix_scatter(const uint32_t* __restrict__ in, int in_is_float,
                                                                  uint32_t* __restrict__ out, long long n, int pass,
                                                                  const uint32_t* __restrict__ tile_base, long long T,
                                                                  unsigned long long* totw) {
    constexpr int NW = kSplitThreads / 64;
    __shared__ uint32_t cnt[256 * NW];
    __shared__ uint32_t stage[kSplitTile];
    __shared__ uint32_t loc[256];
    __shared__ uint32_t gbase[256];
    __shared__ uint32_t scr[NW + 2];
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const int shift = 8 * pass;
    if (blockIdx.x == 0) {  // the scan has read this pass's digit totals (and the non-finite flag)
        uint32_t* t32 = reinterpret_cast<uint32_t*>(totw);
        for (int i = tid; i < kXcds * 256; i += kSplitThreads) t32[i] = 0u;
        if (pass == 0 && tid == 0) totw[4 * 256] = 0ull;
    }
    const long long tile = xcd_tile(T);
    if (tile >= T) return;
    const long long base = tile * kSplitTile;
    for (int e = tid; e < 256 * NW; e += kSplitThreads) cnt[e] = 0u;
    if (tid < 256) gbase[tid] = tile_base[(size_t)tid * (size_t)T + (size_t)tile];
    uint32_t kr[kSplitItems];
    uint32_t rk[kSplitItems];
    if (base + kSplitTile <= n && (reinterpret_cast<uintptr_t>(in) & 15u) == 0u) {
        // a whole tile read with 16-byte loads, then turned into the rows the
        // ranking walks (wave w, row i: keys (w * kSplitItems + i) * 64 + lane)
        // through the stage buffer, which the ranking's barrier frees again
        constexpr int Q = kSplitItems / 4;
        const uint4* in4 = reinterpret_cast<const uint4*>(in + base);
        uint4 q[Q];
#pragma unroll
        for (int j = 0; j < Q; ++j) q[j] = in4[j * kSplitThreads + tid];
#pragma unroll
        for (int j = 0; j < Q; ++j) reinterpret_cast<uint4*>(stage)[j * kSplitThreads + tid] = q[j];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSplitItems; ++i) {
            const uint32_t raw = stage[(w * kSplitItems + i) * 64 + lane];
            kr[i] = in_is_float ? f2key(__uint_as_float(raw)) : raw;
        }
    } else {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSplitItems; ++i) {
            const long long idx = base + (long long)((w * kSplitItems + i) * 64 + lane);
            kr[i] = idx < n ? radix_key(in, in_is_float, idx) : 0u;
        }
    }
    volatile uint32_t* vc = cnt;
#pragma unroll
    for (int i = 0; i < kSplitItems; ++i) {
        const long long idx = base + (long long)((w * kSplitItems + i) * 64 + lane);
        const bool valid = idx < n;
        const unsigned long long act = ballot(valid);
        rk[i] = 0u;
        if (act != 0ull) {
            const uint32_t d = (kr[i] >> shift) & 0xFFu;
            const unsigned long long peers = match_digit8(d, act);
            const uint32_t b0 = vc[d * NW + w];
            rk[i] = b0 + (uint32_t)mbcnt(peers);
            if (valid && lane == 63 - __clzll(peers)) vc[d * NW + w] = b0 + (uint32_t)popc64(peers);
        }
    }
    __syncthreads();
    // thread d < 256: per-wave exclusive offsets and the tile's exclusive
    // digit offsets
    uint32_t tot = 0u;
    if (tid < 256) {
#pragma unroll
        for (int q = 0; q < NW; ++q) { const uint32_t x = cnt[tid * NW + q]; cnt[tid * NW + q] = tot; tot += x; }
    }
    const uint32_t ex = block_exclusive_scan<kSplitThreads>(tot, nullptr, scr);
    if (tid < 256) loc[tid] = ex;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSplitItems; ++i) {
        const long long idx = base + (long long)((w * kSplitItems + i) * 64 + lane);
        if (idx < n) {
            const uint32_t dd = (kr[i] >> shift) & 0xFFu;
            stage[loc[dd] + cnt[dd * NW + w] + rk[i]] = kr[i];
        }
    }
    __syncthreads();
    const long long rem = n - base;
    const int tcount = rem < kSplitTile ? (int)rem : kSplitTile;
    for (int j = tid; j < tcount; j += kSplitThreads) {
        const uint32_t key = stage[j];
        const uint32_t dd = (key >> shift) & 0xFFu;
        out[(size_t)gbase[dd] + (size_t)(j - (int)loc[dd])] = key;
    }
}

// ---------------------------------------------------------------------------
// curve aggregates of the fully sorted scores, then the solve
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCurveThreads) void k_curve_tiles(const uint32_t* __restrict__ keys, long long n,
                                                                SegArrays seg, double inv_t) {
    __shared__ double s_red[kCurveThreads / 64];
    const int tile = blockIdx.x;
    const long long base = (long long)tile * kCurveTile;
    const long long rem = n - base;
    const int c = rem < kCurveTile ? (int)rem : kCurveTile;
    // stored in the slot the one-workgroup root reads it from
    const int at = seg_slot(tile, (int)((gridDim.x + kCurveRootThreads - 1) / kCurveRootThreads), kCurveRootThreads);
    if (c == kCurveTile && (reinterpret_cast<uintptr_t>(keys) & 15u) == 0u) {
        // a whole tile: every key of a thread requested at once (four
        // 16-byte loads), with the tile's first and last key
        constexpr int Q = kCurveTile / (4 * kCurveThreads);
        const uint4* k4 = reinterpret_cast<const uint4*>(keys + base);
        const int tid = threadIdx.x;
        uint4 q[Q];
#pragma unroll
        for (int j = 0; j < Q; ++j) q[j] = k4[j * kCurveThreads + tid];
        const float f = key2f(keys[base]);
        const float l = key2f(keys[base + c - 1]);
        double p = 0.0, bx = 0.0;
        auto one = [&](uint32_t key, bool first) {
            const double v = (double)key2f(key);
            p += (double)exp_neg((float)((v - (double)l) * inv_t));
            if (!first) bx += (double)exp_neg((float)(((double)f - v) * inv_t));
        };
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            one(q[j].x, j == 0 && tid == 0);  // key 0 is v_0 itself: no term in Bx
            one(q[j].y, false);
            one(q[j].z, false);
            one(q[j].w, false);
        }
        const double ps = block_sum<kCurveThreads>(p, s_red);
        const double bs = block_sum<kCurveThreads>(bx, s_red);
        if (tid == 0) { seg.first[at] = f; seg.last[at] = l; seg.P[at] = ps; seg.Bx[at] = bs; }
    } else {
        segment_aggregates<kCurveThreads>(keys + base, c, inv_t, &seg.first[at], &seg.last[at], &seg.P[at],
                                          &seg.Bx[at], s_red);
    }
    if (threadIdx.x == 0) { seg.cnt[at] = (uint32_t)c; seg.off[at] = (uint32_t)base; }
}

// ctl_tails: the scores are a part of a larger set whose rest is summarised
// in ctl as tails (aL, S_L below; aR, S_R and the count c_R above)
// one workgroup of kCurveRootThreads: a thread per segment (several past 4M
// scores, stored in seg_slot order) and four scores per thread in the root
// segment

__global__ __launch_bounds__(kCurveRootThreads) void k_curve_root(const uint32_t* __restrict__ keys, long long n,
                                                                   int ntiles, Ctl* ctl, SegArrays seg,
                                                                   SolveScratch sc, double k, double t, double inv_t,
                                                                   double* b_out, int ctl_tails) {
    __shared__ float s_k[kCurveRootThreads];
    __shared__ double s_v[kCurveRootThreads];
    __shared__ int s_int[32];
    SegView sv{ntiles, seg.first, seg.last, seg.P, seg.Bx, seg.cnt, seg.off, keys, nullptr};
    // the sorted scores run from keys[0] to keys[n - 1]
    Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t, key2f(keys[0]), key2f(keys[n - 1])};
    if (ctl_tails) {
        tl.aL = ctl->aL; tl.S_L = ctl->S_L;
        tl.aR = ctl->aR; tl.S_R = ctl->S_R;
        tl.c_R = (double)ctl->c_R;
        tl.fL = tl.aL; tl.fH = tl.aR;
    }
    SolveOut o = segment_solve<kCurveRootThreads, kCurveTile / kCurveRootThreads>(sv, tl, sc, s_k, s_v, s_int);
    if (threadIdx.x == 0) {
        double b = o.b;
        if (ctl->flags & kFlagNonFinite) b = __longlong_as_double(0x7ff8000000000000ll);
        else if (!o.ok) atomicOr(&ctl->flags, kFlagInternal);
        ctl->b = b;
        ctl->jstar = o.jstar;
        if (b_out) *b_out = b;
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
void launch_small_solve(const float* r, int n, double k, double t, Ctl* ctl, SolveScratch sc, double* b_out,
                        uint32_t* keys_out, hipStream_t s) {
    hipLaunchKernelGGL(k_small_solve, dim3(1), dim3(kSortThreads), 0, s, r, n, k, t, 1.0 / t, ctl, sc, b_out,
                       keys_out);
}

void launch_bucket_solve(uint32_t* bucket_vals, const uint32_t* bucket_cnt, int cap, int nb, Ctl* ctl, SegArrays seg,
                         SolveScratch sc, double k, double t, double* b_out, hipStream_t s, const HeavyArrays* ha,
                         const int* gate, HostSummary* hs, unsigned int seq) {
    HeavyArrays hv{};
    if (ha) hv = *ha;
    hipLaunchKernelGGL(k_bucket_agg, dim3(nb), dim3(kAggThreads), 0, s, bucket_vals, bucket_cnt, cap, seg, 1.0 / t, hv,
                       ha ? 1 : 0, gate);
    hipLaunchKernelGGL(k_band_root, dim3(1), dim3(kSortThreads), 0, s, bucket_vals, nb, ctl, seg, sc, k, t, 1.0 / t,
                       b_out, gate, hs, seq);
}

int radix_hist_blocks(long long n) {
    long long b = (n + 16LL * kRadixThreads - 1) / (16LL * kRadixThreads);  // >= 16 keys per thread
    if (b < 1) b = 1;
    if (b > kRadixHistBlocks) b = kRadixHistBlocks;
    return (int)b;
}

// The resident pass needs every tile on the device at once: at most the
// device's co-resident workgroups of the pass kernel, queried once per device.
static long long onesweep_capacity() {
    static std::atomic<long long> cap[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    long long c = cap[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int cus = 0, per = 0;
        c = -1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_radix_pass, kPassThreads, 0) == hipSuccess)
            c = (long long)cus * (long long)per;
        cap[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// status words of a sort of up to n_cap keys: the split passes' counts and
// tile offsets (32-bit, T each per digit) or the one-kernel passes' count and
// offset words (64-bit, T each per digit)
size_t radix_status_words(long long n_cap) {
    const long long T = std::max<long long>((n_cap + kPassTile - 1) / kPassTile, 1);
    const long long Ts = std::max<long long>((n_cap + kSplitTile - 1) / kSplitTile, 1);
    return (size_t)256 * (size_t)std::max<long long>(Ts, 2 * std::min<long long>(T, kOnesweepMaxTiles));
}

bool radix_uses_onesweep(long long n) {
    const long long T = (n + kPassTile - 1) / kPassTile;
    return T <= kOnesweepMaxTiles && T <= onesweep_capacity();
}

void launch_radix_sort(const float* r, long long n, uint32_t* keysA, uint32_t* keysB, uint32_t* hist_part,
                       uint32_t* goff, unsigned long long* status, uint32_t epoch_base, Ctl* ctl, hipStream_t s,
                       int form) {
    const int hb = radix_hist_blocks(n);
    const bool onesweep = form != 2 && radix_uses_onesweep(n);
    // the lock holder's token: the control block's address (distinct per workspace)
    const unsigned int token = (unsigned int)(reinterpret_cast<uintptr_t>(ctl) >> 8) | 1u;
    // the one-kernel passes take their digit offsets from the histogram
    // kernel; the split passes form them in their scan kernels
    if (onesweep)
        hipLaunchKernelGGL(k_radix_hist, dim3(hb), dim3(kRadixThreads), 0, s, r, n, hist_part, goff, ctl,
                           form == 0 ? 1 : 0, token);
    unsigned long long* totw = reinterpret_cast<unsigned long long*>(hist_part + kSplitTotOffset);
    const long long T = onesweep ? (n + kPassTile - 1) / kPassTile : (n + kSplitTile - 1) / kSplitTile;
    // the status region: the one-kernel passes' count and offset words (8
    // bytes, 256 T each), or the split passes' tile counts and tile offsets
    // (4 bytes, 256 T each)
    uint32_t* counts = reinterpret_cast<uint32_t*>(status);
    uint32_t* tile_base = counts + (size_t)256 * (size_t)T;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(r);
    uint32_t* dst = keysA;
    for (int p = 0; p < 4; ++p) {
        int is_float = p == 0 ? 1 : 0;
        if (onesweep) {
            hipLaunchKernelGGL(k_radix_pass, dim3((unsigned)T), dim3(kPassThreads), 0, s, src, is_float, dst, n, p,
                               status, epoch_base + (uint32_t)p, goff, ctl);
        } else {
            hipLaunchKernelGGL(k_radix_count, dim3(xcd_grid(T)), dim3(kSplitThreads), 0, s, src, is_float, n, p,
                               counts, T, totw);
            hipLaunchKernelGGL(k_radix_scan, dim3(256), dim3(1024), 0, s, counts, T, p, tile_base, totw, ctl);
            hipLaunchKernelGGL(k_radix_scatter, dim3(xcd_grid(T)), dim3(kSplitThreads), 0, s, src, is_float, dst, n,
                               p, tile_base, T, totw);
        }
        src = dst;
        dst = (dst == keysA) ? keysB : keysA;
    }
    // four passes: r -> A -> B -> A -> B; the sorted keys end in keysB
}

void launch_curve_tiles(const uint32_t* keys, long long n, Ctl* ctl, SegArrays seg, SolveScratch sc, double k,
                        double t, double* b_out, hipStream_t s, bool ctl_tails) {
    const unsigned tiles = (unsigned)((n + kCurveTile - 1) / kCurveTile);
    hipLaunchKernelGGL(k_curve_tiles, dim3(tiles), dim3(kCurveThreads), 0, s, keys, n, seg, 1.0 / t);
    hipLaunchKernelGGL(k_curve_root, dim3(1), dim3(kCurveRootThreads), 0, s, keys, n, (int)tiles, ctl, seg, sc, k, t,
                       1.0 / t, b_out, ctl_tails ? 1 : 0);
}

}  // namespace lapsum
