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
//                   workgroup turns them into global digit offsets.
//   k_radix_pass    one LSD digit pass (decoupled look-back across tiles).
//   k_curve_tiles   per-tile curve aggregates of the sorted scores; the last
//                   workgroup solves.
#include "lapsum_blocksolve.h"
#include "lapsum_launch.h"

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
    __shared__ double s_red[kSortThreads / 64];
    __shared__ float sg_first, sg_last;
    __shared__ double sg_P, sg_Bx;
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
    segment_aggregates<kSortThreads>(keys, n, inv_t, &sg_first, &sg_last, &sg_P, &sg_Bx, s_red);
    if (tid == 0) { sg_cnt = (uint32_t)n; sg_off = 0u; }
    __syncthreads();
    SegView sv{1, &sg_first, &sg_last, &sg_P, &sg_Bx, &sg_cnt, &sg_off, keys, nullptr, nullptr, nullptr, nullptr};
    Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t};
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
    SegView sv{nb, seg.first, seg.last, seg.P, seg.Bx, seg.cnt, seg.off, bucket_vals, nullptr, nullptr, nullptr, sortbuf};
    Tails tl{ctl->aL, ctl->aR, ctl->S_L, ctl->S_R, (double)ctl->m, (double)ctl->c_R, k, t, inv_t};
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
// multi-workgroup LSD radix sort (Onesweep-style: one histogram pass, then
// one pass per 8-bit digit with decoupled look-back; Merrill & Garland,
// "Single-pass parallel prefix scan with decoupled look-back", and Adinets
// & Merrill, "Onesweep", 2022)
// ---------------------------------------------------------------------------
// Digit histograms of all four LSD passes in one read.  Per workgroup in LDS,
// one atomic add per key and digit (measured on gfx950: 2.3x faster than
// grouping a wave's equal digits with ballots first), except that a wave
// whose keys all share a digit adds once.  The workgroup totals then go
// into the global totals with integer atomics (order-free: deterministic).
// hist: global uint32[1025] (four 256-bin histograms, then a non-finite
// flag), all zero on entry; k_radix_offsets reads and re-zeroes it.
__global__ __launch_bounds__(kRadixThreads) void k_radix_hist(const float* __restrict__ r, long long n,
                                                               uint32_t* __restrict__ hist) {
    __shared__ uint32_t h[4 * 256];
    __shared__ int s_bad;
    const int tid = threadIdx.x, lane = lane_id();
    for (int i = tid; i < 1024; i += kRadixThreads) h[i] = 0u;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    // whole-wave call: valid marks the lanes that hold a key
    auto add = [&](float v, bool valid) {
        bad |= valid && !finite_f(v);
        const uint32_t key = f2key(v);
        const unsigned long long act = ballot(valid);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t d = (key >> (8 * p)) & 0xFFu;
            const uint32_t d0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)d);
            if (ballot(valid && d == d0) == act) {  // one digit for the whole wave: one add
                if (lane == __ffsll((long long)act) - 1) atomicAdd(&h[p * 256 + d0], (uint32_t)popc64(act));
            } else if (valid) {
                atomicAdd(&h[p * 256 + d], 1u);
            }
        }
    };
    const long long stride = (long long)gridDim.x * kRadixThreads;
    if ((reinterpret_cast<uintptr_t>(r) & 15u) == 0u) {
        const long long n4 = n >> 2;
        const float4* r4 = reinterpret_cast<const float4*>(r);
        for (long long base = (long long)blockIdx.x * kRadixThreads; base < n4; base += stride) {
            const long long i = base + tid;
            const bool valid = i < n4;
            const float4 v = valid ? r4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            add(v.x, valid); add(v.y, valid); add(v.z, valid); add(v.w, valid);
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
    for (int i = tid; i < 1024; i += kRadixThreads)
        if (h[i]) atomicAdd(&hist[i], h[i]);
    if (tid == 0 && s_bad) atomicOr(&hist[1024], 1u);
}

// exclusive digit offsets of the four passes from the global totals; the
// totals are re-zeroed for the next sort
__global__ __launch_bounds__(256) void k_radix_offsets(uint32_t* hist, uint32_t* goff, Ctl* ctl) {
    __shared__ uint32_t scr[256 / 64 + 2];
    const int tid = threadIdx.x;
    uint32_t x[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) x[p] = hist[p * 256 + tid];
    const uint32_t bad = hist[1024];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        goff[p * 256 + tid] = block_exclusive_scan<256>(x[p], nullptr, scr);
        hist[p * 256 + tid] = 0u;
    }
    if (tid == 0) {
        hist[1024] = 0u;
        ctl->flags = bad ? kFlagNonFinite : 0;
        for (int p = 0; p < 4; ++p) ctl->tile_ctr[p] = 0u;
    }
}

// One LSD pass in one kernel (onesweep): each tile takes its digit offsets
// from its predecessors' published counts (decoupled look-back).  Fastest
// when the tiles are few; the look-back chain runs through status words that
// cross the XCDs' separate L2 caches, so for many tiles the split form below
// wins.
constexpr unsigned long long kStAgg = 1ull, kStInc = 2ull;

LS_DEV unsigned long long st_pack(uint32_t epoch, unsigned long long flag, uint32_t v) {
    return ((unsigned long long)epoch << 34) | (flag << 32) | (unsigned long long)v;
}

// 1024 threads per 4096-key tile: each wave ranks four rows of 64 keys, so
// the serial chain of counter updates is four long, not sixteen.  All tiles
// of a pass run at once, so a tile adds up its predecessors' counts until it
// meets an inclusive prefix, several predecessors per round trip (measured
// on gfx950: 8 beats 1 and 32; 8192-key tiles gain nothing)
constexpr int kPassThreads = 1024;
constexpr int kPassItems = 4;
constexpr int kPassTile = kPassThreads * kPassItems;
constexpr int kLookWindow = 8;  // predecessors' status words read per round trip

__global__ __launch_bounds__(kPassThreads) void k_radix_pass(const uint32_t* __restrict__ in, int in_is_float,
                                                              uint32_t* __restrict__ out, long long n, int pass,
                                                              unsigned long long* status, uint32_t epoch,
                                                              const uint32_t* goff, Ctl* ctl) {
    constexpr int NW = kPassThreads / 64;
    __shared__ uint32_t cnt[256 * NW];
    __shared__ uint32_t stage[kPassTile];
    __shared__ uint32_t loc[256];
    __shared__ uint32_t gbase[256];
    __shared__ uint32_t scr[NW + 2];
    __shared__ uint32_t s_tile;
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

// One LSD pass as count, scan, scatter (no tile waits on another; for many
// tiles a second read of the tile costs less than the look-back chain).
//   k_radix_count    per tile (4096 keys): its 256 digit counts, written
//                    digit-major: counts[d * T + tile]
//   k_radix_scan     per digit, over the tiles: tile_base[d * T + tile] =
//                    the digit's global offset + the counts of earlier tiles
//   k_radix_scatter  per tile: stable ranks (wave-level multisplit), a local
//                    scatter into LDS in digit order, coalesced runs to global
LS_DEV uint32_t radix_key(const uint32_t* in, int in_is_float, long long idx) {
    return in_is_float ? f2key(__uint_as_float(in[idx])) : in[idx];
}

__global__ __launch_bounds__(kRadixThreads) void k_radix_count(const uint32_t* __restrict__ in, int in_is_float,
                                                                long long n, int pass, uint32_t* __restrict__ counts,
                                                                long long T) {
    __shared__ uint32_t cnt[256];
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const int shift = 8 * pass;
    const long long tile = blockIdx.x;
    const long long base = tile * kRadixTile;
    cnt[tid] = 0u;  // kRadixThreads == 256
    __syncthreads();
    uint32_t kr[kRadixItems];
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const long long idx = base + (long long)((w * kRadixItems + i) * 64 + lane);
        kr[i] = idx < n ? radix_key(in, in_is_float, idx) : 0u;
    }
    // counts only: one LDS atomic add per key (one per wave when the wave's
    // keys all share the digit)
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const long long idx = base + (long long)((w * kRadixItems + i) * 64 + lane);
        const bool valid = idx < n;
        const unsigned long long act = ballot(valid);
        const uint32_t d = (kr[i] >> shift) & 0xFFu;
        const uint32_t d0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)d);
        if (act != 0ull && ballot(valid && d == d0) == act) {
            if (lane == __ffsll((long long)act) - 1) atomicAdd(&cnt[d0], (uint32_t)popc64(act));
        } else if (valid) {
            atomicAdd(&cnt[d], 1u);
        }
    }
    __syncthreads();
    counts[(size_t)tid * (size_t)T + (size_t)tile] = cnt[tid];  // thread = digit
}

// one workgroup per digit: exclusive scan of its counts over the tiles
__global__ __launch_bounds__(1024) void k_radix_scan(const uint32_t* __restrict__ counts, long long T, int pass,
                                                      const uint32_t* __restrict__ goff,
                                                      uint32_t* __restrict__ tile_base) {
    constexpr int IT = 8;
    __shared__ uint32_t scr[1024 / 64 + 2];
    const int d = blockIdx.x, tid = threadIdx.x;
    const uint32_t* col = counts + (size_t)d * (size_t)T;
    uint32_t* out = tile_base + (size_t)d * (size_t)T;
    uint32_t carry = goff[pass * 256 + d];
    for (long long c0 = 0; c0 < T; c0 += 1024LL * IT) {
        uint32_t v[IT];
        uint32_t sum = 0u;
#pragma unroll
        for (int q = 0; q < IT; ++q) {
            const long long t = c0 + (long long)tid * IT + q;
            v[q] = t < T ? col[t] : 0u;
            sum += v[q];
        }
        uint32_t total = 0u;
        uint32_t ex = block_exclusive_scan<1024>(sum, &total, scr) + carry;
#pragma unroll
        for (int q = 0; q < IT; ++q) {
            const long long t = c0 + (long long)tid * IT + q;
            if (t < T) out[t] = ex;
            ex += v[q];
        }
        carry += total;
    }
}

__global__ __launch_bounds__(kRadixThreads) void k_radix_scatter(const uint32_t* __restrict__ in, int in_is_float,
                                                                  uint32_t* __restrict__ out, long long n, int pass,
                                                                  const uint32_t* __restrict__ tile_base, long long T) {
    constexpr int NW = kRadixThreads / 64;
    __shared__ uint32_t cnt[256 * NW];
    __shared__ uint32_t stage[kRadixTile];
    __shared__ uint32_t loc[256];
    __shared__ uint32_t gbase[256];
    __shared__ uint32_t scr[NW + 2];
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    const int shift = 8 * pass;
    const long long tile = blockIdx.x;
    const long long base = tile * kRadixTile;
    for (int e = tid; e < 256 * NW; e += kRadixThreads) cnt[e] = 0u;
    gbase[tid] = tile_base[(size_t)tid * (size_t)T + (size_t)tile];
    __syncthreads();
    uint32_t kr[kRadixItems];
    uint32_t rk[kRadixItems];
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const long long idx = base + (long long)((w * kRadixItems + i) * 64 + lane);
        kr[i] = idx < n ? radix_key(in, in_is_float, idx) : 0u;
    }
    volatile uint32_t* vc = cnt;
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const long long idx = base + (long long)((w * kRadixItems + i) * 64 + lane);
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
    // thread d: per-wave exclusive offsets and the tile's exclusive digit offsets
    const int d = tid;  // kRadixThreads == 256
    uint32_t tot = 0u;
#pragma unroll
    for (int q = 0; q < NW; ++q) { const uint32_t x = cnt[d * NW + q]; cnt[d * NW + q] = tot; tot += x; }
    loc[d] = block_exclusive_scan<kRadixThreads>(tot, nullptr, scr);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRadixItems; ++i) {
        const long long idx = base + (long long)((w * kRadixItems + i) * 64 + lane);
        if (idx < n) {
            const uint32_t dd = (kr[i] >> shift) & 0xFFu;
            stage[loc[dd] + cnt[dd * NW + w] + rk[i]] = kr[i];
        }
    }
    __syncthreads();
    const long long rem = n - base;
    const int tcount = rem < kRadixTile ? (int)rem : kRadixTile;
    for (int j = tid; j < tcount; j += kRadixThreads) {
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
    segment_aggregates<kCurveThreads>(keys + base, c, inv_t, &seg.first[tile], &seg.last[tile], &seg.P[tile],
                                      &seg.Bx[tile], s_red);
    if (threadIdx.x == 0) { seg.cnt[tile] = (uint32_t)c; seg.off[tile] = (uint32_t)base; }
}

// ctl_tails: the scores are a part of a larger set whose rest is summarised
// in ctl as tails (aL, S_L below; aR, S_R and the count c_R above)
__global__ __launch_bounds__(kCurveThreads) void k_curve_root(const uint32_t* __restrict__ keys, long long n, int ntiles,
                                                               Ctl* ctl, SegArrays seg, SolveScratch sc, double k,
                                                               double t, double inv_t, double* b_out, int ctl_tails) {
    __shared__ float s_k[kCurveThreads];
    __shared__ double s_v[kCurveThreads];
    __shared__ int s_int[32];
    SegView sv{ntiles, seg.first, seg.last, seg.P, seg.Bx, seg.cnt, seg.off, keys, nullptr, nullptr, nullptr, nullptr};
    Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t};
    if (ctl_tails) {
        tl.aL = ctl->aL; tl.S_L = ctl->S_L;
        tl.aR = ctl->aR; tl.S_R = ctl->S_R;
        tl.c_R = (double)ctl->c_R;
    }
    SolveOut o = segment_solve<kCurveThreads, kRadixItems>(sv, tl, sc, s_k, s_v, s_int);
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

constexpr long long kOnesweepMaxTiles = 512;  // up to ~2M keys: one kernel per pass

bool radix_uses_onesweep(long long n) { return (n + kRadixTile - 1) / kRadixTile <= kOnesweepMaxTiles; }

void launch_radix_sort(const float* r, long long n, uint32_t* keysA, uint32_t* keysB, uint32_t* hist_part,
                       uint32_t* goff, unsigned long long* status, uint32_t epoch_base, Ctl* ctl, hipStream_t s) {
    const int hb = radix_hist_blocks(n);
    hipLaunchKernelGGL(k_radix_hist, dim3(hb), dim3(kRadixThreads), 0, s, r, n, hist_part);
    hipLaunchKernelGGL(k_radix_offsets, dim3(1), dim3(256), 0, s, hist_part, goff, ctl);
    const long long T = (n + kRadixTile - 1) / kRadixTile;
    // the status region holds 256 * T words of 8 bytes: look-back status words,
    // or (split form) the tile counts followed by the tile bases
    uint32_t* counts = reinterpret_cast<uint32_t*>(status);
    uint32_t* tile_base = counts + (size_t)256 * (size_t)T;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(r);
    uint32_t* dst = keysA;
    for (int p = 0; p < 4; ++p) {
        const int is_float = p == 0 ? 1 : 0;
        if (T <= kOnesweepMaxTiles) {
            const unsigned Tp = (unsigned)((n + kPassTile - 1) / kPassTile);
            hipLaunchKernelGGL(k_radix_pass, dim3(Tp), dim3(kPassThreads), 0, s, src, is_float, dst, n, p, status,
                               epoch_base + (uint32_t)p, goff, ctl);
        } else {
            hipLaunchKernelGGL(k_radix_count, dim3((unsigned)T), dim3(kRadixThreads), 0, s, src, is_float, n, p,
                               counts, T);
            hipLaunchKernelGGL(k_radix_scan, dim3(256), dim3(1024), 0, s, counts, T, p, goff, tile_base);
            hipLaunchKernelGGL(k_radix_scatter, dim3((unsigned)T), dim3(kRadixThreads), 0, s, src, is_float, dst, n,
                               p, tile_base, T);
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
    hipLaunchKernelGGL(k_curve_root, dim3(1), dim3(kCurveThreads), 0, s, keys, n, (int)tiles, ctl, seg, sc, k, t,
                       1.0 / t, b_out, ctl_tails ? 1 : 0);
}

}  // namespace lapsum
