// Buckets that overflowed in the streaming filter (a cluster of equal or
// near-equal scores inside the band is the usual cause).  The filter counted
// them exactly and its tail and band sums stay exact, so the bracket is still
// certified; only the stored scores of those buckets are incomplete.  One
// more pass over r collects every score of the overflowed ("heavy") buckets
// into slots sized by their exact counts, after which the band solve treats
// them like any other bucket (Fast LapSum paper, gist.science summary section
// 2.2, bracketing steps 2-3: out-of-band scores folded, the band solved).
#include "lapsum_band.h"
#include "lapsum_launch.h"
#include "lapsum_streamio.h"

namespace lapsum {

// The collect pass walks r like the filter: one 1024-thread workgroup per CU
// over a fixed share, its waves taking 512-score tiles at run time (the
// misaligned fallback strides over r with the same workgroups)
constexpr int kHeavyThreads = 1024;
constexpr int kHeavyQueuePerWave = 512;
constexpr int kHeavyQueue = kHeavyQueuePerWave * (kHeavyThreads / 64);  // per workgroup, in LDS
constexpr int kHeavyWaveV = 2, kHeavyGrid = 256;  // measured on gfx950: 2 beats 4
constexpr int kHeavyAggGrid = 1024;

// hoff[b]: element offset (from `base`) of heavy bucket b's slot, or
// kNotHeavy; hfill[b]: scores placed so far (zeroed before the pass)
__global__ __launch_bounds__(kHeavyThreads) void k_heavy_collect(const float* __restrict__ r, long long n,
                                                                   const Ctl* ctl, const float* __restrict__ sp_g,
                                                                   const float* __restrict__ iw_g, HeavyArrays ha,
                                                                   uint32_t* base) {
    __shared__ float sp[kMaxBuckets + 1];
    __shared__ float iw[kMaxBuckets];
    __shared__ uint32_t hoff[kMaxBuckets];
    __shared__ float q[kHeavyQueue];
    __shared__ uint32_t lcnt[kMaxBuckets];
    __shared__ uint32_t gbase[kMaxBuckets];
    __shared__ uint32_t lmin[kMaxBuckets];
    __shared__ uint32_t lmax[kMaxBuckets];
    __shared__ uint32_t s_wq[kHeavyThreads / 64];
    __shared__ unsigned int s_ctr;
    if (!(ctl->flags & kFlagHeavy)) return;  // no slots were laid out
    const uint32_t* __restrict__ hoff_g = ha.hoff;
    uint32_t* hfill = ha.hfill;
    const int tid = threadIdx.x, lane = lane_id();
    FilterState fs;
    fs.aL = ctl->aL; fs.aR = ctl->aR; fs.ls = 0.0f;
    fs.ng = ctl->ng; fs.J = ctl->J; fs.cap = 0;
    const int nb = ctl->nb;
    fs.sp = sp; fs.iw = iw; fs.bucket_cnt = nullptr; fs.bucket_vals = nullptr;
    auto prologue = [&]() {
        for (int i = tid; i <= fs.ng; i += kHeavyThreads) sp[i] = sp_g[i];
        for (int i = tid; i < fs.ng; i += kHeavyThreads) iw[i] = iw_g[i];
        for (int i = tid; i < nb; i += kHeavyThreads) {
            hoff[i] = hoff_g[i];
            lcnt[i] = 0u;
            lmin[i] = 0xFFFFFFFFu;
            lmax[i] = 0u;
        }
        if (tid == 0) s_ctr = 0u;
        __syncthreads();
    };
    const float aL = fs.aL, aR = fs.aR;
    float* const wq = q + (tid >> 6) * kHeavyQueuePerWave;
    uint32_t wfill = 0u;  // wave-uniform
    auto heavy_of = [&](float v) -> int {
        if (!(v >= aL && v < aR)) return -1;
        const int bk = band_bucket(fs, v);
        return hoff[bk] != kNotHeavy ? bk : -1;
    };
    auto direct = [&](float v, int bk) {
        const uint32_t pos = atomicAdd(&hfill[bk], 1u);
        base[(size_t)hoff[bk] + pos] = __float_as_uint(v);
        const uint32_t key = f2key(v);
        atomicMin(&ha.hmin[bk], key);
        atomicMax(&ha.hmax[bk], key);
    };
    // a full wave queue: look the bucket up here and append if it overflowed
    auto put = [&](float v, uint32_t pos) {
        if (pos < (uint32_t)kHeavyQueuePerWave) {
            wq[pos] = v;
        } else {
            const int bk = band_bucket(fs, v);
            if (hoff[bk] != kNotHeavy) direct(v, bk);
        }
    };
    // the walk only queues band scores (four compares per float4); the
    // bucket look-up, a chain of dependent LDS reads, runs after the walk for
    // the whole queue at once (inline it stalled the wave's walk once per
    // band score)
    auto quad = [&](float4 qv) {
        const bool b0 = qv.x >= aL && qv.x < aR, b1 = qv.y >= aL && qv.y < aR;
        const bool b2 = qv.z >= aL && qv.z < aR, b3 = qv.w >= aL && qv.w < aR;
        const unsigned long long m0 = ballot(b0), m1 = ballot(b1), m2 = ballot(b2), m3 = ballot(b3);
        if (m0 | m1 | m2 | m3) {
            const uint32_t c0 = (uint32_t)popc64(m0), c1 = (uint32_t)popc64(m1), c2 = (uint32_t)popc64(m2);
            const uint32_t tot = c0 + c1 + c2 + (uint32_t)popc64(m3);
            const uint32_t wb = wfill;
            wfill += tot;
            if (b0) put(qv.x, wb + (uint32_t)mbcnt(m0));
            if (b1) put(qv.y, wb + c0 + (uint32_t)mbcnt(m1));
            if (b2) put(qv.z, wb + c0 + c1 + (uint32_t)mbcnt(m2));
            if (b3) put(qv.w, wb + c0 + c1 + c2 + (uint32_t)mbcnt(m3));
        }
    };
    auto one_lane = [&](float v) {
        const int bk = heavy_of(v);
        if (bk >= 0) direct(v, bk);
    };
    const long long n4 = n >> 2;
    if ((reinterpret_cast<uintptr_t>(r) & 15u) == 0u && n4 >= 64LL * kHeavyWaveV) {
        constexpr long long WT = 64LL * kHeavyWaveV;
        const long long tiles = (n4 + WT - 1) / WT;
        const long long per = (tiles + gridDim.x - 1) / gridDim.x;
        const long long t0 = min(tiles, (long long)blockIdx.x * per), t1 = min(tiles, t0 + per);
        wave_tiles_dynamic<kHeavyWaveV, true>(reinterpret_cast<const float4*>(r), n4, t0, t1, &s_ctr,
                                              [&](float4 qv, long long) { quad(qv); },
                                              [&](float4 qv, long long) {
                                                  one_lane(qv.x); one_lane(qv.y); one_lane(qv.z); one_lane(qv.w);
                                              },
                                              prologue, [](long long) {});
        if (blockIdx.x == 0 && tid < 4) {
            const long long j = (n4 << 2) + tid;
            if (j < n) one_lane(r[j]);
        }
    } else {
        prologue();
        const long long stride = (long long)gridDim.x * kHeavyThreads;
        for (long long i = (long long)blockIdx.x * kHeavyThreads + tid; i < n; i += stride) one_lane(r[i]);
    }
    // flush: rank within the workgroup per bucket, one global atomic per bucket
    if (lane == 0) s_wq[tid >> 6] = min(wfill, (uint32_t)kHeavyQueuePerWave);
    __syncthreads();
    constexpr int QPT = kHeavyQueue / kHeavyThreads;
    int bk[QPT];
    uint32_t rk[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const uint32_t i = (uint32_t)tid + (uint32_t)k * kHeavyThreads;
        bk[k] = -1;
        if (i % (uint32_t)kHeavyQueuePerWave < s_wq[i / (uint32_t)kHeavyQueuePerWave]) {
            const int b = band_bucket(fs, q[i]);
            if (hoff[b] == kNotHeavy) continue;  // a band score of a bucket that did not overflow
            bk[k] = b;
            rk[k] = atomicAdd(&lcnt[bk[k]], 1u);
            const uint32_t key = f2key(q[i]);
            atomicMin(&lmin[bk[k]], key);
            atomicMax(&lmax[bk[k]], key);
        }
    }
    __syncthreads();
    // per bucket one returning atomic for the slots and two for the range;
    // a thread's returning atomics are all issued before any result is used
    constexpr int BPT = (kMaxBuckets + kHeavyThreads - 1) / kHeavyThreads;
    uint32_t got[BPT];
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
        const int j = tid + u * kHeavyThreads;
        const uint32_t c = j < nb ? lcnt[j] : 0u;
        got[u] = c ? atomicAdd(&hfill[j], c) : 0u;
        if (c) {
            atomicMin(&ha.hmin[j], lmin[j]);
            atomicMax(&ha.hmax[j], lmax[j]);
        }
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
        const int j = tid + u * kHeavyThreads;
        if (j < nb) gbase[j] = got[u];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        if (bk[k] >= 0) {
            const uint32_t i = (uint32_t)tid + (uint32_t)k * kHeavyThreads;
            base[(size_t)hoff[bk[k]] + gbase[bk[k]] + rk[k]] = __float_as_uint(q[i]);
        }
    }
}

// One workgroup per chunk of kHeavyChunk scores of an overflowed bucket:
// the two fixed-point sums of the chunk, taken against the bucket's score
// range (known once the collect pass is done), written as four 64-bit words.
// The bucket aggregation adds a bucket's chunks (integer addition: the order
// does not matter).  A persistent grid walks the chunks.
__global__ __launch_bounds__(kStreamThreads) void k_heavy_agg(const uint32_t* __restrict__ base,
                                                              const uint32_t* __restrict__ bucket_cnt,
                                                              const Ctl* ctl, HeavyArrays ha, double inv_t) {
    __shared__ uint32_t s_ch0[kMaxBuckets + 1];
    __shared__ unsigned long long s_fx[4 * (kStreamThreads / 64)];
    if (!(ctl->flags & kFlagHeavy)) return;
    const int tid = threadIdx.x;
    const int nb = ctl->nb;
    const uint32_t nch = ctl->hchunks;
    if ((uint32_t)blockIdx.x >= nch) return;
    for (int i = tid; i < nb; i += kStreamThreads) s_ch0[i] = ha.hch0[i];
    if (tid == 0) s_ch0[nb] = nch;
    __syncthreads();
    constexpr int E = kHeavyChunk / kStreamThreads;
    for (uint32_t j = blockIdx.x; j < nch; j += gridDim.x) {
        // the bucket whose chunk range holds j: the first b with s_ch0[b + 1] > j
        int lo = 0, hi = nb - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_ch0[mid + 1] > j) hi = mid;
            else lo = mid + 1;
        }
        const int b = lo;
        const uint32_t c = bucket_cnt[b];
        const uint32_t start = (j - s_ch0[b]) * (uint32_t)kHeavyChunk;
        const uint32_t* vals = base + ha.hoff[b];
        const double vmin = (double)key2f(ha.hmin[b]), vmax = (double)key2f(ha.hmax[b]);
        Fx128 P = fx_zero(), Q = fx_zero();
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const uint32_t i = start + (uint32_t)tid + (uint32_t)q * kStreamThreads;
            if (i < c) {
                const double v = (double)key2f(f2key(__uint_as_float(vals[i])));
                fx_add_term(P, exp((v - vmax) * inv_t));
                fx_add_term(Q, exp((vmin - v) * inv_t));
            }
        }
        block_sum_fx2<kStreamThreads>(P, Q, s_fx);
        if (tid == 0) {
            unsigned long long* o = ha.hpart + 4ull * j;
            o[0] = P.lo; o[1] = P.hi; o[2] = Q.lo; o[3] = Q.hi;
        }
    }
}

void launch_heavy_collect(const float* r, long long n, const Ctl* ctl, const float* sp, const float* iw,
                          const HeavyArrays& ha, uint32_t* base, uint32_t hchunks, double t, hipStream_t st) {
    const long long wt = ((n >> 2) + 64LL * kHeavyWaveV - 1) / (64LL * kHeavyWaveV);
    const int blocks = (int)std::max<long long>(1, std::min<long long>(kHeavyGrid, (wt + 15) / 16));
    hipLaunchKernelGGL(k_heavy_collect, dim3(blocks), dim3(kHeavyThreads), 0, st, r, n, ctl, sp, iw, ha, base);
    const int ablocks = (int)std::max<uint32_t>(1u, std::min<uint32_t>(hchunks, (uint32_t)kHeavyAggGrid));
    hipLaunchKernelGGL(k_heavy_agg, dim3(ablocks), dim3(kStreamThreads), 0, st, base, ha.hfill, ctl, ha, 1.0 / t);
}

}  // namespace lapsum
