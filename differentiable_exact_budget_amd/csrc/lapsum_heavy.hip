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

constexpr int kHeavyQueue = 2048;                            // per workgroup, in LDS
constexpr int kHeavyQueuePerWave = kHeavyQueue / (kStreamThreads / 64);
constexpr int kHeavyV = 4, kHeavyGrid = 1536;

// hoff[b]: element offset (from `base`) of heavy bucket b's slot, or
// kNotHeavy; hfill[b]: scores placed so far (zeroed before the pass)
__global__ __launch_bounds__(kStreamThreads) void k_heavy_collect(const float* __restrict__ r, long long n,
                                                                   const Ctl* ctl, const float* __restrict__ sp_g,
                                                                   const float* __restrict__ iw_g,
                                                                   const uint32_t* __restrict__ hoff_g, uint32_t* hfill,
                                                                   uint32_t* base) {
    __shared__ float sp[kMaxBuckets + 1];
    __shared__ float iw[kMaxBuckets];
    __shared__ uint32_t hoff[kMaxBuckets];
    __shared__ float q[kHeavyQueue];
    __shared__ uint32_t lcnt[kMaxBuckets];
    __shared__ uint32_t gbase[kMaxBuckets];
    __shared__ uint32_t s_wq[kStreamThreads / 64];
    const int tid = threadIdx.x, lane = lane_id();
    FilterState fs;
    fs.aL = ctl->aL; fs.aR = ctl->aR; fs.ls = 0.0f;
    fs.ng = ctl->ng; fs.J = ctl->J; fs.cap = 0;
    const int nb = ctl->nb;
    for (int i = tid; i <= fs.ng; i += kStreamThreads) sp[i] = sp_g[i];
    for (int i = tid; i < fs.ng; i += kStreamThreads) iw[i] = iw_g[i];
    for (int i = tid; i < nb; i += kStreamThreads) { hoff[i] = hoff_g[i]; lcnt[i] = 0u; }
    fs.sp = sp; fs.iw = iw; fs.bucket_cnt = nullptr; fs.bucket_vals = nullptr;
    __syncthreads();
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
    };
    auto put = [&](float v, uint32_t pos) {
        if (pos < (uint32_t)kHeavyQueuePerWave) wq[pos] = v;
        else direct(v, band_bucket(fs, v));
    };
    auto quad = [&](float4 qv) {
        const bool b0 = heavy_of(qv.x) >= 0, b1 = heavy_of(qv.y) >= 0;
        const bool b2 = heavy_of(qv.z) >= 0, b3 = heavy_of(qv.w) >= 0;
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
    if ((reinterpret_cast<uintptr_t>(r) & 15u) == 0u) {
        const long long n4 = n >> 2;
        tile_f4_pipelined<kHeavyV, true>(reinterpret_cast<const float4*>(r), n4,
                                         [&](float4 qv, long long) { quad(qv); },
                                         [&](float4 qv, long long) {
                                             one_lane(qv.x); one_lane(qv.y); one_lane(qv.z); one_lane(qv.w);
                                         });
        if (blockIdx.x == 0 && tid < 4) {
            const long long j = (n4 << 2) + tid;
            if (j < n) one_lane(r[j]);
        }
    } else {
        const long long stride = (long long)gridDim.x * kStreamThreads;
        for (long long i = (long long)blockIdx.x * kStreamThreads + tid; i < n; i += stride) one_lane(r[i]);
    }
    // flush: rank within the workgroup per bucket, one global atomic per bucket
    if (lane == 0) s_wq[tid >> 6] = min(wfill, (uint32_t)kHeavyQueuePerWave);
    __syncthreads();
    constexpr int QPT = kHeavyQueue / kStreamThreads;
    int bk[QPT];
    uint32_t rk[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const uint32_t i = (uint32_t)tid + (uint32_t)k * kStreamThreads;
        bk[k] = -1;
        if (i % (uint32_t)kHeavyQueuePerWave < s_wq[i / (uint32_t)kHeavyQueuePerWave]) {
            bk[k] = band_bucket(fs, q[i]);
            rk[k] = atomicAdd(&lcnt[bk[k]], 1u);
        }
    }
    __syncthreads();
    for (int j = tid; j < nb; j += kStreamThreads) {
        const uint32_t c = lcnt[j];
        gbase[j] = c ? atomicAdd(&hfill[j], c) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        if (bk[k] >= 0) {
            const uint32_t i = (uint32_t)tid + (uint32_t)k * kStreamThreads;
            base[(size_t)hoff[bk[k]] + gbase[bk[k]] + rk[k]] = __float_as_uint(q[i]);
        }
    }
}

__global__ void k_zero_u32(uint32_t* a, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) a[i] = 0u;
}

void launch_heavy_collect(const float* r, long long n, const Ctl* ctl, const float* sp, const float* iw,
                          const uint32_t* hoff, uint32_t* hfill, uint32_t* base, hipStream_t st) {
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1024), 0, st, hfill, kMaxBuckets);
    const bool vec = (reinterpret_cast<uintptr_t>(r) & 15u) == 0u;
    const long long tiles = stream_tiles<kHeavyV>(n >> 2);
    const int blocks = vec ? (int)std::max<long long>(1, std::min<long long>(tiles, kHeavyGrid)) : stream_blocks(n);
    hipLaunchKernelGGL(k_heavy_collect, dim3(blocks), dim3(kStreamThreads), 0, st, r, n, ctl, sp, iw, hoff, hfill,
                       base);
}

}  // namespace lapsum
