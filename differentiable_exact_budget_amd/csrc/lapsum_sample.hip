// Localisation step of the bracketing path (Fast LapSum paper, gist.science
// section 2.2, "Localizacion"; the arxivdaily abstract: "a binomial
// order-statistic from kernel-noised samples").
//
//  k_sample  x_j = r_{I_j} + eps_j, j < s: I_j uniform in [0, n) with
//            replacement, eps_j ~ Laplace(0, t) by inverse CDF.  Because the
//            noise is the operator's own kernel, P(x > b) = G(b)/n = k/n, so
//            b is the (1 - k/n) quantile of x whatever the scores are.
//            Random numbers: Philox4x32-10 (Salmon et al., SC'11), counter
//            (j_lo, j_hi, 0, 0), key (seed_lo, seed_hi).
//  k_select  one workgroup: a_L = x_(l), a_R = x_(h) by 8-bit MSD radix
//            select, then up to 256 value-ordered buckets for the band:
//            sample values between a_L and a_R as gap splitters, each finite
//            gap cut into J equal-width sub-buckets.
#include "lapsum_launch.h"

namespace lapsum {

LS_DEV void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

__global__ __launch_bounds__(256) void k_sample(const float* __restrict__ r, long long n, double t,
                                                unsigned long long seed, int s, float* __restrict__ x,
                                                long long* idx_out) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= s) return;
    uint32_t c[4] = {(uint32_t)j, 0u, 0u, 0u};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const unsigned long long u64 = ((unsigned long long)c[1] << 32) | c[0];
    const long long idx = (long long)__umul64hi(u64, (unsigned long long)n);
    const unsigned long long m53 = ((((unsigned long long)c[3]) << 32) | c[2]) >> 11;
    const double u = ((double)m53 + 0.5) * 0x1p-53;
    const double eps = (u < 0.5) ? t * log(2.0 * u) : -t * log(2.0 * (1.0 - u));
    x[j] = (float)((double)r[idx] + eps);
    if (idx_out) idx_out[j] = idx;
}

void launch_sample(const float* r, long long n, double t, unsigned long long seed, int s, float* x, long long* idx_out,
                   hipStream_t st) {
    hipLaunchKernelGGL(k_sample, dim3((s + 255) / 256), dim3(256), 0, st, r, n, t, seed, s, x, idx_out);
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelectThreads) void k_select(const float* __restrict__ x, int s, long long l, long long h,
                                                            int cap, Ctl* ctl, float* sp, float* iw,
                                                            uint32_t* bucket_cnt) {
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t cand[kCandMax];
    __shared__ uint32_t scr[kSelectThreads / 64 + 2];
    __shared__ uint32_t s_pre[2], s_rem[2];
    const int tid = threadIdx.x;
    uint32_t kr[kSelectItems];
#pragma unroll
    for (int i = 0; i < kSelectItems; ++i) {
        const int j = i * kSelectThreads + tid;
        kr[i] = j < s ? f2key(x[j]) : 0u;
    }
    const bool want_l = l >= 1 && l <= s;
    const bool want_h = h >= 1 && h <= s;
    if (tid == 0) {
        s_pre[0] = 0u; s_pre[1] = 0u;
        s_rem[0] = want_l ? (uint32_t)l : 1u;
        s_rem[1] = want_h ? (uint32_t)h : 1u;
    }
    // MSD radix select of ranks l and h (1-based), 8 bits at a time
    for (int pass = 3; pass >= 0; --pass) {
        const int shift = 8 * pass;
        const uint32_t hmask = pass == 3 ? 0u : (0xFFFFFFFFu << (shift + 8));
        for (int e = tid; e < 512; e += kSelectThreads) (&hist[0][0])[e] = 0u;
        __syncthreads();
        const uint32_t p0 = s_pre[0], p1 = s_pre[1];
#pragma unroll
        for (int i = 0; i < kSelectItems; ++i) {
            const int j = i * kSelectThreads + tid;
            if (j < s) {
                const uint32_t kk = kr[i];
                const uint32_t d = (kk >> shift) & 0xFFu;
                if ((kk & hmask) == (p0 & hmask)) atomicAdd(&hist[0][d], 1u);
                if ((kk & hmask) == (p1 & hmask)) atomicAdd(&hist[1][d], 1u);
            }
        }
        __syncthreads();
        if (tid == 0 || tid == 64) {
            const int q = tid == 0 ? 0 : 1;
            uint32_t rem = s_rem[q], cum = 0u;
            int d = 0;
            for (; d < 255; ++d) {
                const uint32_t c = hist[q][d];
                if (cum + c >= rem) break;
                cum += c;
            }
            s_pre[q] |= (uint32_t)d << shift;
            s_rem[q] = rem - cum;
        }
        __syncthreads();
    }
    const uint32_t key_l = s_pre[0], key_h = s_pre[1];
    const float aL = want_l ? key2f(key_l) : -INFINITY;
    const float aR = want_h ? key2f(key_h) : INFINITY;
    const uint32_t klo = want_l ? key_l : 0u;
    const uint32_t khi = want_h ? key_h : 0xFFFFFFFFu;

    // candidates for splitters: sample keys in [klo, khi], in sample order
    uint32_t mine = 0u;
#pragma unroll
    for (int i = 0; i < kSelectItems; ++i) {
        const int j = i * kSelectThreads + tid;
        if (j < s && kr[i] >= klo && kr[i] <= khi) ++mine;
    }
    // order candidates by (thread, item): deterministic
    uint32_t total = 0u;
    uint32_t pos = block_exclusive_scan<kSelectThreads>(mine, &total, scr);
    const uint32_t stride = (total + kCandMax - 1) / kCandMax > 0 ? (total + kCandMax - 1) / kCandMax : 1u;
#pragma unroll
    for (int i = 0; i < kSelectItems; ++i) {
        const int j = i * kSelectThreads + tid;
        if (j < s && kr[i] >= klo && kr[i] <= khi) {
            if (pos % stride == 0u) cand[pos / stride] = kr[i];
            ++pos;
        }
    }
    const int cc = (int)((total + stride - 1) / stride);
    __syncthreads();
    for (int e = cc + tid; e < kCandMax; e += kSelectThreads) cand[e] = 0xFFFFFFFFu;
    __syncthreads();
    // bitonic sort of kCandMax keys (one pair per thread per step)
    for (int size = 2; size <= kCandMax; size <<= 1) {
        for (int half = size >> 1; half > 0; half >>= 1) {
            const int a = 2 * half * (tid / half) + (tid % half);
            const int b = a + half;
            const bool up = (a & size) == 0;
            const uint32_t va = cand[a], vb = cand[b];
            if ((va > vb) == up) { cand[a] = vb; cand[b] = va; }
            __syncthreads();
        }
    }
    // gaps: ng <= 256, interior splitters evenly spaced over the sorted candidates
    const int ng = cc >= 2 ? (cc - 1 < kMaxBuckets ? cc - 1 : kMaxBuckets) : 1;
    const int J = kMaxBuckets / ng > 0 ? kMaxBuckets / ng : 1;
    for (int g = tid; g <= ng; g += kSelectThreads) {
        float v;
        if (g == 0) v = aL;
        else if (g == ng) v = aR;
        else v = key2f(cand[(int)(((long long)g * (cc - 1)) / ng)]);
        sp[g] = v;
    }
    __syncthreads();
    __threadfence_block();
    for (int g = tid; g < ng; g += kSelectThreads) {
        const float lo = sp[g], hi = sp[g + 1];
        float w = 0.0f;
        if (finite_f(lo) && finite_f(hi) && hi > lo) {
            const float width = hi - lo;
            w = finite_f(width) ? (float)J / width : 0.0f;
            if (!finite_f(w)) w = 0.0f;
        }
        iw[g] = w;
    }
    for (int b = tid; b < kMaxBuckets; b += kSelectThreads) bucket_cnt[b] = 0u;
    if (tid == 0) {
        ctl->aL = aL; ctl->aR = aR;
        ctl->ng = ng; ctl->J = J; ctl->nb = ng * J;
        ctl->cap = cap;
        ctl->flags = 0;
    }
}

void launch_select(const float* x, int s, long long l, long long h, int cap, Ctl* ctl, float* sp, float* iw,
                   uint32_t* bucket_cnt, hipStream_t st) {
    hipLaunchKernelGGL(k_select, dim3(1), dim3(kSelectThreads), 0, st, x, s, l, h, cap, ctl, sp, iw, bucket_cnt);
}

}  // namespace lapsum
