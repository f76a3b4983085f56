// Localisation step of the bracketing path (Fast LapSum paper, gist.science
// summary section 2.2, bracketing step 1; the arxivdaily abstract names the
// same step: order statistics of a sample noised with the operator's kernel).
//
//  k_sample  x_j = r_{I_j} + eps_j, j < s: I_j uniform in [0, n) with
//            replacement, eps_j ~ Laplace(0, t) by inverse CDF.  Because the
//            noise is the operator's own kernel, P(x > b) = G(b)/n = k/n, so
//            b is the (1 - k/n) quantile of x whatever the scores are.
//            Random numbers: Philox4x32-10 (Salmon et al., SC'11), counter
//            (j_lo, j_hi, 0, 0), key (seed_lo, seed_hi).
//  k_select  one workgroup: a_L = x_(l), a_R = x_(h) by 8-bit MSD radix
//            select, then up to 1024 value-ordered buckets for the band:
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
// Fast path: sort a subsample of 1024 sample keys, read off a rank window
// that contains ranks l..h with a wide safety margin, count the sample keys
// below the window and collect the ones inside it, and sort only those
// (<= 4096).  The exact order statistics x_(l) .. x_(h) are then read from
// the sorted window.  If the window check fails (or the window is too wide)
// an 8-bit MSD radix select finds x_(l) and x_(h) instead.
// ---------------------------------------------------------------------------
constexpr int kWinMax = 4096;
constexpr int kSubMax = 1024;  // measured on gfx950: 1024 beats 2048 (C3, C4) and 512 (C4)

__global__ __launch_bounds__(kSelectThreads) void k_select(const float* __restrict__ x, int s, long long l, long long h,
                                                            int cap, Ctl* ctl, float* sp, float* iw,
                                                            uint32_t* bucket_cnt) {
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t sub[kSubMax > kCandMax ? kSubMax : kCandMax];  // the fallback's candidates too
    __shared__ uint32_t win[kWinMax];
    __shared__ uint32_t scr[kSelectThreads / 64 + 2];
    __shared__ uint32_t s_pre[2], s_rem[2];
    const int tid = threadIdx.x;
    // the sample, 16 bytes per load where it can (thread tid holds elements
    // i * kSelectThreads + tid)
    uint32_t kr[kSelectItems];
    unsigned long long vmask = 0ull;
    static_assert(kSelectItems % 4 == 0 && kSelectItems <= 64, "");
    if ((reinterpret_cast<uintptr_t>(x) & 15u) == 0u) {
        const float4* x4 = reinterpret_cast<const float4*>(x);
#pragma unroll
        for (int i = 0; i < kSelectItems; i += 4) {
            // float4 number (i/4)*kSelectThreads + tid: elements 4*that .. +3
            // (every use of kr treats it as an unordered set of the sample's
            // keys; vmask marks the slots that hold one)
            const int j4 = (i / 4) * kSelectThreads + tid;
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (4 * j4 + 3 < s) v = x4[j4];
            else {
                if (4 * j4 + 0 < s) v.x = x[4 * j4 + 0];
                if (4 * j4 + 1 < s) v.y = x[4 * j4 + 1];
                if (4 * j4 + 2 < s) v.z = x[4 * j4 + 2];
            }
            kr[i + 0] = f2key(v.x);
            kr[i + 1] = f2key(v.y);
            kr[i + 2] = f2key(v.z);
            kr[i + 3] = f2key(v.w);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * j4 + c < s) vmask |= 1ull << (i + c);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kSelectItems; ++i) {
            const int j = i * kSelectThreads + tid;
            kr[i] = j < s ? f2key(x[j]) : 0u;
            if (j < s) vmask |= 1ull << i;
        }
    }
    const bool want_l = l >= 1 && l <= s;
    const bool want_h = h >= 1 && h <= s;

    // ---- subsample and window ----
    // The sample values are independent draws, so any fixed subset of them is
    // a random subsample: thread i contributes its first key (sample value
    // 4i, already in its registers), for the first kSubMax threads.
    static_assert(kSubMax <= kSelectThreads, "one subsample key per thread");
    const int msub = (s + 3) / 4 < kSubMax ? (s + 3) / 4 : kSubMax;
    if (tid < kSubMax) sub[tid] = tid < msub ? kr[0] : 0xFFFFFFFFu;
    __syncthreads();
    sort_pow2_lds<kSelectThreads>(sub, kSubMax);
    // every thread reads the window ends off the sorted subsample (the sort
    // ends with a barrier)
    uint32_t wlo = 0u, whi = 0xFFFFFFFFu;
    if (want_l) {
        const double pl = (double)l / (double)s;
        const long long r0 = (long long)floor((double)msub * pl - 5.0 * sqrt((double)msub * pl * (1.0 - pl)) - 3.0);
        wlo = r0 < 0 ? 0u : sub[r0];
    }
    if (want_h) {
        const double ph = (double)h / (double)s;
        const long long r1 = (long long)ceil((double)msub * ph + 5.0 * sqrt((double)msub * ph * (1.0 - ph)) + 3.0);
        whi = r1 >= msub ? 0xFFFFFFFFu : sub[r1];
    }
    uint32_t nbelow = 0u, nin = 0u;
#pragma unroll
    for (int i = 0; i < kSelectItems; ++i) {
        if ((vmask >> i) & 1ull) { nbelow += kr[i] < wlo; nin += (kr[i] >= wlo && kr[i] <= whi); }
    }
    // one scan of both counts packed in a word (each total <= kSampleMax <
    // 2^16): the low half gives each thread its slot in the window, and every
    // thread gets both totals and takes the same decision
    static_assert(kSampleMax < 65536, "two 16-bit counts per word");
    uint32_t tot2 = 0u;
    uint32_t pos = block_exclusive_scan<kSelectThreads>(nin | (nbelow << 16), &tot2, scr) & 0xFFFFu;
    const uint32_t W = tot2 & 0xFFFFu;
    const long long nlo_all = (long long)(tot2 >> 16);
    const bool okl = !want_l || nlo_all <= l - 1;
    const bool okh = !want_h || nlo_all + (long long)W >= h;
    const bool fast = okl && okh && W >= 1 && W <= (uint32_t)kWinMax;

    uint32_t key_l = 0u, key_h = 0xFFFFFFFFu;
    const uint32_t* csorted;  // sorted sample keys from x_(l) (or the minimum) to x_(h) (or the maximum)
    int cc;
    if (fast) {
#pragma unroll
        for (int i = 0; i < kSelectItems; ++i) {
            if (((vmask >> i) & 1ull) && kr[i] >= wlo && kr[i] <= whi) win[pos++] = kr[i];
        }
        const int wp = max(next_pow2((int)W), 64);
        for (int e = (int)W + tid; e < wp; e += kSelectThreads) win[e] = 0xFFFFFFFFu;
        __syncthreads();
        sort_pow2_lds<kSelectThreads>(win, wp);
        const int i0 = want_l ? (int)(l - 1 - nlo_all) : 0;
        const int i1 = want_h ? (int)(h - 1 - nlo_all) : (int)W - 1;
        key_l = win[i0];
        key_h = win[i1];
        csorted = win + i0;
        cc = i1 - i0 + 1;
    } else {
        // ---- fallback: MSD radix select of ranks l and h ----
        if (tid == 0) {
            s_pre[0] = 0u; s_pre[1] = 0u;
            s_rem[0] = want_l ? (uint32_t)l : 1u;
            s_rem[1] = want_h ? (uint32_t)h : 1u;
        }
        for (int pass = 3; pass >= 0; --pass) {
            const int shift = 8 * pass;
            const uint32_t hmask = pass == 3 ? 0u : (0xFFFFFFFFu << (shift + 8));
            for (int e = tid; e < 512; e += kSelectThreads) (&hist[0][0])[e] = 0u;
            __syncthreads();
            const uint32_t p0 = s_pre[0], p1 = s_pre[1];
#pragma unroll
            for (int i = 0; i < kSelectItems; ++i) {
                if ((vmask >> i) & 1ull) {
                    const uint32_t kk = kr[i];
                    const uint32_t d = (kk >> shift) & 0xFFu;
                    if ((kk & hmask) == (p0 & hmask)) atomicAdd(&hist[0][d], 1u);
                    if ((kk & hmask) == (p1 & hmask)) atomicAdd(&hist[1][d], 1u);
                }
            }
            __syncthreads();
            if (tid == 0 || tid == 64) {
                const int qq = tid == 0 ? 0 : 1;
                uint32_t rem = s_rem[qq], cum = 0u;
                int d = 0;
                for (; d < 255; ++d) {
                    const uint32_t c = hist[qq][d];
                    if (cum + c >= rem) break;
                    cum += c;
                }
                s_pre[qq] |= (uint32_t)d << shift;
                s_rem[qq] = rem - cum;
            }
            __syncthreads();
        }
        key_l = want_l ? s_pre[0] : 0u;
        key_h = want_h ? s_pre[1] : 0xFFFFFFFFu;
        // candidates for splitters: sample keys in [key_l, key_h], thinned in sample order
        uint32_t mine = 0u;
#pragma unroll
        for (int i = 0; i < kSelectItems; ++i) {
            if (((vmask >> i) & 1ull) && kr[i] >= key_l && kr[i] <= key_h) ++mine;
        }
        uint32_t total = 0u;
        uint32_t cpos = block_exclusive_scan<kSelectThreads>(mine, &total, scr);
        const uint32_t stride = (total + kCandMax - 1) / kCandMax > 0 ? (total + kCandMax - 1) / kCandMax : 1u;
#pragma unroll
        for (int i = 0; i < kSelectItems; ++i) {
            if (((vmask >> i) & 1ull) && kr[i] >= key_l && kr[i] <= key_h) {
                if (cpos % stride == 0u) sub[cpos / stride] = kr[i];
                ++cpos;
            }
        }
        cc = (int)((total + stride - 1) / stride);
        __syncthreads();
        for (int e = cc + tid; e < kCandMax; e += kSelectThreads) sub[e] = 0xFFFFFFFFu;
        __syncthreads();
        sort_pow2_lds<kSelectThreads>(sub, kCandMax);
        csorted = sub;
        if (cc < 1) cc = 1;
    }
    const float aL = want_l ? key2f(key_l) : -INFINITY;
    const float aR = want_h ? key2f(key_h) : INFINITY;

    // gaps: ng <= kMaxBuckets, interior splitters evenly spaced over the sorted candidates
    const int ng = cc >= 2 ? (cc - 1 < kMaxBuckets ? cc - 1 : kMaxBuckets) : 1;
    const int J = kMaxBuckets / ng > 0 ? kMaxBuckets / ng : 1;
    for (int g = tid; g <= ng; g += kSelectThreads) {
        float v;
        if (g == 0) v = aL;
        else if (g == ng) v = aR;
        else v = key2f(csorted[(int)(((long long)g * (cc - 1)) / ng)]);
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
        ctl->pad0 = fast ? 1 : 0;
    }
}

void launch_select(const float* x, int s, long long l, long long h, int cap, Ctl* ctl, float* sp, float* iw,
                   uint32_t* bucket_cnt, hipStream_t st) {
    hipLaunchKernelGGL(k_select, dim3(1), dim3(kSelectThreads), 0, st, x, s, l, h, cap, ctl, sp, iw, bucket_cnt);
}

}  // namespace lapsum
