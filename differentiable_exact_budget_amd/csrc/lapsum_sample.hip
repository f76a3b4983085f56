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
//  k_select  one workgroup: a_L = x_(l), a_R = x_(h), exactly: a window
//            of sample ranks around l..h from two order statistics of a
//            1024-key subsample (radix select), the sample keys inside it
//            sorted and the two read off (an 8-bit MSD radix select over
//            the whole sample when the window misses); then up to 1024
//            value-ordered buckets for the band: sample values between a_L
//            and a_R as gap splitters, each finite gap cut into J
//            equal-width sub-buckets.
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

constexpr int kSampleThreads = 512;  // measured on gfx950: sample + select 1-2 us below 256 or 1024 threads

// The workgroup's sample keys into the sample histogram (hist: leading 12
// bits of each key, kSelHistBins words): counted in LDS first, so that a bin
// the whole workgroup hits (tied or clustered scores) takes one global add
// per workgroup; the adds are integer, so the totals do not depend on their
// order.  hclr (may be null) is cleared by the grid.  Every thread calls it.
LS_DEV void sample_hist_block(uint32_t key, bool valid, uint32_t* lh, uint32_t* hist, uint32_t* hclr) {
    const int tid = threadIdx.x;
    if (hclr)
        for (int i = blockIdx.x * kSampleThreads + tid; i < kSelHistBins; i += gridDim.x * kSampleThreads) hclr[i] = 0u;
    for (int i = tid; i < kSelHistBins; i += kSampleThreads) lh[i] = 0u;
    __syncthreads();
    if (valid) atomicAdd(&lh[key >> kSelHistShift], 1u);
    __syncthreads();
    for (int i = tid; i < kSelHistBins; i += kSampleThreads) {
        const uint32_t c = lh[i];
        if (c) atomicAdd(&hist[i], c);
    }
}

__global__ __launch_bounds__(kSampleThreads) void k_sample(const float* __restrict__ r, long long n, double t,
                                                           unsigned long long seed, int s, float* __restrict__ x,
                                                           long long* idx_out, uint32_t* hist, uint32_t* hclr) {
    __shared__ uint32_t lh[kSelHistBins];
    const int j = blockIdx.x * kSampleThreads + threadIdx.x;
    const bool valid = j < s;
    float xv = 0.0f;
    if (valid) {
        uint32_t c[4] = {(uint32_t)j, 0u, 0u, 0u};
        philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
        const unsigned long long u64 = ((unsigned long long)c[1] << 32) | c[0];
        const long long idx = (long long)__umul64hi(u64, (unsigned long long)n);
        const unsigned long long m53 = ((((unsigned long long)c[3]) << 32) | c[2]) >> 11;
        const double u = ((double)m53 + 0.5) * 0x1p-53;
        const double eps = (u < 0.5) ? t * log(2.0 * u) : -t * log(2.0 * (1.0 - u));
        xv = (float)((double)r[idx] + eps);
        x[j] = xv;
        if (idx_out) idx_out[j] = idx;
    }
    if (hist) sample_hist_block(f2key(xv), valid, lh, hist, hclr);  // hist is uniform
}

__global__ __launch_bounds__(kSampleThreads) void k_key_hist(const float* __restrict__ x, int s, uint32_t* hist,
                                                             uint32_t* hclr) {
    __shared__ uint32_t lh[kSelHistBins];
    const int j = blockIdx.x * kSampleThreads + threadIdx.x;
    const bool valid = j < s;
    sample_hist_block(valid ? f2key(x[j]) : 0u, valid, lh, hist, hclr);
}

void launch_sample(const float* r, long long n, double t, unsigned long long seed, int s, float* x, long long* idx_out,
                   hipStream_t st, uint32_t* hist, uint32_t* hclr) {
    hipLaunchKernelGGL(k_sample, dim3((s + kSampleThreads - 1) / kSampleThreads), dim3(kSampleThreads), 0, st, r, n,
                       t, seed, s, x, idx_out, hist, hist ? hclr : nullptr);
}

void launch_key_hist(const float* x, int s, uint32_t* hist, uint32_t* hclr, hipStream_t st) {
    hipLaunchKernelGGL(k_key_hist, dim3((s + kSampleThreads - 1) / kSampleThreads), dim3(kSampleThreads), 0, st, x,
                       s, hist, hclr);
}

// ---------------------------------------------------------------------------
// select
// x_(l) .. x_(h) are read from a sorted window of sample keys: the keys
// whose leading 12 bits lie between those of x_(l) and x_(h), which the
// sample histogram names exactly (the bins holding ranks l and h, and the
// count below them).  When the histogram is there and that window holds at
// most kWinMax keys, many workgroups gather it (k_select_window) and the
// select sorts only those keys.  Otherwise the select takes the whole sample
// itself: two order statistics of a subsample of 1024 sample keys give a
// rank window that contains ranks l..h with a wide safety margin; count the
// sample keys below the window, collect the ones inside it, and sort those
// (<= kWinMax).  If that window check fails too an 8-bit MSD radix select
// finds x_(l) and x_(h).
// ---------------------------------------------------------------------------
constexpr int kWinThreads = 256;
constexpr int kWinKeys = 4;  // sample keys per thread of k_select_window

// One workgroup per kWinThreads * kWinKeys sample keys: every workgroup
// scans the histogram (the same result in each), and appends its keys inside
// the window to the window buffer, each wave at a place taken with one
// atomic add.  Workgroup 0 writes the header (ok, window size, keys below
// it); the fill count starts at zero and k_select sets it back to zero.
__global__ __launch_bounds__(kWinThreads) void k_select_window(const float* __restrict__ x, int s, long long l,
                                                               long long h, const uint32_t* __restrict__ hist,
                                                               uint32_t* win) {
    constexpr int NT = kWinThreads, BPT = kSelHistBins / NT;
    static_assert(BPT % 4 == 0, "");
    __shared__ uint32_t scr[NT / 64 + 2];
    __shared__ uint32_t s_res[4];  // bin of rank l, keys below it; bin of rank h, keys up to its end
    const int tid = threadIdx.x;
    uint32_t kk[kWinKeys];
    bool kv[kWinKeys];
#pragma unroll
    for (int q = 0; q < kWinKeys; ++q) {
        const long long e = (long long)blockIdx.x * NT * kWinKeys + q * NT + tid;
        kv[q] = e < s;
        kk[q] = kv[q] ? f2key(x[e]) : 0u;
    }
    uint32_t hb[BPT];  // bins BPT * tid .. BPT * tid + BPT - 1
    const uint4* h4 = reinterpret_cast<const uint4*>(hist) + tid * (BPT / 4);
#pragma unroll
    for (int q = 0; q < BPT / 4; ++q) {
        const uint4 v = h4[q];
        hb[4 * q] = v.x; hb[4 * q + 1] = v.y; hb[4 * q + 2] = v.z; hb[4 * q + 3] = v.w;
    }
    uint32_t sum = 0u;
#pragma unroll
    for (int b = 0; b < BPT; ++b) sum += hb[b];
    if (tid == 0) { s_res[0] = 0u; s_res[1] = 0u; s_res[2] = kSelHistBins - 1; s_res[3] = 0u; }
    uint32_t tot = 0u;
    uint32_t c = block_exclusive_scan<NT>(sum, &tot, scr);
    const bool want_l = l >= 1 && l <= s, want_h = h >= 1 && h <= s;
    const uint32_t ql = want_l ? (uint32_t)(l - 1) : 0u, qh = want_h ? (uint32_t)(h - 1) : 0u;  // 0-based ranks
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        const uint32_t cnt = hb[b];
        if (want_l && c <= ql && ql - c < cnt) { s_res[0] = (uint32_t)(BPT * tid + b); s_res[1] = c; }
        if (want_h && c <= qh && qh - c < cnt) { s_res[2] = (uint32_t)(BPT * tid + b); s_res[3] = c + cnt; }
        c += cnt;
    }
    __syncthreads();
    const uint32_t binl = s_res[0], nlo = s_res[1], binh = s_res[2];
    const uint32_t hend = want_h ? s_res[3] : tot;
    const uint32_t W = hend - nlo;
    const bool ok = tot == (uint32_t)s && hend >= nlo && binh >= binl && W >= 1u && W <= (uint32_t)kWinMax;
    if (blockIdx.x == 0 && tid == 0) { win[1] = ok ? 1u : 0u; win[2] = W; win[3] = nlo; }
    if (!ok) return;  // uniform
    // key in the window: wlo <= key <= wlo + wspan (one unsigned compare;
    // a window over all 4096 bins gives wspan = 2^32 - 1)
    const uint32_t wlo = binl << kSelHistShift;
    const uint32_t wspan = ((binh - binl + 1u) << kSelHistShift) - 1u;
    uint32_t m = 0u;
#pragma unroll
    for (int q = 0; q < kWinKeys; ++q) m += (kv[q] && kk[q] - wlo <= wspan) ? 1u : 0u;
    // a place per wave (no barrier): the wave's scan, one atomic add by its
    // last lane, the base to every lane
    const uint32_t inc = wave_inclusive_scan(m);
    uint32_t base = 0u;
    if (lane_id() == 63 && inc) base = atomicAdd(&win[0], inc);
    uint32_t pos = __shfl(base, 63, 64) + inc - m;
#pragma unroll
    for (int q = 0; q < kWinKeys; ++q) {
        if (kv[q] && kk[q] - wlo <= wspan) {
            if (pos < (uint32_t)kWinMax) win[kWinHdr + pos] = kk[q];
            ++pos;
        }
    }
}

// The leading DIGITS 8-bit digits of the keys of two ranks (0-based,
// ascending) among the keys the NT threads hold, at most one each (has), by
// MSD radix select: per digit, a histogram of the keys that share each
// target's prefix so far (LDS adds into four copies picked by lane), then one
// wave per target finds the digit holding its rank.  want[q] = false skips
// target q.  out[q] is the prefix with the remaining low bits zero: the
// target key lies in [out[q], out[q] | (2^(32 - 8 DIGITS) - 1)].  The result
// is in every thread.  h: 2 * 4 * 256 words; st: 4 words.
template <int NT, int DIGITS>
LS_DEV void block_select2(uint32_t key, bool has, const uint32_t rank[2], const bool want[2], uint32_t out[2],
                          uint32_t* h, uint32_t* st) {
    static_assert(DIGITS >= 1 && DIGITS <= 4, "");
    const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
    if (tid < 2) { st[tid] = 0u; st[2 + tid] = rank[tid]; }  // prefix, rank left inside it
    for (int pass = 3; pass >= 4 - DIGITS; --pass) {
        const int shift = 8 * pass;
        const uint32_t hmask = pass == 3 ? 0u : (0xFFFFFFFFu << (shift + 8));
        for (int e = tid; e < 2 * 4 * 256; e += NT) h[e] = 0u;
        __syncthreads();
        const uint32_t d = (key >> shift) & 0xFFu;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            if (want[q] && has && (key & hmask) == (st[q] & hmask)) atomicAdd(&h[(q * 4 + (lane & 3)) * 256 + d], 1u);
        __syncthreads();
        if (wv < 2 && want[wv]) {  // wave q: lane l sums digits 4l .. 4l + 3
            const int q = wv;
            uint32_t c[4], sum = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dd = 4 * lane + j;
                c[j] = h[(q * 4 + 0) * 256 + dd] + h[(q * 4 + 1) * 256 + dd] + h[(q * 4 + 2) * 256 + dd] +
                       h[(q * 4 + 3) * 256 + dd];
                sum += c[j];
            }
            const uint32_t inc = wave_inclusive_scan(sum);
            const uint32_t rem = st[2 + q];
            uint32_t below = inc - sum;
            if (below <= rem && rem < inc) {  // the one lane holding the rank
                int j = 0;
                while (j < 3 && below + c[j] <= rem) below += c[j++];
                st[q] |= (uint32_t)(4 * lane + j) << shift;
                st[2 + q] = rem - below;
            }
        }
        __syncthreads();
    }
    out[0] = st[0];
    out[1] = st[1];
    __syncthreads();
}

constexpr int kSubMax = 1024;  // measured on gfx950: 1024 beats 2048 (C3, C4) and 512 (C4)

// wg (may be null): the window buffer k_select_window filled
__global__ __launch_bounds__(kSelectThreads) void k_select(const float* __restrict__ x, int s, long long l, long long h,
                                                            int cap, Ctl* ctl, float* sp, float* iw,
                                                            uint32_t* bucket_cnt, uint32_t* wg) {
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t sub[kSubMax > kCandMax ? kSubMax : kCandMax];  // the fallback's candidates too
    __shared__ uint32_t win[kWinMax];
    __shared__ uint32_t scr[kSelectThreads / 64 + 2];
    __shared__ uint32_t s_pre[2], s_rem[2];
    __shared__ uint32_t s_selh[2 * 4 * 256];  // the subsample's radix select
    __shared__ uint32_t s_selst[4];
    const int tid = threadIdx.x;
    const bool want_l = l >= 1 && l <= s;
    const bool want_h = h >= 1 && h <= s;
    uint32_t key_l = 0u, key_h = 0xFFFFFFFFu;
    const uint32_t* csorted;  // sorted sample keys from x_(l) (or the minimum) to x_(h) (or the maximum)
    int cc;
    int how;  // 2: gathered window, 1: own window, 0: radix select
    // the gathered window, if k_select_window found one (the same header in
    // every thread; its fill count must match the size the histogram gave)
    uint32_t gW = 0u, gnlo = 0u;
    bool gathered = false;
    if (wg) {
        const uint32_t fill = wg[0], ok = wg[1];
        gW = wg[2];
        gnlo = wg[3];
        gathered = ok != 0u && fill == gW && gW >= 1u && gW <= (uint32_t)kWinMax;
    }
    if (gathered) {
        const int W = (int)gW;
        const int wp = max(next_pow2(W), 64);
        for (int e = tid; e < wp; e += kSelectThreads) win[e] = e < W ? wg[kWinHdr + e] : 0xFFFFFFFFu;
        __syncthreads();
        sort_pow2_lds<kSelectThreads>(win, wp);
        const int i0 = want_l ? (int)(l - 1 - (long long)gnlo) : 0;
        const int i1 = want_h ? (int)(h - 1 - (long long)gnlo) : W - 1;
        key_l = win[i0];
        key_h = win[i1];
        csorted = win + i0;
        cc = i1 - i0 + 1;
        how = 2;
    } else {
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

        // ---- subsample and window ----
        // The sample values are independent draws, so any fixed subset of them is
        // a random subsample: thread i contributes its first key (sample value
        // 4i, already in its registers), for the first kSubMax threads.
        // The window ends are two order statistics of the subsample, found by a
        // radix select (two ranks need no full sort) to their leading 16 bits:
        // the window runs from the low end of the lower one's 16-bit bin to the
        // high end of the upper one's, a bin of relative width 2^-7 at most on
        // each side (measured on gfx950: two digits in place of four, select
        // -2 us at the 10^7 and 10^8 workloads).
        static_assert(kSubMax <= kSelectThreads, "one subsample key per thread");
        const int msub = (s + 3) / 4 < kSubMax ? (s + 3) / 4 : kSubMax;
        long long r0 = -1, r1 = msub;
        if (want_l) {
            const double pl = (double)l / (double)s;
            r0 = (long long)floor((double)msub * pl - 5.0 * sqrt((double)msub * pl * (1.0 - pl)) - 3.0);
        }
        if (want_h) {
            const double ph = (double)h / (double)s;
            r1 = (long long)ceil((double)msub * ph + 5.0 * sqrt((double)msub * ph * (1.0 - ph)) + 3.0);
        }
        const bool sel[2] = {r0 >= 0 && r0 < msub, r1 >= 0 && r1 < msub};
        const uint32_t rk2[2] = {sel[0] ? (uint32_t)r0 : 0u, sel[1] ? (uint32_t)r1 : 0u};
        uint32_t wend[2];
        block_select2<kSelectThreads, 2>(kr[0], tid < msub, rk2, sel, wend, s_selh, s_selst);
        const uint32_t wlo = r0 < 0 ? 0u : (sel[0] ? wend[0] : 0xFFFFFFFFu);
        const uint32_t whi = r1 >= msub ? 0xFFFFFFFFu : (wend[1] | 0xFFFFu);
        // Per key: below the window, or inside it (wlo <= k <= whi as one
        // unsigned compare).  Groups of four keys past the sample's end are
        // skipped, and only the group that straddles it tests vmask (uniform).
        const uint32_t wspan = whi - wlo;
        uint32_t nbelow = 0u, nin = 0u;
#pragma unroll
        for (int i = 0; i < kSelectItems; ++i) {
            if ((i & 3) == 0 && (i / 4) * 4 * kSelectThreads >= s) break;
            const bool v = (i / 4 + 1) * 4 * kSelectThreads <= s || ((vmask >> i) & 1ull);
            nbelow += (v && kr[i] < wlo) ? 1u : 0u;
            nin += (v && kr[i] - wlo <= wspan) ? 1u : 0u;
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

        how = fast ? 1 : 0;
        if (fast) {
#pragma unroll
            for (int i = 0; i < kSelectItems; ++i) {
                if ((i & 3) == 0 && (i / 4) * 4 * kSelectThreads >= s) break;
                const bool v = (i / 4 + 1) * 4 * kSelectThreads <= s || ((vmask >> i) & 1ull);
                if (v && kr[i] - wlo <= wspan) win[pos++] = kr[i];
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
        ctl->pad0 = how;
        if (wg) wg[0] = 0u;  // the window's fill count, for the next gather
    }
}

void launch_select(const float* x, int s, long long l, long long h, int cap, Ctl* ctl, float* sp, float* iw,
                   uint32_t* bucket_cnt, hipStream_t st, const uint32_t* hist, uint32_t* win) {
    if (hist && win) {
        const int wgs = (s + kWinThreads * kWinKeys - 1) / (kWinThreads * kWinKeys);
        hipLaunchKernelGGL(k_select_window, dim3(wgs), dim3(kWinThreads), 0, st, x, s, l, h, hist, win);
    }
    hipLaunchKernelGGL(k_select, dim3(1), dim3(kSelectThreads), 0, st, x, s, l, h, cap, ctl, sp, iw, bucket_cnt,
                       hist ? win : nullptr);
}

}  // namespace lapsum
