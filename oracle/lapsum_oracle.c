/*
 * Reference oracle for the exact-budget LapSum soft top-k (CPU, fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two meet only through seeded inputs.
 *
 * What it computes, and where the definition comes from (the pages are the
 * paper Fast LapSum: Exact Differentiable Top-k at Million Scale as
 * summarised on gist.science, section 2.1 on the LapSum operator, and the
 * arxivdaily abstract of the same paper):
 *
 *   F(x) = Laplace CDF with scale 1:  F(x) = e^x / 2 for x < 0,
 *                                      F(x) = 1 - e^-x / 2 for x >= 0.
 *   p_i  = F((r_i - b) / t)           (perturbed score r_i + eps, eps ~
 *                                      Laplace(0, t), exceeds threshold b)
 *   b    = the unique root of G(b) = sum_i F((r_i - b)/t) = k
 *                                     (the budget constraint sum p = k).
 *   VJP  : dp_i/dr_j = (f_i/t)(delta_ij - f_j / sum f), with f_i the Laplace
 *          density 0.5 e^{-|r_i - b|/t}; hence for an upstream g
 *          grad_j = (f_j/t) (g_j - sum_i g_i f_i / sum_i f_i).
 *          (Derived by implicit differentiation of the budget constraint:
 *           dG/db = -sum f / t, dp_i/dr_j|_b = f_i/t delta_ij.)
 *
 * The method on the pages reaches this b exactly (closed-form root after a
 * sort, optionally with probabilistic bracketing and certification), so the
 * oracle is the plain definition: b is found by bisection on G to fp64
 * exhaustion.  This is the "per-query bisection" style the pages contrast
 * the fast solver against (gist.science section 2.2 and 4.1).
 *
 * Summation: Neumaier-compensated, over a fixed partition of [0, n) into
 * contiguous chunks whose partial sums are combined in chunk order, so a
 * result does not depend on the number of threads.
 *
 * Pins (tests/test_oracle_*.py): brute-force interval enumeration for
 * n <= 16 at 50-digit precision, closed forms (all-equal scores, n = 1),
 * the t -> 0 limit (midpoint of order statistics k and k+1, i.e. hard top-k),
 * invariants (sum p = k, monotone p, shift/scale equivariance), central
 * finite differences and Jacobian symmetry of the VJP, Philox known-answer
 * vectors, exact binomial sums at small s.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MIN_CHUNK 8192
#define ORACLE_MAX_CHUNKS 512

/* ------------------------------------------------------------------ */
/* threads                                                             */
/* ------------------------------------------------------------------ */
static int g_threads = 0; /* 0: OpenMP default */

void oracle_set_threads(int nthreads) { g_threads = nthreads; }

int oracle_get_threads(void) {
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Laplace CDF and density (scale 1)                                   */
/* ------------------------------------------------------------------ */
static double lap_cdf(double x) { return x < 0.0 ? 0.5 * exp(x) : 1.0 - 0.5 * exp(-x); }
static double lap_pdf(double x) { return 0.5 * exp(-fabs(x)); }

/* ------------------------------------------------------------------ */
/* Neumaier summation                                                  */
/* ------------------------------------------------------------------ */
typedef struct { double s, c; } nsum_t;

static void nadd(nsum_t* a, double x) {
    double t = a->s + x;
    if (fabs(a->s) >= fabs(x)) a->c += (a->s - t) + x;
    else a->c += (x - t) + a->s;
    a->s = t;
}
static double nval(const nsum_t* a) { return a->s + a->c; }

/* fixed chunking, independent of thread count */
static int64_t nchunks_for(int64_t n) {
    int64_t c = (n + ORACLE_MIN_CHUNK - 1) / ORACLE_MIN_CHUNK;
    if (c < 1) c = 1;
    if (c > ORACLE_MAX_CHUNKS) c = ORACLE_MAX_CHUNKS;
    return c;
}
static int64_t chunk_lo(int64_t n, int64_t nc, int64_t c) { return (n / nc) * c + (c < n % nc ? c : n % nc); }

/*
 * Generic chunked reduction of up to 4 per-element terms.
 * kind selects the terms (see the switch in term_eval).
 */
enum { T_G = 0, T_PROBS = 1, T_VJP = 2, T_BRACKET = 3, T_VJP_KT = 4 };

typedef struct {
    const double* r; const double* g; double* out; double t, b, aL, aR;
} red_args_t;

static void term_eval(int kind, const red_args_t* a, int64_t i, double v[4], int64_t cnt[3]) {
    double ri = a->r[i];
    switch (kind) {
    case T_G: {
        /* F(x) split into its integer part and its small part:
         * x < 0: 0 + e^x/2;  x >= 0: 1 - e^-x/2.  Counting the ones exactly
         * keeps the e^-x/2 terms that fp64 would round away next to 1. */
        double x = (ri - a->b) / a->t;
        if (x < 0.0) v[0] = exp(x); else { cnt[0]++; v[1] = exp(-x); }
        break; }
    case T_PROBS: {
        double x = (ri - a->b) / a->t;
        double p = lap_cdf(x);
        if (a->out) a->out[i] = p;
        if (x < 0.0) v[0] = exp(x); else { cnt[0]++; v[1] = exp(-x); }
        break; }
    case T_VJP: {
        double f = lap_pdf((ri - a->b) / a->t);
        v[0] = f * a->g[i]; v[1] = f; break; }
    case T_VJP_KT: {
        double d = ri - a->b;
        double f = lap_pdf(d / a->t);
        v[0] = f * a->g[i]; v[1] = f; v[2] = f * a->g[i] * d; v[3] = f * d; break; }
    case T_BRACKET: {
        /* band is a_L <= r < a_R; below r < a_L; above r >= a_R (gist.science 2.2 step 2) */
        if (ri < a->aL) { cnt[0]++; v[0] = exp((ri - a->aL) / a->t); }
        else if (ri >= a->aR) { cnt[2]++; v[1] = exp((a->aR - ri) / a->t); }
        else {
            cnt[1]++;
            v[2] = isinf(a->aL) ? 0.0 : exp((a->aL - ri) / a->t);
            v[3] = isinf(a->aR) ? 0.0 : exp((ri - a->aR) / a->t);
        }
        break; }
    }
}

static void reduce(int kind, const red_args_t* a, int64_t n, double res[4], int64_t cnt_out[3]) {
    int64_t nc = nchunks_for(n);
    nsum_t* parts = (nsum_t*)calloc((size_t)nc * 4, sizeof(nsum_t));
    int64_t* cparts = (int64_t*)calloc((size_t)nc * 3, sizeof(int64_t));
#ifdef _OPENMP
    int nt = oracle_get_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int64_t c = 0; c < nc; ++c) {
        int64_t lo = chunk_lo(n, nc, c), hi = chunk_lo(n, nc, c + 1);
        nsum_t s[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
        int64_t cnt[3] = {0, 0, 0};
        for (int64_t i = lo; i < hi; ++i) {
            double v[4] = {0, 0, 0, 0};
            term_eval(kind, a, i, v, cnt);
            for (int q = 0; q < 4; ++q) if (v[q] != 0.0) nadd(&s[q], v[q]);
        }
        for (int q = 0; q < 4; ++q) parts[c * 4 + q] = s[q];
        for (int q = 0; q < 3; ++q) cparts[c * 3 + q] = cnt[q];
    }
    nsum_t tot[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    int64_t ct[3] = {0, 0, 0};
    for (int64_t c = 0; c < nc; ++c) {
        for (int q = 0; q < 4; ++q) { nadd(&tot[q], parts[c * 4 + q].s); nadd(&tot[q], parts[c * 4 + q].c); }
        for (int q = 0; q < 3; ++q) ct[q] += cparts[c * 3 + q];
    }
    for (int q = 0; q < 4; ++q) res[q] = nval(&tot[q]);
    if (cnt_out) for (int q = 0; q < 3; ++q) cnt_out[q] = ct[q];
    free(parts); free(cparts);
}

/* ------------------------------------------------------------------ */
/* G(b) = sum_i F((r_i - b)/t)       (gist.science 2.1, budget sum)    */
/* ------------------------------------------------------------------ */
double oracle_budget_G(const double* r, int64_t n, double t, double b) {
    if (isinf(b)) return b < 0 ? (double)n : 0.0;
    red_args_t a = {r, NULL, NULL, t, b, 0, 0};
    double res[4];
    int64_t cnt[3];
    reduce(T_G, &a, n, res, cnt);
    return (double)cnt[0] + 0.5 * (res[0] - res[1]);
}

/* G(b) - k, evaluated as (#{r_i >= b} - k) + (sum_{r<b} e^x - sum_{r>=b} e^-x)/2
 * so that its sign is right even when every term is within an ulp of 0 or 1. */
double oracle_budget_excess(const double* r, int64_t n, double t, double b, double k) {
    red_args_t a = {r, NULL, NULL, t, b, 0, 0};
    double res[4];
    int64_t cnt[3];
    reduce(T_G, &a, n, res, cnt);
    return ((double)cnt[0] - k) + 0.5 * (res[0] - res[1]);
}

/*
 * Root of G(b) = k by bisection.  G is continuous and strictly decreasing
 * from n to 0, so for 0 < k < n the root is unique (gist.science 2.1).
 * Initial bracket: lo = min r - t (max(0, ln(n / (2(n-k)))) + 1) has every
 * term F >= 1 - (n-k)/(e n) > k/n (or >= 0.82 > k/n when k < n/2), hence
 * G(lo) > k; symmetrically G(hi) < k for hi = max r + t (max(0, ln(n/(2k))) + 1).
 * Each step keeps the half whose ends have G - k of opposite sign (G - k
 * from oracle_budget_excess).  Iterates until the midpoint no longer moves or
 * the bracket is below 1e-15 max(1, |mid|).  Returns 0 on success, -1 on invalid arguments.
 */
int oracle_solve(const double* r, int64_t n, double k, double t, double* b_out, int* iters_out) {
    if (n < 1 || !(k > 0.0) || !(k < (double)n) || !(t > 0.0) || !isfinite(t)) return -1;
    double mn = r[0], mx = r[0];
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(r[i])) return -1;
        if (r[i] < mn) mn = r[i];
        if (r[i] > mx) mx = r[i];
    }
    double nn = (double)n;
    double lo = mn - t * (fmax(0.0, log(nn / (2.0 * (nn - k)))) + 1.0);
    double hi = mx + t * (fmax(0.0, log(nn / (2.0 * k))) + 1.0);
    int it = 0;
    for (;;) {
        double mid = lo + 0.5 * (hi - lo);
        if (!(mid > lo) || !(mid < hi)) break;
        if (oracle_budget_excess(r, n, t, mid, k) >= 0.0) lo = mid; else hi = mid;
        ++it;
        if (hi - lo <= 1e-15 * fmax(1.0, fabs(mid))) break;
        if (it > 400) break;
    }
    *b_out = lo + 0.5 * (hi - lo);
    if (iters_out) *iters_out = it;
    return 0;
}

/* p_i = F((r_i - b)/t) and sum p (gist.science 2.1); sum p uses the same
 * integer/small-part split as G. */
double oracle_probs(const double* r, int64_t n, double t, double b, double* p_out) {
    red_args_t a = {r, NULL, p_out, t, b, 0, 0};
    double res[4];
    int64_t cnt[3];
    reduce(T_PROBS, &a, n, res, cnt);
    return (double)cnt[0] + 0.5 * (res[0] - res[1]);
}

/*
 * Analytic VJP (gist.science 2.1: backward is a vector-Jacobian product).
 * grad_j = (f_j / t) (g_j - c),  c = sum g f / sum f,  f_j = 0.5 e^{-|r_j-b|/t}.
 * Writes c to *c_out (may be NULL) and sum f to *sumf_out (may be NULL).
 */
void oracle_vjp(const double* r, const double* g, int64_t n, double t, double b,
                double* grad_out, double* c_out, double* sumf_out) {
    red_args_t a = {r, g, NULL, t, b, 0, 0};
    double res[4];
    reduce(T_VJP, &a, n, res, NULL);
    double c = res[0] / res[1];
    for (int64_t i = 0; i < n; ++i) {
        double f = lap_pdf((r[i] - b) / t);
        grad_out[i] = (f / t) * (g[i] - c);
    }
    if (c_out) *c_out = c;
    if (sumf_out) *sumf_out = res[1];
}

/*
 * Gradients of L = sum_i g_i p_i with respect to the budget k and the
 * temperature t, through the threshold b(k, t) that G(b) = k fixes
 * (gist.science 2.1; implicit differentiation of the budget equation).
 * With d_i = r_i - b and f_i = 0.5 e^{-|d_i|/t}, dp_i/dx_i = f_i for
 * x_i = d_i / t, and differentiating sum_i F(d_i / t) = k gives
 *   db/dk = -t / sum f,        so dL/dk = sum g f / sum f;
 *   db/dt = -mu,  mu = sum f d / sum f,
 *                              so dL/dt = -(sum g f d - mu sum g f) / t^2.
 */
void oracle_vjp_kt(const double* r, const double* g, int64_t n, double t, double b,
                   double* dk_out, double* dt_out) {
    red_args_t a = {r, g, NULL, t, b, 0, 0};
    double res[4];
    reduce(T_VJP_KT, &a, n, res, NULL);
    const double mu = res[3] / res[1];
    if (dk_out) *dk_out = res[0] / res[1];
    if (dt_out) *dt_out = -(res[2] - mu * res[0]) / (t * t);
}

/*
 * Bracket bookkeeping for a given [a_L, a_R) (gist.science 2.2, streaming
 * and filtering): counts below / in band / above, the tail sums
 *   S_L = sum_{r < a_L} e^{(r - a_L)/t},   S_R = sum_{r >= a_R} e^{(a_R - r)/t},
 * the band sums  B_L = sum_band e^{(a_L - v)/t},  B_R = sum_band e^{(v - a_R)/t},
 * the direct G(a_L), G(a_R) (the certification quantities), and the band
 * values themselves in ascending order (written to band_out when it is not
 * NULL and band_cap is large enough).
 * sums_out: {S_L, S_R, B_L, B_R, G(a_L), G(a_R)}.  counts_out: {below, band, above}.
 * Returns the band size, or -1 when band_out is given and too small.
 */
static int cmp_double(const void* x, const void* y) {
    double a = *(const double*)x, b = *(const double*)y;
    return (a > b) - (a < b);
}

int64_t oracle_bracket(const double* r, int64_t n, double t, double aL, double aR,
                       int64_t counts_out[3], double sums_out[6], double* band_out, int64_t band_cap) {
    red_args_t a = {r, NULL, NULL, t, 0.0, aL, aR};
    double res[4];
    int64_t cnt[3];
    reduce(T_BRACKET, &a, n, res, cnt);
    for (int q = 0; q < 3; ++q) counts_out[q] = cnt[q];
    for (int q = 0; q < 4; ++q) sums_out[q] = res[q];
    sums_out[4] = oracle_budget_G(r, n, t, aL);
    sums_out[5] = oracle_budget_G(r, n, t, aR);
    if (band_out) {
        if (cnt[1] > band_cap) return -1;
        int64_t m = 0;
        for (int64_t i = 0; i < n; ++i)
            if (r[i] >= aL && r[i] < aR) band_out[m++] = r[i];
        qsort(band_out, (size_t)m, sizeof(double), cmp_double);
    }
    return cnt[1];
}

/* ------------------------------------------------------------------ */
/* Sorted keys: ascending fp32 order with -0.0 canonicalised to +0.0   */
/* ------------------------------------------------------------------ */
static int cmp_float(const void* x, const void* y) {
    float a = *(const float*)x, b = *(const float*)y;
    return (a > b) - (a < b);
}

void oracle_sort_keys(const float* r, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (r[i] == 0.0f) ? 0.0f : r[i];
    qsort(out, (size_t)n, sizeof(float), cmp_float);
}

/* ------------------------------------------------------------------ */
/* Order statistics from the top, the hard top-k threshold and the      */
/* DFTopK operator (gist.science summary 2.3: DFTopK puts the threshold */
/* at the midpoint of the k-th and (k+1)-th order statistics, which is */
/* the zero-temperature limit of LapSum; at finite t its mass sum p     */
/* drifts from k).                                                      */
/* ------------------------------------------------------------------ */

/* k-th and (k+1)-th largest of r (1 <= k <= n; the (k+1)-th is -inf when
 * k = n), from a sorted copy.  Returns 0, or -1 on a bad k or allocation. */
int oracle_order_stats(const double* r, int64_t n, int64_t k, double* tk_out, double* tk1_out) {
    if (n < 1 || k < 1 || k > n) return -1;
    double* v = (double*)malloc(sizeof(double) * (size_t)n);
    if (!v) return -1;
    for (int64_t i = 0; i < n; ++i) v[i] = r[i];
    qsort(v, (size_t)n, sizeof(double), cmp_double);
    *tk_out = v[n - k];
    *tk1_out = k < n ? v[n - k - 1] : -INFINITY;
    free(v);
    return 0;
}

/* hard top-k: mask_i = 1 when r_i >= the k-th largest score, else 0.  With
 * ties at the threshold more than k scores qualify.  Returns the number of
 * ones (-1 on a bad k); *tau_out gets the threshold. */
int64_t oracle_hard_topk(const double* r, int64_t n, int64_t k, double* mask_out, double* tau_out) {
    double tk, tk1;
    if (oracle_order_stats(r, n, k, &tk, &tk1) != 0) return -1;
    int64_t ones = 0;
    for (int64_t i = 0; i < n; ++i) {
        mask_out[i] = r[i] >= tk ? 1.0 : 0.0;
        ones += r[i] >= tk;
    }
    *tau_out = tk;
    return ones;
}

/* DFTopK: b = (k-th largest + (k+1)-th largest) / 2 (1 <= k < n) and
 * p_i = F((r_i - b)/t) with the same Laplace CDF as LapSum.  Returns sum p
 * (NaN on a bad k); *b_out gets b. */
double oracle_dftopk(const double* r, int64_t n, int64_t k, double t, double* p_out, double* b_out) {
    double tk, tk1;
    if (k >= n || oracle_order_stats(r, n, k, &tk, &tk1) != 0) return NAN;
    const double b = 0.5 * (tk + tk1);
    *b_out = b;
    return oracle_probs(r, n, t, b, p_out);
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: */
/* as easy as 1, 2, 3", SC'11): 10 rounds of the Philox S-box          */
/* (two 32x32->64 multiplies by 0xD2511F53 and 0xCD9E8D57) with a Weyl */
/* key schedule (0x9E3779B9, 0xBB67AE85).                               */
/* ------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)p1;
        uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)p0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/*
 * The kernel-noised sample (gist.science summary 2.2, bracketing step 1;
 * the arxivdaily abstract names the same step):
 * draw j = 0..s-1: Philox4x32-10 with counter (j_lo, j_hi, 0, 0) and key
 * (seed_lo, seed_hi) gives words w0..w3;
 *   index I_j = floor(((w1 << 32) | w0) * n / 2^64)       (uniform, with replacement)
 *   u_j       = ((((w3 << 32) | w2) >> 11) + 0.5) / 2^53   (open (0, 1))
 *   eps_j     = t ln(2u) if u < 1/2 else -t ln(2(1-u))     (Laplace(0, t), inverse CDF)
 *   x_j       = fp32 rounding of (r_{I_j} + eps_j) evaluated in fp64.
 * Then P(r_I + eps > b) = G(b)/n, so the (1 - k/n) quantile of x is b.
 */
void oracle_sample(const double* r, int64_t n, double t, uint64_t seed, int64_t s,
                   int64_t* idx_out, float* x_out) {
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int64_t j = 0; j < s; ++j) {
        uint32_t ctr[4] = {(uint32_t)j, (uint32_t)((uint64_t)j >> 32), 0u, 0u};
        uint32_t w[4];
        oracle_philox4x32_10(ctr, key, w);
        uint64_t u64 = ((uint64_t)w[1] << 32) | w[0];
        int64_t idx = (int64_t)(((unsigned __int128)u64 * (unsigned __int128)(uint64_t)n) >> 64);
        uint64_t m53 = ((((uint64_t)w[3]) << 32) | w[2]) >> 11;
        double u = ((double)m53 + 0.5) * 0x1p-53;
        double eps = (u < 0.5) ? t * log(2.0 * u) : -t * log(2.0 * (1.0 - u));
        if (idx_out) idx_out[j] = idx;
        x_out[j] = (float)(r[idx] + eps);
    }
}

/* ------------------------------------------------------------------ */
/* Binomial order-statistic bounds (gist.science summary 2.2, bracketing step 1). */
/* Y = #{samples below b} ~ Bin(s, q), q = 1 - k/n.                     */
/*   a_L = x_(l) <= b  <=>  Y >= l ;  l = largest l with P(Y <= l-1) <= delta */
/*   a_R = x_(h) >  b  <=>  Y <= h-1; h = smallest h with P(Y >= h) <= delta  */
/* l = 0 means a_L = -inf, h = s + 1 means a_R = +inf.                  */
/* ------------------------------------------------------------------ */
static double binom_logpmf(int64_t s, double lq, double l1q, int64_t i) {
    return lgamma((double)s + 1.0) - lgamma((double)i + 1.0) - lgamma((double)(s - i) + 1.0)
           + (double)i * lq + (double)(s - i) * l1q;
}

void oracle_binomial_bounds(int64_t s, double q, double delta, int64_t* l_out, int64_t* h_out) {
    double lq = log(q), l1q = log1p(-q);
    double cdf = 0.0;
    int64_t l = 0;
    for (int64_t y = 0; y <= s; ++y) {
        cdf += exp(binom_logpmf(s, lq, l1q, y));
        if (cdf <= delta) l = y + 1; else break;
    }
    double tail = 0.0;
    int64_t h = s + 1;
    for (int64_t i = s; i >= 0; --i) {
        tail += exp(binom_logpmf(s, lq, l1q, i));
        if (tail <= delta) h = i; else break;
    }
    *l_out = l; *h_out = h;
}

/* exact miss probability P(Y <= l-1) + P(Y >= h), each tail summed directly */
double oracle_binomial_miss(int64_t s, double q, int64_t l, int64_t h) {
    double lq = log(q), l1q = log1p(-q);
    double lower = 0.0, upper = 0.0;
    for (int64_t y = 0; y <= l - 1 && y <= s; ++y) lower += exp(binom_logpmf(s, lq, l1q, y));
    for (int64_t y = s; y >= h && y >= 0; --y) upper += exp(binom_logpmf(s, lq, l1q, y));
    return lower + upper;
}
