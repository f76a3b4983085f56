/*
 * lapsum.h -- C ABI of the MI355X (gfx950) Fast LapSum solver.
 *
 * The operator (Fast LapSum paper, gist.science summary section 2.1 "El
 * Operador LapSum"): given scores r[n], a temperature t > 0 and a budget
 * 0 < k < n, the threshold b is the unique root of
 *
 *     G(b) = sum_i F((r_i - b) / t) = k,
 *
 * F the Laplace CDF with scale 1 (F(x) = e^x/2 for x < 0, 1 - e^-x/2 for
 * x >= 0).  The selection probabilities are p_i = F((r_i - b)/t), and they
 * sum to exactly k.  The backward pass is the analytic vector-Jacobian
 * product (same section):
 *
 *     grad_i = (f_i / t) (g_i - sum_j g_j f_j / sum_j f_j),
 *     f_i = e^{-|r_i - b| / t} / 2  (the Laplace density).
 *
 * Two forward paths (section 2.2 "Fast LapSum: El Solucionador de GPU"):
 * a full sort followed by one stable prefix/suffix scan, an interval search
 * and a closed-form root; and, for large n, probabilistic bracketing (a
 * kernel-noised sample and a binomial order statistic give a band
 * [a_L, a_R); one streaming pass folds the scores outside it into tail sums;
 * only the band is sorted and solved; the bracket is certified and widened
 * when it fails, with the full sort as the fallback -- the arxivdaily
 * abstract names both the certification pass and the full-sort fallback).
 *
 * Conventions for every entry point:
 *  - Pointers to scores, p, g, grad and b are DEVICE pointers (gfx950), owned
 *    by the caller.  The library never frees caller memory.
 *  - All work is ordered on `stream` (a hipStream_t; NULL is the default
 *    stream).  Scratch memory is a per-(device, stream) workspace that the
 *    library allocates on first use and keeps until lapsum_release_workspaces.
 *  - Argument errors are returned before anything is launched and nothing is
 *    written.
 *  - Errors found on the device: non-finite scores (b and p are then NaN) and
 *    failed consistency checks (LAPSUM_ERR_INTERNAL).  A call given a
 *    lapsum_stats_t waits for the device and returns what it found (also in
 *    stats->status).  Without stats, only what the device reported before the
 *    host's last wait is returned: the bracketing path waits for its
 *    certification verdict and returns non-finite scores found by then; the
 *    full-sort path and the VJP never block the host, and a check that fails
 *    after the last wait is visible only through stats.
 *  - n is limited to [1, 2^32 - 1].
 *  - No exception crosses this ABI.  Calls may come from several host
 *    threads: a call holds its (device, stream) workspace from its start to
 *    its return, so calls on one stream take turns (their device work is
 *    ordered on the stream in the order they took it), calls on different
 *    streams run side by side, and lapsum_release_workspaces waits for the
 *    calls in flight.
 */
#ifndef LAPSUM_H_
#define LAPSUM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t is `struct ihipStream_t*`; declared here so C callers need no HIP header. */
typedef struct ihipStream_t* lapsum_stream_t;

typedef enum {
    LAPSUM_OK = 0,
    LAPSUM_ERR_INVALID_ARGUMENT = 1, /* n, k, t or a pointer out of range; nothing written */
    LAPSUM_ERR_NONFINITE_INPUT = 2,  /* a score is NaN or +-inf; b and p set to NaN */
    LAPSUM_ERR_OUT_OF_MEMORY = 3,    /* workspace allocation failed */
    LAPSUM_ERR_HIP = 4,              /* a HIP runtime call failed */
    LAPSUM_ERR_INTERNAL = 5          /* a consistency check failed (reported, never silent) */
} lapsum_status_t;

typedef enum {
    LAPSUM_PATH_AUTO = 0,           /* bracketing iff n > auto_threshold (default 10^6) */
    LAPSUM_PATH_FULL = 1,           /* full sort */
    LAPSUM_PATH_BRACKET = 2,        /* bracketing (with widening and full-sort fallback) */
    LAPSUM_PATH_FORCE_FALLBACK = 3  /* bracketing pass, then the full-sort fallback regardless */
} lapsum_path_t;

/* Options of lapsum_forward_ex.  Obtain defaults from lapsum_default_options. */
typedef struct {
    int32_t path;           /* lapsum_path_t */
    int32_t max_widen;      /* bracket widenings before the full-sort fallback (default 2) */
    uint64_t seed;          /* Philox4x32-10 key of the sampler (default 0x5EED) */
    double sample_factor;   /* sample size s = ceil(sample_factor * sqrt(n)), capped at 40960 (default 4) */
    double delta;           /* per-side probability that the bracket misses b (default 1e-5) */
    double margin_scale;    /* multiplies both order-statistic margins; 1 = exact binomial ranks,
                               0 = a zero-width bracket (forces widening; for tests) */
    int64_t auto_threshold; /* LAPSUM_PATH_AUTO uses bracketing iff n > auto_threshold (default 10^6) */
    int32_t bucket_capacity;/* band scores per bucket, <= 16384 (default 16384; small values force
                               the overflow fallback in tests) */
    int32_t profile;        /* 1: time every kernel with HIP events (reported in stats) */
    int32_t cert_mode;      /* certification of the bracket: 0 (default) from the streaming pass's own
                               sums at no extra read; 1 one more linear pass over the scores that sums
                               G(a_L) and G(a_R) directly, whose verdict decides (the pages' form) */
} lapsum_options_t;

#define LAPSUM_MAX_TIMED_KERNELS 24

/* Filled by lapsum_forward_ex when stats is not NULL (the call then waits
 * for the device before returning). */
typedef struct {
    int32_t status;          /* lapsum_status_t of the device-side checks */
    int32_t path_taken;      /* 1 full sort, 2 bracketing certified, 3 bracketing -> full-sort fallback */
    int32_t widenings;       /* bracket widenings performed */
    int32_t certified;       /* 1 if the final bracket held (G(a_L) >= k > G(a_R)) */
    int64_t count_below;     /* scores < a_L */
    int64_t band_size;       /* scores in [a_L, a_R) */
    int64_t count_above;     /* scores >= a_R */
    int64_t sample_size;     /* s */
    int64_t rank_lo, rank_hi;/* order-statistic ranks l, h (1-based; 0 = -inf, s+1 = +inf) */
    int32_t buckets;         /* band buckets used */
    int32_t n_timed;         /* entries in kernel_ms / kernel_name */
    float a_L, a_R;          /* final bracket */
    double g_aL, g_aR;       /* G at the bracket ends, rebuilt from the streaming pass's tail sums */
    double g_aL_direct, g_aR_direct; /* cert_mode 1: G at the bracket ends summed by the certification
                                        pass (0 otherwise) */
    double sum_p;            /* sum of the written p, accumulated in fp64 on the device */
    double b;                /* threshold */
    double tail_S_L, tail_S_R, band_B_L, band_B_R; /* the streaming pass's sums (fp64 per tile and lane, then
                                                      fixed point in units of 2^-36: the same every run) */
    double vjp_c, vjp_sum_f;  /* lapsum_vjp_ex: c = sum g f / sum f and sum f */
    float kernel_ms[LAPSUM_MAX_TIMED_KERNELS];     /* with options.profile: per-launch times */
    const char* kernel_name[LAPSUM_MAX_TIMED_KERNELS];
} lapsum_stats_t;

/* Default options (see the field comments). */
void lapsum_default_options(lapsum_options_t* opt);

/* Human-readable name of a status code (static storage). */
const char* lapsum_status_string(lapsum_status_t status);

/*
 * Forward solve (gist.science section 2.1 and 2.2).
 *   scores : device fp32[n], read only.
 *   n      : number of scores, 1 <= n < 2^32.
 *   k      : budget, 0 < k < n (real valued).
 *   t      : temperature, finite and > 0.
 *   p_out  : device fp32[n], receives p_i = F((r_i - b)/t) (may alias nothing else).
 *   b_out  : device fp64[1], receives b.
 * Path: full sort for n <= 10^6, bracketing above.  Returns LAPSUM_OK,
 * LAPSUM_ERR_INVALID_ARGUMENT, LAPSUM_ERR_NONFINITE_INPUT (bracketing path),
 * LAPSUM_ERR_OUT_OF_MEMORY or LAPSUM_ERR_HIP.
 */
lapsum_status_t lapsum_forward(const float* scores, int64_t n, double k, float t,
                               float* p_out, double* b_out, lapsum_stream_t stream);

/* lapsum_forward with explicit options (NULL = defaults) and optional host
 * stats (NULL = none; non-NULL makes the call wait for the device). */
lapsum_status_t lapsum_forward_ex(const float* scores, int64_t n, double k, float t,
                                  float* p_out, double* b_out, const lapsum_options_t* opt,
                                  lapsum_stats_t* stats, lapsum_stream_t stream);

/*
 * Analytic VJP (gist.science section 2.1): grad_i = (f_i/t)(g_i - c),
 * c = sum g f / sum f, f_i = e^{-|r_i - b|/t}/2, recomputed from (scores, b).
 *   scores  : device fp32[n], the forward's scores.
 *   p       : device fp32[n] or NULL; accepted for symmetry and not read
 *             (f from an fp32 p near 1 would lose the accuracy f needs).
 *   g       : device fp32[n], upstream gradient dL/dp.
 *   t       : the forward's temperature.
 *   b       : device fp64[1], the forward's threshold.
 *   grad_out: device fp32[n], receives dL/dr.
 * Never blocks the host.
 */
lapsum_status_t lapsum_vjp(const float* scores, const float* p, const float* g, int64_t n, float t,
                           const double* b, float* grad_out, lapsum_stream_t stream);

/* lapsum_vjp with options (only `profile` is read) and optional host stats
 * (kernel times, vjp_c, vjp_sum_f; non-NULL makes the call wait). */
lapsum_status_t lapsum_vjp_ex(const float* scores, const float* p, const float* g, int64_t n, float t,
                              const double* b, float* grad_out, const lapsum_options_t* opt,
                              lapsum_stats_t* stats, lapsum_stream_t stream);

/*
 * Analytic VJP together with the gradients with respect to the budget and the
 * temperature (gist.science summary section 2.1; implicit differentiation of
 * the budget equation G(b) = k).  With d_i = r_i - b and
 * f_i = e^{-|d_i|/t}/2, for L = sum_i g_i p_i:
 *
 *     dL/dk = sum g f / sum f,
 *     dL/dt = -(sum g f d - mu sum g f) / t^2,   mu = sum f d / sum f.
 *
 * grad_out: device fp32[n], the score gradient as in lapsum_vjp (NULL: only
 * the two scalars are formed, one pass over scores and g).  dk_out, dt_out:
 * device fp64[1] each, or NULL.  At least one of the three outputs must be
 * given.  Argument rules, errors and stream semantics as lapsum_vjp_ex.
 */
lapsum_status_t lapsum_vjp_kt(const float* scores, const float* g, int64_t n, float t, const double* b,
                              float* grad_out, double* dk_out, double* dt_out,
                              const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream);

/*
 * Order statistics from the top (hard top-k and DFTopK; gist.science summary
 * section 2.3: DFTopK puts the threshold at the midpoint of the k-th and
 * (k+1)-th order statistics and is LapSum's zero-temperature limit).  They
 * run through the same machinery as lapsum_forward_ex: the full sort for
 * n <= opt->auto_threshold, else a noiseless sample, the streaming filter and
 * a count-based certification (both order statistics inside the band), with
 * widening and the full-sort fallback.  opt and stats as in
 * lapsum_forward_ex (the LapSum-only stats fields stay zero).
 *
 * lapsum_topk_threshold: tau_out (device fp64[2]) gets the k-th largest score
 *   and the (k+1)-th largest (-inf when k = n).  1 <= k <= n.
 * lapsum_hard_topk: mask_out (device fp32[n]) gets 1 where
 *   scores[i] >= the k-th largest, else 0 (with ties at the threshold more
 *   than k entries are 1); tau_out as above, or NULL.  1 <= k <= n.
 * lapsum_dftopk: b_out (device fp64[1], or NULL) gets
 *   b = (k-th largest + (k+1)-th largest) / 2, p_out (device fp32[n]) gets
 *   p_i = F((scores[i] - b)/t) with LapSum's Laplace CDF; its mass generally
 *   differs from k.  1 <= k <= n - 1, t > 0.
 * Errors: LAPSUM_ERR_INVALID_ARGUMENT (checked before any launch) for NULL
 * required pointers, n outside [1, 2^32), k outside its range, a bad t or
 * bad options; LAPSUM_ERR_NONFINITE_INPUT when the bracketing path meets a
 * NaN or infinity (outputs become NaN; the full-sort path reports it in
 * stats->status).
 */
lapsum_status_t lapsum_topk_threshold(const float* scores, int64_t n, int64_t k, double* tau_out,
                                      const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream);
lapsum_status_t lapsum_hard_topk(const float* scores, int64_t n, int64_t k, float* mask_out, double* tau_out,
                                 const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream);
lapsum_status_t lapsum_dftopk(const float* scores, int64_t n, int64_t k, float t, float* p_out, double* b_out,
                              const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream);

/*
 * Many independent rows (the operator applied per row, as in routing and
 * pruning; gist.science summary sections 1 and 5).  scores, p_out, g,
 * grad_out: device fp32[rows * n], row i at offset i * n.  b_out / b: device
 * fp64[rows].  Budget: k_rows (device fp64[rows], each in (0, n)) when not
 * NULL, else the scalar k for every row.  Rows with n <= 16384 are solved one
 * workgroup per row in LDS (sort, curve scan, closed-form root, p); rows up
 * to 65536 scores one workgroup per row that sorts its row through scratch
 * memory of the stream's workspace (2 n words per workgroup of a grid of one
 * round of co-resident workgroups), then solves and writes p; longer rows run
 * through lapsum_forward_ex's solver one after another.  A row with a
 * non-finite score or a budget outside (0, n) gets b = NaN and p = NaN; the
 * call still returns LAPSUM_OK.  Argument errors (NULL pointers, rows < 1, n
 * outside [1, 2^32), a bad scalar k when k_rows is NULL, a bad t) return
 * LAPSUM_ERR_INVALID_ARGUMENT before any launch.  Asynchronous on `stream`
 * (except for rows longer than 65536 with k_rows, whose budgets are read
 * first).  The VJP (lapsum_vjp_batched) runs one workgroup per row up to
 * 65536 scores, and longer rows through lapsum_vjp's kernels one by one.
 */
lapsum_status_t lapsum_forward_batched(const float* scores, int64_t rows, int64_t n, double k,
                                       const double* k_rows, float t, float* p_out, double* b_out,
                                       lapsum_stream_t stream);
lapsum_status_t lapsum_vjp_batched(const float* scores, const float* g, int64_t rows, int64_t n, float t,
                                   const double* b, float* grad_out, lapsum_stream_t stream);

/*
 * lapsum_forward without any device allocation, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and conventions as
 * lapsum_forward on its full-sort path, for 1 <= n <= 2^20 scores; a larger n
 * is LAPSUM_ERR_INVALID_ARGUMENT before anything is launched.  Scratch memory
 * is one fixed device array of about 9 MB per GPU, inside the library's code
 * object, held until the process ends; the call allocates nothing and frees
 * nothing (its first call on a device only looks up that array's address).
 * Every call on a GPU uses the same array: calls that overlap on one GPU
 * (two streams, two host threads) race and must be serialised by the caller.
 * Never blocks the host; non-finite scores give b = NaN and p = NaN.
 */
lapsum_status_t lapsum_forward_noalloc(const float* scores, int64_t n, double k, float t, float* p_out,
                                       double* b_out, lapsum_stream_t stream);

/* Free every cached workspace (waits for their streams). */
void lapsum_release_workspaces(void);

/* Bytes of device workspace a forward of n scores with options `opt` (NULL =
 * defaults) holds on its stream: the library allocates it on the first call
 * on a stream that needs that much and keeps it until
 * lapsum_release_workspaces.  It includes the full-sort fallback's buffers,
 * which any forward may need.  0 for n outside [1, 2^32) or bad options. */
size_t lapsum_workspace_bytes(int64_t n, const lapsum_options_t* opt);

#ifdef __cplusplus
}
#endif

#endif /* LAPSUM_H_ */
