/*
 * lapsum_testing.h -- entry points that expose single stages of the Fast
 * LapSum solver for parity tests.  They run the same kernels as
 * lapsum_forward_ex; each waits for the device before returning.
 * All pointers are device pointers unless named *_host.
 */
#ifndef LAPSUM_TESTING_H_
#define LAPSUM_TESTING_H_

#include "lapsum.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Ascending sort of fp32 scores as order-preserving keys (-0.0 read as
 * +0.0): the full-sort path's sort (gist.science section 2.2, full-sort
 * solver).  n <= 16384 uses the single-workgroup LDS sort, larger n the
 * multi-workgroup LSD radix sort.  out: device fp32[n].
 */
lapsum_status_t lapsum_test_sort(const float* scores, int64_t n, float* out, lapsum_stream_t stream);

/*
 * The kernel-noised sample (section 2.2, localisation step): x_j = fp32 of
 * r[I_j] + eps_j for j < s, with Philox4x32-10 counter (j, 0, 0) and key
 * `seed`; I_j uniform in [0, n), eps_j ~ Laplace(0, t).  idx_out may be NULL.
 */
lapsum_status_t lapsum_test_sample(const float* scores, int64_t n, float t, uint64_t seed, int64_t s,
                                   float* x_out, int64_t* idx_out, lapsum_stream_t stream);

/*
 * Order statistics of a sample x[s] (device): a_L = x_(l), a_R = x_(h)
 * (1-based ranks; l = 0 gives -inf, h = s + 1 gives +inf), written to the
 * host.  Also returns the bucket layout the bracketing path would use.
 */
lapsum_status_t lapsum_test_select(const float* x, int64_t s, int64_t l, int64_t h,
                                   float* aL_host, float* aR_host, int32_t* nbuckets_host,
                                   lapsum_stream_t stream);

/*
 * The streaming filter for a given bracket [a_L, a_R) (section 2.2,
 * streaming and filtering), with no interior splitters: counts_host gets
 * {below, band, above}, sums_host {S_L, S_R, B_L, B_R}; the band values go
 * to band_out (device fp32, capacity band_cap) bucket by bucket in bucket
 * order (unordered inside a bucket; buckets are value-ordered);
 * *band_size_host gets the band size (or -1 if it exceeded band_cap or a
 * bucket's capacity), *nbuckets_host the bucket count and
 * bucket_sizes_host[0..nbuckets) (host, capacity 1024) their sizes.
 */
lapsum_status_t lapsum_test_filter(const float* scores, int64_t n, float t, float a_L, float a_R,
                                   int64_t* counts_host, double* sums_host, float* band_out,
                                   int64_t band_cap, int64_t* band_size_host, int32_t* nbuckets_host,
                                   int64_t* bucket_sizes_host, lapsum_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LAPSUM_TESTING_H_ */
