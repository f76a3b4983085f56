/*
 * lapsum_testing.h -- entry points that expose single stages of the Fast
 * LapSum solver for parity tests.  They run the same kernels as
 * lapsum_forward_ex; each waits for the device before returning, except the
 * two bandwidth-ceiling kernels at the end.
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
 * The same sort in a given form of its multi-workgroup passes: form 0 picks
 * by size (as lapsum_test_sort); 1 takes the one-kernel passes in their
 * look-back design (the design a sort uses while another holds the device's
 * resident-pass lock) where the size allows one-kernel passes; 2 takes the
 * split passes (count, scan, scatter).  The result is the same in every
 * form.  LAPSUM_ERR_INVALID_ARGUMENT for another form.
 */
lapsum_status_t lapsum_test_sort_form(const float* scores, int64_t n, float* out, int32_t form,
                                      lapsum_stream_t stream);

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

/*
 * The bracket's sample ranks (section 2.2, bracketing step 1), host only:
 * for a sample of s noised scores each above b with probability 1 - q,
 * l = the largest rank with P(Bin(s, q) < l) <= delta and h = the smallest
 * with P(Bin(s, q) >= h) <= delta, so a_L = x_(l) and a_R = x_(h) (1-based;
 * l = 0 and h = s + 1 mean an open end).  Needs no device.
 */
lapsum_status_t lapsum_test_binomial_ranks(int64_t s, double q, double delta, int64_t* l, int64_t* h);

/*
 * Plain streaming kernels: the achievable HBM ceilings the solver's
 * streaming passes are compared with, and a transfer of known size for
 * calibrating hardware traffic counters.  lapsum_test_copy copies n fp32
 * from src to dst (device, 16-byte aligned, not overlapping);
 * lapsum_test_read reads n fp32 from src (16-byte aligned) and may write
 * to sink (device fp32[256]).  Both are asynchronous on `stream` (they do
 * not wait for the device); misaligned or NULL pointers and n < 1 give
 * LAPSUM_ERR_INVALID_ARGUMENT before any launch.
 */
lapsum_status_t lapsum_test_copy(const float* src, float* dst, int64_t n, lapsum_stream_t stream);
lapsum_status_t lapsum_test_read(const float* src, int64_t n, float* sink, lapsum_stream_t stream);

/*
 * Error-path check: the next forward solve on `stream` (on the current
 * device) ends with a kernel that sets the consistency-failure flag in its
 * control block, exactly as a failed device-side check does, so that the
 * call reports LAPSUM_ERR_INTERNAL when it is given stats.  The solve itself
 * runs as usual.  Returns an allocation or HIP error, else LAPSUM_OK.
 */
lapsum_status_t lapsum_test_inject_internal(lapsum_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LAPSUM_TESTING_H_ */
