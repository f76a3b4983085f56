// Host-side launchers of the Fast LapSum kernels (each defined next to its kernels).
#pragma once
#include "lapsum_blocksolve.h"
#include "lapsum_device.h"

namespace lapsum {

struct SegArrays {
    float* first;
    float* last;
    double* P;
    double* Bx;
    uint32_t* cnt;
    uint32_t* off;
};

// lapsum_sample.hip
// hist (may be null): zero on entry, left holding the histogram of the
// sample keys' leading 12 bits (kSelHistBins words); hclr (may be null): a
// histogram buffer to clear for the next call
void launch_sample(const float* r, long long n, double t, unsigned long long seed, int s, float* x, long long* idx_out,
                   hipStream_t st, uint32_t* hist = nullptr, uint32_t* hclr = nullptr);
// the sample histogram alone (clears hclr as launch_sample does)
void launch_key_hist(const float* x, int s, uint32_t* hist, uint32_t* hclr, hipStream_t st);
// hist, win (both or neither): the sample's histogram from launch_sample and
// a window buffer (kWinHdr + kWinMax words, fill count zero on entry and on
// exit): the window of sample keys around ranks l..h is gathered by many
// workgroups first
void launch_select(const float* x, int s, long long l, long long h, int cap, Ctl* ctl, float* sp, float* iw,
                   uint32_t* bucket_cnt, hipStream_t st, const uint32_t* hist = nullptr, uint32_t* win = nullptr);

// lapsum_stream.hip
int stream_blocks(long long n);
// k: the budget the finalize kernel certifies the bracket against
// the filter pass alone (returns its workgroup count, the number of
// partials) and its finalize kernel; launch_filter runs both
int launch_filter_pass(const float* r, long long n, double t, Ctl* ctl, const float* sp, const float* iw,
                       uint32_t* bucket_cnt, uint32_t* bucket_vals, int cap, double* part, hipStream_t st);
// defer: the certification pass (launch_cert) decides instead; the gate
// stays shut and the host summary is left to it
void launch_filter_finalize(long long n, double t, Ctl* ctl, const uint32_t* bucket_cnt, int cap, double* part,
                            int nparts, HostSummary* hs_dev, unsigned int seq, hipStream_t st, double k,
                            const HeavyArrays* ha, bool defer = false);
// The certification pass as a pass of its own (cert_mode 1): G(a_L) and
// G(a_R) summed directly over every score, then the verdict, the gate and the
// host summary (after a deferred launch_filter_finalize)
void launch_cert(const float* r, long long n, double t, Ctl* ctl, double* part, HostSummary* hs_dev,
                 unsigned int seq, double k, hipStream_t st);
void launch_or_flags(Ctl* ctl, int flags, hipStream_t st);
void launch_filter(const float* r, long long n, double t, Ctl* ctl, const float* sp, const float* iw,
                   uint32_t* bucket_cnt, uint32_t* bucket_vals, int cap, double* part, HostSummary* hs_dev,
                   unsigned int seq, hipStream_t st, double k, const HeavyArrays* ha = nullptr);
// returns the number of partials it left (for launch_sum_p)
// gate (device, may be null): when it holds 0 the kernels return at once
int launch_probs(const float* r, long long n, double t, float* p, Ctl* ctl, double* part, hipStream_t st,
                 const int* gate = nullptr);
void launch_sum_p(Ctl* ctl, const double* part, int nparts, hipStream_t st);
// grad may be null (only the reduction and c); kt adds dL/dk, dL/dt (each output may be null)
void launch_vjp(const float* r, const float* g, long long n, double t, const double* b, float* grad, Ctl* ctl,
                double* part, hipStream_t st, hipEvent_t* ev_mid, bool kt, double* dk_out, double* dt_out);
void launch_fill(float* p, long long n, float v, hipStream_t st);
void launch_set_nan_b(Ctl* ctl, double* b_out, hipStream_t st);
void launch_copy_b(const Ctl* ctl, double* b_out, hipStream_t st);  // b_out may be null

// lapsum_ceiling.hip
void launch_copy(const float* a, float* b, long long n, hipStream_t st);
void launch_read(const float* a, long long n, float* sink, hipStream_t st);

// lapsum_topk.hip
void launch_small_sort(const float* r, int n, Ctl* ctl, uint32_t* keys_out, hipStream_t st);
void launch_pick_sorted(const uint32_t* keys, long long n, long long k, Ctl* ctl, double* tau_out, hipStream_t st);
void launch_bucket_pick(const uint32_t* bucket_vals, const uint32_t* bucket_cnt, int cap, long long k, Ctl* ctl,
                        double* tau_out, hipStream_t st);
void launch_mask(const float* r, long long n, const Ctl* ctl, float* mask, hipStream_t st);

// lapsum_heavy.hip
// collect every score of the overflowed buckets into their slots, then the
// chunk sums of their aggregates (both run only when the finalize kernel set
// kFlagHeavy; hchunks bounds the aggregation grid)
void launch_heavy_collect(const float* r, long long n, const Ctl* ctl, const float* sp, const float* iw,
                          const HeavyArrays& ha, uint32_t* base, uint32_t hchunks, double t, hipStream_t st);

// lapsum_batched.hip
int rows_supported_max();  // longest row the row kernels take (longer rows: the single-vector solver)
constexpr int kRowsLdsMax = kSmallMax;  // rows up to this length are sorted in LDS
size_t rows_long_scratch_words(long long rows, int n);  // scratch of launch_rows_forward_long (uint32 words)
void launch_rows_forward_long(const float* r, long long rows, int n, const double* k_rows, double k_all, double t,
                              float* p, double* b_out, uint32_t* scratch, hipStream_t st);
void launch_rows_forward(const float* r, long long rows, int n, const double* k_rows, double k_all, double t, float* p,
                         double* b_out, hipStream_t st);
void launch_rows_vjp(const float* r, const float* g, long long rows, int n, double t, const double* b, float* grad,
                     hipStream_t st);

// lapsum_sort.hip
void launch_small_solve(const float* r, int n, double k, double t, Ctl* ctl, SolveScratch sc, double* b_out,
                        uint32_t* keys_out, hipStream_t s);
// hoff: null, or per bucket the slot offset of an overflowed bucket's scores (kNotHeavy otherwise)
// ha: the overflowed buckets' slots (null: none); gate: run only when *gate
// is nonzero; hs / seq: tell the host through the pinned summary when done
void launch_bucket_solve(uint32_t* bucket_vals, const uint32_t* bucket_cnt, int cap, int nb, Ctl* ctl, SegArrays seg,
                         SolveScratch sc, double k, double t, double* b_out, hipStream_t s,
                         const HeavyArrays* ha = nullptr, const int* gate = nullptr, HostSummary* hs = nullptr,
                         unsigned int seq = 0);
int radix_hist_blocks(long long n);
bool radix_uses_onesweep(long long n);
size_t radix_status_words(long long n_cap);  // else the split passes (counts, scan, scatter)
void launch_radix_sort(const float* r, long long n, uint32_t* keysA, uint32_t* keysB, uint32_t* hist_part,
                       uint32_t* goff, unsigned long long* status, uint32_t epoch_base, Ctl* ctl, hipStream_t s,
                       int form = 0);  // 0: by size; 1: one-kernel passes in the look-back design; 2: split passes
void launch_curve_tiles(const uint32_t* keys, long long n, Ctl* ctl, SegArrays seg, SolveScratch sc, double k, double t,
                        double* b_out, hipStream_t s, bool ctl_tails = false);

}  // namespace lapsum
