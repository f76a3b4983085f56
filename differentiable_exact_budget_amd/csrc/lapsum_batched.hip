// Many independent rows at once: the exact-budget operator applied per row
// (the pages' uses -- expert routing, memory selection, pruning; gist.science
// summary sections 1 and 5 -- apply it to many short vectors).  One
// workgroup per row.  It first solves the row without sorting it: the
// full-sort solver's closed-form root on the piece of the curve around a
// start next to the k-th largest score, moved from piece to piece until the
// root falls inside its own piece (below).  A row that does not settle that
// way is sorted and solved as in the full-sort path (gist.science section
// 2.2): radix sort, the curve solve of one segment.  Then p for the row; the
// VJP reduces and applies per row.  Rows must be contiguous (row i starts at
// i * n).  Rows of n <= 16384 are held in registers (and sorted in LDS), the
// workgroup size following n; longer rows, up to 65536, are read from global
// memory at every pass (and sorted through global scratch, below).
#include <algorithm>

#include "lapsum_blocksolve.h"
#include "lapsum_launch.h"
#include "lapsum_steps.h"

namespace lapsum {

constexpr int kHistCopies_rows = 4;  // lane-group copies of the long-row histograms (as in the radix sort)

// The sort-free start and steps (lapsum_steps.h) for a row: the
// start is the middle of the key range that shares its top 16 bits (sign,
// exponent and 7 mantissa bits: 2^-7 wide relative to the score) with the
// k-th largest score, from two radix-select digits (measured on gfx950: two
// digits beat all four, 4096 x 4096 rows 0.094 against 0.109 ms, as the steps
// that follow cost less than the two more digits would).
template <int NT, class Row>
LS_DEV StepRoot row_solve(const Row& row, double k, double t, double inv_t, uint32_t* hist, uint32_t* s_sel,
                          double* sd, unsigned long long* su, uint32_t* sm) {
    const double kf = floor(k);
    const uint32_t kk = (uint32_t)(kf < 1.0 ? 1.0 : (kf > (double)row.n ? (double)row.n : kf));
    const float b0 = key2f(start_key<NT, 2>(row, kk, hist, s_sel));
    return solve_steps<NT>(row, k, t, inv_t, (double)b0, sd, su, sm);
}

template <int NT, int ITEMS>
__global__ __launch_bounds__(NT, (NT == 256 ? 4 : 1)) void k_rows_forward(const float* __restrict__ r, int n, const double* k_rows,
                                                      double k_all, double t, double inv_t, float* __restrict__ p,
                                                      double* b_out) {
    __shared__ uint32_t keys[NT * ITEMS];
    __shared__ uint32_t cnt[256 * (NT / 64)];
    __shared__ uint32_t scr[32];
    __shared__ float s_k[NT];
    __shared__ double s_v[NT];
    __shared__ int s_int[32];
    __shared__ uint32_t sg_cnt, sg_off;
    __shared__ float sc_pk, sc_bk;
    __shared__ double sc_pv, sc_bv, sc_bfx;
    __shared__ uint32_t sc_rank;
    __shared__ int s_bad;
    __shared__ double s_b;
    __shared__ uint32_t s_hist[4 * 256];
    __shared__ uint32_t s_sel[2];
    __shared__ double s_rd[2 * (NT / 64)];
    __shared__ unsigned long long s_ru[NT / 64];
    __shared__ uint32_t s_rm[2 * (NT / 64)];
    const int tid = threadIdx.x;
    const long long row = blockIdx.x;
    const float* rr = r + row * (long long)n;
    const double k = k_rows ? k_rows[row] : k_all;
    if (tid == 0) s_bad = !(k > 0.0 && k < (double)n);
    // the row into registers
    float v[ITEMS];
    int bad = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = j * NT + tid;
        v[j] = i < n ? rr[i] : 0.0f;
        bad |= i < n && !finite_f(v[j]);
    }
    __syncthreads();
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    StepRoot rt{0.0, 0};
    if (!s_bad) rt = row_solve<NT>(RegRow<NT, ITEMS>{v, n}, k, t, inv_t, s_hist, s_sel, s_rd, s_ru, s_rm);
    if (rt.ok) {
        if (tid == 0) { s_b = rt.b; b_out[row] = rt.b; }
    } else {
        // sorted in LDS: up to 4 keys per thread the bitonic sort (padded with
        // the largest key) beats the radix sort
        const int np = n <= 4 * NT ? max(next_pow2(n), 64) : n;
        for (int i = tid; i < np; i += NT) keys[i] = i < n ? f2key(rr[i]) : 0xFFFFFFFFu;
        __syncthreads();
        if (n <= 4 * NT) sort_pow2_lds<NT>(keys, np);
        else block_sort_lds<NT, ITEMS>(keys, n, cnt, scr);
        if (tid == 0) { sg_cnt = (uint32_t)n; sg_off = 0u; }
        __syncthreads();
        // the whole sorted array as one segment, no aggregates: the solve
        // tests G at every score
        SegView sv{1, nullptr, nullptr, nullptr, nullptr, &sg_cnt, &sg_off, keys, nullptr};
        SolveScratch sc{&sc_pk, &sc_pv, &sc_bk, &sc_bv, &sc_bfx, &sc_rank, nullptr, nullptr};
        Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t, -INFINITY, INFINITY};
        const SolveOut o = segment_solve<NT, ITEMS>(sv, tl, sc, s_k, s_v, s_int);
        if (tid == 0) {
            const double nanv = __longlong_as_double(0x7ff8000000000000ll);
            const double b = (s_bad || !o.ok) ? nanv : o.b;
            s_b = b;
            b_out[row] = b;
        }
    }
    __syncthreads();
    const double b = s_b;
    float* pr = p + row * (long long)n;
    for (int i = tid; i < n; i += NT) {
        const float x = (float)(((double)rr[i] - b) * inv_t);
        const float e = 0.5f * __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
        pr[i] = (b == b) ? (x < 0.0f ? e : 1.0f - e) : b;
    }
}

// per row: c = sum g f / sum f, grad = (f/t)(g - c), with f/t carried at
// 2^32 times its value (one exp2 with log2(1/(2t)) + 32 folded in) so that
// it does not flush where f itself would.  The two sums are taken with
// f = e^{-a}/2 (a = |r - b|/t) while the row's smallest a is tracked; when
// that is above 60 (every term of the row below e^{-60}, where fp32 flushes
// the far ones and, past ~87, all of them) the row is summed again relative
// to it, terms e^{a_min - a}/2, so sum f cannot vanish however far b lies
// from every score in units of t.
template <int NT>
__global__ __launch_bounds__(NT) void k_rows_vjp(const float* __restrict__ r, const float* __restrict__ g, int n,
                                                  double inv_t, float log2_inv_2t, const double* __restrict__ b,
                                                  float* __restrict__ grad) {
    __shared__ double s_red[NT / 64 > 0 ? NT / 64 : 1];
    __shared__ double s_mn[NT / 64 > 0 ? NT / 64 : 1];
    const int tid = threadIdx.x;
    const long long row = blockIdx.x;
    const float* rr = r + row * (long long)n;
    const float* gg = g + row * (long long)n;
    const double bb = b[row];
    double sfg = 0.0, sf = 0.0, dmin = INFINITY;
    for (int i = tid; i < n; i += NT) {
        const double d = (double)rr[i] - bb;
        const float x = (float)(d * inv_t);
        const float f = 0.5f * __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
        sfg += (double)(f * gg[i]);
        sf += (double)f;
        dmin = fmin(dmin, fabs(d));
    }
    const double M = block_min_nonneg_f64<NT>(dmin, s_mn) * inv_t;  // workgroup-uniform
    if (M > 60.0) {
        sfg = 0.0;
        sf = 0.0;
        for (int i = tid; i < n; i += NT) {
            const float y = (float)fma(-fabs((double)rr[i] - bb), inv_t, M);  // M - a <= 0
            const float f = __builtin_amdgcn_exp2f(fmaf(y, 1.4426950408889634f, -1.0f));
            sfg += (double)(f * gg[i]);
            sf += (double)f;
        }
    }
    const double T0 = block_sum<NT>(sfg, s_red);  // valid in wave 0
    const double T1 = block_sum<NT>(sf, s_red);
    __shared__ float s_c;
    if (tid == 0) s_c = (float)(T0 / T1);
    __syncthreads();
    const float c = s_c;
    float* gr = grad + row * (long long)n;
    for (int i = tid; i < n; i += NT) {
        const float x = (float)(((double)rr[i] - bb) * inv_t);
        const float f_over_t_2p32 = __builtin_amdgcn_exp2f(fmaf(-fabsf(x), 1.4426950408889634f, log2_inv_2t));
        gr[i] = (f_over_t_2p32 * (gg[i] - c)) * 0x1p-32f;
    }
}

// ---------------------------------------------------------------------------
// Long rows (16384 < n <= 65536), first without a sort: one 1024-thread
// workgroup per row reads the row from global memory at every pass (two
// select digits and the steps) and writes b and p; a row it does not settle
// gets kRowUnsolved (a NaN payload no other result carries) as its b, and
// the sorting kernel below, launched behind it, takes exactly those rows.
// The steps have a kernel of their own so that the sort's register pressure
// (its spills) stays out of their loops.
// ---------------------------------------------------------------------------
constexpr unsigned long long kRowUnsolved = 0x7FF8D0D0D0D0D0D0ull;
constexpr int kLongStepsNT = 1024;

__global__ __launch_bounds__(kLongStepsNT) void k_rows_steps_long(const float* __restrict__ r, int n,
                                                                  const double* k_rows, double k_all, double t,
                                                                  double inv_t, float* __restrict__ p,
                                                                  double* b_out) {
    constexpr int NT = kLongStepsNT, NW = NT / 64;
    __shared__ uint32_t hist[4 * 256];
    __shared__ uint32_t s_sel[2];
    __shared__ double s_rd[2 * NW];
    __shared__ unsigned long long s_ru[NW];
    __shared__ uint32_t s_rm[2 * NW];
    __shared__ int s_bad;
    const int tid = threadIdx.x;
    const long long row = blockIdx.x;
    const float* rr = r + row * (long long)n;
    const double k = k_rows ? k_rows[row] : k_all;
    if (tid == 0) s_bad = !(k > 0.0 && k < (double)n);
    int bad = 0;
    for (int i = tid; i < n; i += NT) bad |= !finite_f(rr[i]);
    __syncthreads();
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    StepRoot rt{0.0, 0};
    if (!s_bad) rt = row_solve<NT>(GlobalRow<NT>{rr, n}, k, t, inv_t, hist, s_sel, s_rd, s_ru, s_rm);
    if (tid == 0) b_out[row] = rt.ok ? rt.b : __longlong_as_double((long long)kRowUnsolved);
    if (!rt.ok) return;  // workgroup-uniform
    const double b = rt.b;
    float* pr = p + row * (long long)n;
    for (int i = tid; i < n; i += NT) {
        const float x = (float)(((double)rr[i] - b) * inv_t);
        const float e = 0.5f * __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
        pr[i] = x < 0.0f ? e : 1.0f - e;
    }
}

// ---------------------------------------------------------------------------
// Long rows (16384 < n <= 65536) that the steps left: a row does not fit one
// workgroup's LDS, so one workgroup per row sorts it through two global
// scratch buffers of its own -- an LSD radix sort whose passes it runs alone, 4096 keys at a time:
// all four digit histograms in one read, then per pass each chunk ranked
// stably in LDS and written out at its digits' running offsets -- and solves
// over the sorted row in 4096-key segments (aggregates per segment, the curve
// across them, the root segment's per-score curve, the root), then writes p.
// A fixed grid of such workgroups takes rows blockIdx.x, + gridDim.x, ...
// ---------------------------------------------------------------------------
constexpr int kLongNT = 1024, kLongItems = 4, kLongChunk = kLongNT * kLongItems;  // 4096 keys
constexpr int kLongMax = 65536;
constexpr int kLongSegs = kLongMax / kLongChunk;  // 16

__global__ __launch_bounds__(kLongNT) void k_rows_forward_long(const float* __restrict__ r, int n, long long rows,
                                                                const double* k_rows, double k_all, double t,
                                                                double inv_t, float* __restrict__ p,
                                                                double* b_out, uint32_t* scratch) {
    constexpr int NT = kLongNT, NW = NT / 64;
    __shared__ uint32_t hist[kHistCopies_rows * 4 * 256];  // lane-group copies x digit positions x bins
    __shared__ uint32_t offs[4 * 256];                      // per digit position: running digit offsets
    __shared__ uint32_t cnt[256 * NW];                      // a chunk's per-wave digit counters
    __shared__ uint32_t stage[kLongChunk];
    __shared__ uint32_t loc[256];
    __shared__ uint32_t scr[NW + 2];
    __shared__ int s_bad, s_skip;
    __shared__ float sg_first[kLongSegs], sg_last[kLongSegs];
    __shared__ double sg_P[kLongSegs], sg_Bx[kLongSegs];
    __shared__ uint32_t sg_cnt[kLongSegs], sg_off[kLongSegs];
    __shared__ float sc_pk[kLongSegs], sc_bk[kLongSegs];
    __shared__ double sc_pv[kLongSegs], sc_bv[kLongSegs], sc_bfx[kLongSegs];
    __shared__ uint32_t sc_rank[kLongSegs];
    __shared__ float s_k[NT];
    __shared__ double s_v[NT];
    __shared__ int s_int[32];
    __shared__ double s_red[NW];
    __shared__ double s_b;
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    uint32_t* const bufA = scratch + (size_t)blockIdx.x * 2 * (size_t)n;
    uint32_t* const bufB = bufA + n;
    for (long long row = blockIdx.x; row < rows; row += gridDim.x) {  // workgroup-uniform
        const float* rr = r + row * (long long)n;
        const double k = k_rows ? k_rows[row] : k_all;
        // rows the sort-free kernel settled are done
        if ((unsigned long long)__double_as_longlong(b_out[row]) != kRowUnsolved) continue;
        // 1. the four digit histograms in one read, and the finiteness check
        for (int e = tid; e < kHistCopies_rows * 4 * 256; e += NT) hist[e] = 0u;
        if (tid == 0) { s_bad = !(k > 0.0 && k < (double)n); s_skip = 0; }
        __syncthreads();
        {
            int bad = 0;
            uint32_t* hl = hist + (lane & (kHistCopies_rows - 1)) * 1024;
            for (int i = tid; i < n; i += NT) {
                const float v = rr[i];
                bad |= !finite_f(v);
                const uint32_t key = f2key(v);
#pragma unroll
                for (int q = 0; q < 4; ++q) atomicAdd(&hl[q * 256 + ((key >> (8 * q)) & 0xFFu)], 1u);
            }
            if (bad) atomicOr(&s_bad, 1);
        }
        __syncthreads();
        // exclusive digit offsets per position; a position whose digit is the
        // same for every key (one bin holds n) needs no pass
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t tot = 0u;
            if (tid < 256)
#pragma unroll
                for (int c = 0; c < kHistCopies_rows; ++c) tot += hist[c * 1024 + q * 256 + tid];
            const uint32_t ex = block_exclusive_scan<NT>(tot, nullptr, scr);
            if (tid < 256) {
                offs[q * 256 + tid] = ex;
                if (q > 0 && tot == (uint32_t)n) atomicOr(&s_skip, 1 << q);
            }
        }
        __syncthreads();
        const int skip = s_skip;
        // 2. the passes (the first always runs: it turns the scores into keys)
        const uint32_t* src = reinterpret_cast<const uint32_t*>(rr);
        bool src_float = true;
        uint32_t* dst = bufA;
        for (int q = 0; q < 4; ++q) {
            if ((skip >> q) & 1) continue;  // workgroup-uniform
            const int shift = 8 * q;
            for (int c0 = 0; c0 < n; c0 += kLongChunk) {
                const int cc = n - c0 < kLongChunk ? n - c0 : kLongChunk;
                uint32_t kr[kLongItems], rk[kLongItems];
#pragma unroll
                for (int i = 0; i < kLongItems; ++i) {
                    const int o = (w * kLongItems + i) * 64 + lane;
                    kr[i] = o < cc ? (src_float ? f2key(__uint_as_float(src[c0 + o])) : src[c0 + o]) : 0u;
                }
                for (int e = tid; e < 256 * NW; e += NT) cnt[e] = 0u;
                __syncthreads();
                // stable ranks: per wave and digit, in row order
                volatile uint32_t* vc = cnt;
#pragma unroll
                for (int i = 0; i < kLongItems; ++i) {
                    const bool valid = (w * kLongItems + i) * 64 + lane < cc;
                    const unsigned long long act = ballot(valid);
                    rk[i] = 0u;
                    if (act != 0ull) {
                        const uint32_t d = (kr[i] >> shift) & 0xFFu;
                        const unsigned long long peers = match_digit8(d, act);
                        const uint32_t b0 = vc[d * NW + w];
                        rk[i] = b0 + (uint32_t)mbcnt(peers);
                        if (valid && lane == 63 - __clzll(peers)) vc[d * NW + w] = b0 + (uint32_t)popc64(peers);
                    }
                }
                __syncthreads();
                // per-wave exclusive offsets of each digit and the chunk's digit totals
                uint32_t tot = 0u;
                if (tid < 256) {
                    uint32_t cw[NW];
#pragma unroll
                    for (int x = 0; x < NW; ++x) cw[x] = cnt[tid * NW + x];
#pragma unroll
                    for (int x = 0; x < NW; ++x) { cnt[tid * NW + x] = tot; tot += cw[x]; }
                }
                const uint32_t lx = block_exclusive_scan<NT>(tot, nullptr, scr);
                if (tid < 256) loc[tid] = lx;
                __syncthreads();
#pragma unroll
                for (int i = 0; i < kLongItems; ++i) {
                    if ((w * kLongItems + i) * 64 + lane < cc) {
                        const uint32_t d = (kr[i] >> shift) & 0xFFu;
                        stage[loc[d] + cnt[d * NW + w] + rk[i]] = kr[i];
                    }
                }
                __syncthreads();
                // runs out at the digits' running offsets
                for (int j = tid; j < cc; j += NT) {
                    const uint32_t key = stage[j];
                    const uint32_t d = (key >> shift) & 0xFFu;
                    dst[offs[q * 256 + d] + (uint32_t)j - loc[d]] = key;
                }
                __syncthreads();
                if (tid < 256) offs[q * 256 + tid] += tot;
            }
            __syncthreads();  // the pass's writes before the next pass reads them
            src = dst;
            src_float = false;
            dst = dst == bufA ? bufB : bufA;
        }
        const uint32_t* sorted = src;
        // 3. segment aggregates and the solve over the sorted row
        const int nseg = (n + kLongChunk - 1) / kLongChunk;
        for (int sgi = 0; sgi < nseg; ++sgi) {
            const int c = n - sgi * kLongChunk < kLongChunk ? n - sgi * kLongChunk : kLongChunk;
            segment_aggregates<NT>(sorted + sgi * kLongChunk, c, inv_t, &sg_first[sgi], &sg_last[sgi], &sg_P[sgi],
                                   &sg_Bx[sgi], s_red);
            if (tid == 0) { sg_cnt[sgi] = (uint32_t)c; sg_off[sgi] = (uint32_t)(sgi * kLongChunk); }
        }
        __syncthreads();
        SegView sv{nseg, sg_first, sg_last, sg_P, sg_Bx, sg_cnt, sg_off, sorted, nullptr};
        SolveScratch sc{sc_pk, sc_pv, sc_bk, sc_bv, sc_bfx, sc_rank, nullptr, nullptr};
        Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t, key2f(sorted[0]), key2f(sorted[n - 1])};
        const SolveOut o = segment_solve<NT, kLongItems>(sv, tl, sc, s_k, s_v, s_int);
        if (tid == 0) {
            const double nanv = __longlong_as_double(0x7ff8000000000000ll);
            const double b = (s_bad || !o.ok) ? nanv : o.b;
            s_b = b;
            b_out[row] = b;
        }
        __syncthreads();
        // 4. p for the row
        const double b = s_b;
        float* pr = p + row * (long long)n;
        for (int i = tid; i < n; i += NT) {
            const float x = (float)(((double)rr[i] - b) * inv_t);
            const float e = 0.5f * __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
            pr[i] = (b == b) ? (x < 0.0f ? e : 1.0f - e) : b;
        }
        __syncthreads();  // LDS is reused by the next row
    }
}

int rows_supported_max() { return kLongMax; }

// workgroups of the long-row kernel: one round of co-resident ones at most
int rows_long_grid(long long rows) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_rows_forward_long, kLongNT, 0) != hipSuccess)
        per = 0;
    const long long g = std::max<long long>(1, (long long)cus * std::max(per, 1));
    return (int)std::min<long long>(rows, g);
}

size_t rows_long_scratch_words(long long rows, int n) { return (size_t)rows_long_grid(rows) * 2 * (size_t)n; }

void launch_rows_forward_long(const float* r, long long rows, int n, const double* k_rows, double k_all, double t,
                              float* p, double* b_out, uint32_t* scratch, hipStream_t st) {
    hipLaunchKernelGGL(k_rows_steps_long, dim3((unsigned)rows), dim3(kLongStepsNT), 0, st, r, n, k_rows, k_all, t,
                       1.0 / t, p, b_out);
    hipLaunchKernelGGL(k_rows_forward_long, dim3((unsigned)rows_long_grid(rows)), dim3(kLongNT), 0, st, r, n, rows,
                       k_rows, k_all, t, 1.0 / t, p, b_out, scratch);
}

void launch_rows_forward(const float* r, long long rows, int n, const double* k_rows, double k_all, double t, float* p,
                         double* b_out, hipStream_t st) {
    const double inv_t = 1.0 / t;
    const dim3 grid((unsigned)rows);
    if (n <= 256)
        hipLaunchKernelGGL((k_rows_forward<64, 4>), grid, dim3(64), 0, st, r, n, k_rows, k_all, t, inv_t, p, b_out);
    else if (n <= 4096)
        hipLaunchKernelGGL((k_rows_forward<256, 16>), grid, dim3(256), 0, st, r, n, k_rows, k_all, t, inv_t, p, b_out);
    else
        hipLaunchKernelGGL((k_rows_forward<1024, 16>), grid, dim3(1024), 0, st, r, n, k_rows, k_all, t, inv_t, p,
                           b_out);
}

void launch_rows_vjp(const float* r, const float* g, long long rows, int n, double t, const double* b, float* grad,
                     hipStream_t st) {
    const double inv_t = 1.0 / t;
    const float l2 = (float)(std::log2(0.5 * inv_t) + 32.0);
    const dim3 grid((unsigned)rows);
    if (n <= 256) hipLaunchKernelGGL(k_rows_vjp<64>, grid, dim3(64), 0, st, r, g, n, inv_t, l2, b, grad);
    else if (n <= 4096) hipLaunchKernelGGL(k_rows_vjp<256>, grid, dim3(256), 0, st, r, g, n, inv_t, l2, b, grad);
    else hipLaunchKernelGGL(k_rows_vjp<1024>, grid, dim3(1024), 0, st, r, g, n, inv_t, l2, b, grad);
}

}  // namespace lapsum
