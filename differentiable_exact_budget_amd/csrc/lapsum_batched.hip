// Many independent rows at once: the exact-budget operator applied per row
// (the pages' uses -- expert routing, memory selection, pruning; gist.science
// summary sections 1 and 5 -- apply it to many short vectors).  One
// workgroup per row holds the row in LDS: radix sort, the full-sort curve
// solve of one segment (gist.science section 2.2, full-sort solver), then p
// for the row; the VJP reduces and applies per row.  Rows must be contiguous
// (row i starts at i * n) and n <= 16384; the workgroup size follows n.
#include "lapsum_blocksolve.h"
#include "lapsum_launch.h"

namespace lapsum {

template <int NT, int ITEMS>
__global__ __launch_bounds__(NT) void k_rows_forward(const float* __restrict__ r, int n, const double* k_rows,
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
    const int tid = threadIdx.x;
    const long long row = blockIdx.x;
    const float* rr = r + row * (long long)n;
    const double k = k_rows ? k_rows[row] : k_all;
    if (tid == 0) s_bad = !(k > 0.0 && k < (double)n);
    __syncthreads();
    int bad = 0;
    // up to 4 keys per thread the bitonic sort (padded with the largest key)
    // beats the radix sort
    const int np = n <= 4 * NT ? max(next_pow2(n), 64) : n;
    for (int i = tid; i < np; i += NT) {
        if (i < n) {
            const float v = rr[i];
            bad |= !finite_f(v);
            keys[i] = f2key(v);
        } else {
            keys[i] = 0xFFFFFFFFu;
        }
    }
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    if (n <= 4 * NT) sort_pow2_lds<NT>(keys, np);
    else block_sort_lds<NT, ITEMS>(keys, n, cnt, scr);
    if (tid == 0) { sg_cnt = (uint32_t)n; sg_off = 0u; }
    __syncthreads();
    // the whole sorted array as one segment, no aggregates: the solve tests G
    // at every score
    SegView sv{1, nullptr, nullptr, nullptr, nullptr, &sg_cnt, &sg_off, keys, nullptr, nullptr, nullptr, nullptr};
    SolveScratch sc{&sc_pk, &sc_pv, &sc_bk, &sc_bv, &sc_bfx, &sc_rank, nullptr, nullptr};
    Tails tl{-INFINITY, INFINITY, 0.0, 0.0, (double)n, 0.0, k, t, inv_t, -INFINITY, INFINITY};
    const SolveOut o = segment_solve<NT, ITEMS>(sv, tl, sc, s_k, s_v, s_int);
    if (tid == 0) {
        const double nanv = __longlong_as_double(0x7ff8000000000000ll);
        const double b = (s_bad || !o.ok) ? nanv : o.b;
        s_b = b;
        b_out[row] = b;
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

int rows_supported_max() { return kSmallMax; }

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
