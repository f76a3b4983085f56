// Sort-free threshold solve of one workgroup over one row of scores (gfx950),
// for the batched rows.
//
// Between two consecutive scores G(x) = sum_i F((r_i - x)/t) has the closed
// form P/(2w) + N - Q w/2 with w = e^{(x - b)/t}, for any b in that interval:
// P sums e^{(r_i - b)/t} over the scores below b, Q sums e^{(b - r_i)/t} over
// those at or above it, N counts the latter (the full-sort solver's curve and
// its quadratic root in w, gist.science summary section 2.2).
//
// A step takes P, Q, N and the scores next to b in one pass and solves this
// piece for G = k.  When the root x lies in b's interval it is the root of
// G; otherwise the next step starts at x.  Carried past a score, the piece
// underestimates G to the right of b and overestimates it to the left (each
// branch of the Laplace CDF, extended, stays on one side of it), so the steps
// approach the root from one side and never step over it: each step but the
// last crosses at least one score.  The start is next to the k-th largest
// score (an MSD radix select).  A row still moving after kSolveSteps steps,
// or whose sums vanish on one side (every score there more than ~87 t from
// b, where the fp32 exponential flushes), is left to the sorting solver.
#pragma once
#include "lapsum_device.h"

namespace lapsum {

constexpr int kSolveSteps = 16;

// a thread's scores of the row: held in registers, or read from global memory
// at every pass (rows too long for registers)
template <int NT, int ITEMS>
struct RegRow {
    const float (&v)[ITEMS];
    int n;
    template <class F>
    LS_DEV void each(F&& f) const {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j)
            if (j * NT + (int)threadIdx.x < n) f(v[j]);
    }
};
template <int NT>
struct GlobalRow {
    const float* rr;
    int n;
    template <class F>
    LS_DEV void each(F&& f) const {
        constexpr int B = 16;  // loads in flight per thread
        for (int i0 = (int)threadIdx.x; i0 < n; i0 += B * NT) {
            float x[B];
#pragma unroll
            for (int q = 0; q < B; ++q) x[q] = i0 + q * NT < n ? rr[i0 + q * NT] : 0.0f;
#pragma unroll
            for (int q = 0; q < B; ++q)
                if (i0 + q * NT < n) f(x[q]);
        }
    }
};

struct StepRoot {
    double b;
    int ok;
};

// Start: the key range that shares its top 8 * DIGITS bits with the kk-th
// largest key of the row (1 <= kk <= n), and its middle as the start (all 32
// bits: the kk-th largest key itself).  Per 8-bit digit from the top, the
// keys that agree with the digits found so far are counted by digit (four
// LDS copies picked by lane), and the digit where the count from the top
// reaches the rank still to go is kept.  hist: 4 * 256 words.
template <int NT, int DIGITS, class Row>
LS_DEV uint32_t start_key(const Row& row, uint32_t kk, uint32_t* hist, uint32_t* s_sel) {
    const int tid = threadIdx.x, lane = lane_id();
    uint32_t prefix = 0u, mask = 0u, rank = kk;
    for (int shift = 24; shift >= 32 - 8 * DIGITS; shift -= 8) {
        for (int e = tid; e < 4 * 256; e += NT) hist[e] = 0u;
        __syncthreads();
        uint32_t* const hl = hist + (lane & 3) * 256;
        row.each([&](float x) {
            const uint32_t key = f2key(x);
            if ((key & mask) == prefix) atomicAdd(&hl[(key >> shift) & 0xFFu], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            // lane l holds digits 255 - 4l down to 252 - 4l
            uint32_t c[4], sl = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 255 - 4 * lane - q;
                c[q] = hist[d] + hist[256 + d] + hist[512 + d] + hist[768 + d];
                sl += c[q];
            }
            const uint32_t incl = wave_inclusive_scan(sl);
            const unsigned long long hit = ballot(incl >= rank);
            const int first = hit ? __ffsll((long long)hit) - 1 : 63;
            if (lane == first) {
                uint32_t before = incl - sl;
                int q = 0;
                while (q < 3 && before + c[q] < rank) { before += c[q]; ++q; }
                s_sel[0] = (uint32_t)(255 - 4 * lane - q);
                s_sel[1] = before;
            }
        }
        __syncthreads();
        prefix |= s_sel[0] << shift;
        mask |= 0xFFu << shift;
        rank -= s_sel[1];
        __syncthreads();  // s_sel and hist are rewritten by the next digit
    }
    if constexpr (DIGITS < 4) prefix |= 1u << (31 - 8 * DIGITS);
    return prefix;
}

// The steps from b (block sums in a fixed order: every thread takes the same
// x).  sd, su, sm: block_reduce_multi scratch for two fp64, one 64-bit and two
// 32-bit values.
template <int NT, class Row>
LS_DEV StepRoot solve_steps(const Row& row, double k, double t, double inv_t, double b, double* sd,
                            unsigned long long* su, uint32_t* sm) {
    const int n = row.n;
    for (int step = 0; step < kSolveSteps; ++step) {
        double P = 0.0, Q = 0.0;
        unsigned long long N = 0ull;
        uint32_t kb = 0u, ka = 0u;  // largest key below b; complement of the smallest key at or above b
        row.each([&](float x) {
            const double d = (double)x - b;
            const float e = __builtin_amdgcn_exp2f((float)(-fabs(d) * inv_t) * 1.4426950408889634f);
            const uint32_t key = f2key(x);
            if (d < 0.0) {
                P += (double)e;
                kb = max(kb, key);
            } else {
                Q += (double)e;
                ++N;
                ka = max(ka, ~key);
            }
        });
        double dd[2] = {P, Q};
        unsigned long long uu[1] = {N};
        uint32_t mm[2] = {kb, ka};
        block_reduce_multi<NT>(dd, uu, mm, sd, su, sm);
        __syncthreads();  // the scratch is rewritten by the next step
        P = dd[0];
        Q = dd[1];
        N = uu[0];
        const bool below = N < (unsigned long long)n, above = N > 0ull;
        if ((below && !(P > 0.0)) || (above && !(Q > 0.0))) return {b, 0};
        const double lo = below ? (double)key2f(mm[0]) : -INFINITY;  // the largest score below b
        const double hi = above ? (double)key2f(~mm[1]) : INFINITY;  // the smallest score at or above b
        // P/(2w) + D - Q w/2 = 0 with D = N - k, in the form without cancellation
        const double D = (double)N - k;
        double w;
        if (!above) w = D < 0.0 ? P / (-2.0 * D) : -1.0;
        else if (!below) w = D > 0.0 ? 2.0 * D / Q : -1.0;
        else {
            const double sq = sqrt(D * D + P * Q);
            w = D >= 0.0 ? (D + sq) / Q : P / (sq - D);
        }
        if (!(w > 0.0) || !(w < INFINITY)) return {b, 0};
        const double x = b + t * log(w);
        if (!(x == x)) return {b, 0};
        if (lo < x && x <= hi) return {x, 1};
        b = x;
    }
    return {b, 0};
}

}  // namespace lapsum
