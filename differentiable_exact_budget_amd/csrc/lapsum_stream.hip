// Streaming (HBM-bound) kernels of the Fast LapSum solver (gfx950).
//
//  k_filter      the single streaming pass of the bracketing path (Fast
//                LapSum paper, gist.science section 2.2, "Streaming y
//                Filtrado"): scores below a_L are folded into
//                S_L = sum e^{(r - a_L)/t}, scores at or above a_R into
//                S_R = sum e^{(a_R - r)/t}, and the middle band is kept,
//                already split into value-ordered buckets.  Its last
//                workgroup reduces the per-workgroup partials in a fixed
//                order and hands the totals to the host (certification).
//  k_probs       p_i = F((r_i - b)/t) and sum p (section 2.1).
//  k_vjp_reduce  sum f g and sum f, f_i = e^{-|r_i - b|/t}/2 (section 2.1, VJP);
//                the last workgroup forms c = sum f g / sum f.
//  k_vjp_apply   grad_i = (f_i / t)(g_i - c).
//
// Memory access: 16-byte loads/stores in a grid-stride loop with four loads
// in flight per thread (the host picks the scalar variant for misaligned
// pointers).  Reductions: fp32 within one float4, fp64 across float4s and
// workgroups, combined in a fixed order (bitwise reproducible).
#include <cmath>

#include "lapsum_launch.h"

namespace lapsum {

int stream_blocks(long long n) {
    long long per_block = (long long)kStreamThreads * 16;  // >= 16 scores per thread
    long long b = (n + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > kMaxStreamBlocks) b = kMaxStreamBlocks;
    return (int)b;
}

struct FilterPart {
    double S[4];               // S_L, S_R, B_L, B_R
    unsigned long long c[2];   // below, above
    float mn, mx;              // smallest and largest score seen
    int nan;                   // a NaN was seen
    int pad;
};

// ---------------------------------------------------------------------------
// streaming filter
// ---------------------------------------------------------------------------
struct FilterState {
    float aL, aR, ls, ng_f;
    int ng, J, cap;
    const float* sp;
    const float* iw;
    uint32_t* bucket_cnt;
    uint32_t* bucket_vals;
};

// band score: bucket by splitter gap, then equal-width sub-bucket (monotone in v)
LS_DEV void filter_band(const FilterState& fs, float v, double& BL, int& nan, int& ovf) {
    if (v != v) { nan = 1; return; }
    int g = 0;
    for (int step = 128; step > 0; step >>= 1)
        if (g + step < fs.ng && fs.sp[g + step] <= v) g += step;
    int sub = 0;
    const float iwg = fs.iw[g];
    if (fs.J > 1 && iwg > 0.0f) {
        const float f = (v - fs.sp[g]) * iwg;
        sub = f < (float)(fs.J - 1) ? (int)f : fs.J - 1;
    }
    const int bkt = g * fs.J + sub;
    if (fs.aL > -INFINITY) BL += (double)__builtin_amdgcn_exp2f(-(v - fs.aL) * fs.ls);
    const uint32_t pos = atomicAdd(&fs.bucket_cnt[bkt], 1u);
    if (pos < (uint32_t)fs.cap) fs.bucket_vals[(size_t)bkt * (size_t)fs.cap + pos] = __float_as_uint(v);
    else ovf = 1;
}

template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void k_filter(const float* __restrict__ r, long long n, float ls,
                                                            Ctl* ctl, const float* __restrict__ sp_g,
                                                            const float* __restrict__ iw_g, uint32_t* bucket_cnt,
                                                            uint32_t* bucket_vals, int cap, FilterPart* part,
                                                            HostSummary* hs, unsigned int seq) {
    __shared__ float sp[kMaxBuckets + 1];
    __shared__ float iw[kMaxBuckets];
    __shared__ double s_red[kStreamThreads / 64];
    __shared__ unsigned long long s_redu[kStreamThreads / 64];
    __shared__ uint32_t s_mn, s_mx;
    __shared__ int s_nan;
    __shared__ unsigned long long s_mxb;
    __shared__ int s_last;
    const int tid = threadIdx.x;
    FilterState fs;
    fs.aL = ctl->aL; fs.aR = ctl->aR; fs.ls = ls;
    fs.ng = ctl->ng; fs.J = ctl->J; fs.cap = cap;
    for (int i = tid; i <= fs.ng; i += kStreamThreads) sp[i] = sp_g[i];
    for (int i = tid; i < fs.ng; i += kStreamThreads) iw[i] = iw_g[i];
    if (tid == 0) { s_mn = 0xFFFFFFFFu; s_mx = 0u; s_nan = 0; s_mxb = 0ull; }
    fs.sp = sp; fs.iw = iw; fs.bucket_cnt = bucket_cnt; fs.bucket_vals = bucket_vals;
    __syncthreads();

    double SL = 0.0, SR = 0.0, BL = 0.0, BR = 0.0;
    unsigned long long cLw = 0ull, cRw = 0ull;  // wave totals from ballots (same in every lane)
    unsigned long long cLl = 0ull, cRl = 0ull;  // this lane's own counts (tail and scalar path)
    float mn = INFINITY, mx = -INFINITY;
    int nan = 0, ovf = 0;
    const float aL = fs.aL, aR = fs.aR;

    // one score, every lane of the wave active (ballots are wave-wide)
    auto elem = [&](float v, float& eL, float& eR) {
        const bool below = v < aL;
        const bool above = v >= aR;
        const float e = __builtin_amdgcn_exp2f(-fabsf(v - (below ? aL : aR)) * ls);
        eL += below ? e : 0.0f;
        eR += above ? e : 0.0f;
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
        cLw += (unsigned long long)popc64(ballot(below));
        cRw += (unsigned long long)popc64(ballot(above));
        const bool band = !(below || above);
        if (ballot(band)) {
            if (band) {
                BR += (double)e;
                filter_band(fs, v, BL, nan, ovf);
            }
        }
    };
    // one score, per-lane bookkeeping (no ballots)
    auto elem_lane = [&](float v) {
        const bool below = v < aL;
        const bool above = v >= aR;
        const float e = __builtin_amdgcn_exp2f(-fabsf(v - (below ? aL : aR)) * ls);
        if (below) SL += (double)e;
        if (above) SR += (double)e;
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
        cLl += below;
        cRl += above;
        if (!(below || above)) { BR += (double)e; filter_band(fs, v, BL, nan, ovf); }
    };
    auto quad = [&](float4 q) {
        float eL = 0.0f, eR = 0.0f;
        elem(q.x, eL, eR);
        elem(q.y, eL, eR);
        elem(q.z, eL, eR);
        elem(q.w, eL, eR);
        SL += (double)eL;
        SR += (double)eR;
    };

    const long long stride = (long long)gridDim.x * kStreamThreads;
    const long long gt = (long long)blockIdx.x * kStreamThreads + tid;
    if (VEC) {
        const long long n4 = n >> 2;
        const float4* r4 = reinterpret_cast<const float4*>(r);
        long long i = gt;
        // main loop: the trip test uses the wave's last lane, so the whole wave
        // iterates together and the ballot counts see every lane
        const long long to_last_lane = 63 - lane_id();
        for (; i + to_last_lane + 3 * stride < n4; i += 4 * stride) {
            const float4 q0 = r4[i], q1 = r4[i + stride], q2 = r4[i + 2 * stride], q3 = r4[i + 3 * stride];
            quad(q0); quad(q1); quad(q2); quad(q3);
        }
        for (; i < n4; i += stride) {
            const float4 q = r4[i];
            elem_lane(q.x); elem_lane(q.y); elem_lane(q.z); elem_lane(q.w);
        }
        if (blockIdx.x == 0 && tid < 4) {
            const long long j = (n4 << 2) + tid;
            if (j < n) elem_lane(r[j]);
        }
    } else {
        for (long long i = gt; i < n; i += stride) elem_lane(r[i]);
    }
    (void)ovf;  // per-bucket overflow is decided from the bucket counts below

    // ---- workgroup reduction (fixed order) ----
    const unsigned long long myL = cLl + (lane_id() == 0 ? cLw : 0ull);
    const unsigned long long myR = cRl + (lane_id() == 0 ? cRw : 0ull);
    const double tS0 = block_sum<kStreamThreads>(SL, s_red);
    const double tS1 = block_sum<kStreamThreads>(SR, s_red);
    const double tS2 = block_sum<kStreamThreads>(BL, s_red);
    const double tS3 = block_sum<kStreamThreads>(BR, s_red);
    const unsigned long long tcL = block_sum_u64<kStreamThreads>(myL, s_redu);
    const unsigned long long tcR = block_sum_u64<kStreamThreads>(myR, s_redu);
    if (mn <= mx) { atomicMin(&s_mn, f2key(mn)); atomicMax(&s_mx, f2key(mx)); }
    if (nan) atomicOr(&s_nan, 1);
    __syncthreads();
    if (tid == 0) {
        FilterPart& fp = part[blockIdx.x];
        fp.S[0] = tS0; fp.S[1] = tS1; fp.S[2] = tS2; fp.S[3] = tS3;
        fp.c[0] = tcL; fp.c[1] = tcR;
        fp.mn = (s_mn == 0xFFFFFFFFu) ? INFINITY : key2f(s_mn);
        fp.mx = (s_mx == 0u) ? -INFINITY : key2f(s_mx);
        fp.nan = s_nan;
    }
    if (!last_block_ticket(&ctl->done[kDoneFilter], &s_last)) return;

    // ---- last workgroup: totals in a fixed order, bucket statistics, hand-off ----
    if (tid == 0) { s_mn = 0xFFFFFFFFu; s_mx = 0u; s_nan = 0; }
    __syncthreads();
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    unsigned long long u0 = 0ull, u1 = 0ull;
    for (unsigned b = tid; b < gridDim.x; b += kStreamThreads) {
        const FilterPart& fp = part[b];
        a0 += fp.S[0]; a1 += fp.S[1]; a2 += fp.S[2]; a3 += fp.S[3];
        u0 += fp.c[0]; u1 += fp.c[1];
        if (fp.nan) atomicOr(&s_nan, 1);
        if (fp.mn <= fp.mx) { atomicMin(&s_mn, f2key(fp.mn)); atomicMax(&s_mx, f2key(fp.mx)); }
    }
    const double T0 = block_sum<kStreamThreads>(a0, s_red);
    const double T1 = block_sum<kStreamThreads>(a1, s_red);
    const double T2 = block_sum<kStreamThreads>(a2, s_red);
    const double T3 = block_sum<kStreamThreads>(a3, s_red);
    const unsigned long long U0 = block_sum_u64<kStreamThreads>(u0, s_redu);
    const unsigned long long U1 = block_sum_u64<kStreamThreads>(u1, s_redu);
    unsigned long long mloc = 0ull, mxb = 0ull;
    const int nb = ctl->nb;
    for (int b = tid; b < nb; b += kStreamThreads) {
        const unsigned long long c = bucket_cnt[b];
        mloc += c;
        mxb = c > mxb ? c : mxb;
    }
    const unsigned long long M = block_sum_u64<kStreamThreads>(mloc, s_redu);
    atomicMax(&s_mxb, mxb);
    __syncthreads();
    if (tid == 0) {
        int flags = 0;
        const float gmn = (s_mn == 0xFFFFFFFFu) ? INFINITY : key2f(s_mn);
        const float gmx = (s_mx == 0u) ? -INFINITY : key2f(s_mx);
        if (s_nan || !finite_f(gmn) || !finite_f(gmx)) flags |= kFlagNonFinite;
        if (s_mxb > (unsigned long long)cap) flags |= kFlagOverflow;
        ctl->S_L = T0; ctl->S_R = T1; ctl->B_L = T2; ctl->B_R = T3;
        ctl->c_L = U0; ctl->c_R = U1; ctl->m = M;
        ctl->flags = flags;
        ctl->done[kDoneFilter] = 0u;
        if (hs) {
            hs->c_L = U0; hs->m = M; hs->c_R = U1;
            hs->S_L = T0; hs->S_R = T1; hs->B_L = T2; hs->B_R = T3;
            hs->aL = fs.aL; hs->aR = fs.aR;
            hs->flags = flags; hs->nb = nb; hs->max_bucket = s_mxb;
            __threadfence_system();
            hs->seq = seq;
            __threadfence_system();
        }
    }
}

void launch_filter(const float* r, long long n, double t, Ctl* ctl, const float* sp, const float* iw,
                   uint32_t* bucket_cnt, uint32_t* bucket_vals, int cap, double* part, unsigned long long* /*partc*/,
                   HostSummary* hs_dev, unsigned int seq, hipStream_t st) {
    const int blocks = stream_blocks(n);
    const float ls = (float)(1.4426950408889634 / t);
    FilterPart* fp = reinterpret_cast<FilterPart*>(part);
    if ((reinterpret_cast<uintptr_t>(r) & 15u) == 0u)
        hipLaunchKernelGGL(k_filter<true>, dim3(blocks), dim3(kStreamThreads), 0, st, r, n, ls, ctl, sp, iw,
                           bucket_cnt, bucket_vals, cap, fp, hs_dev, seq);
    else
        hipLaunchKernelGGL(k_filter<false>, dim3(blocks), dim3(kStreamThreads), 0, st, r, n, ls, ctl, sp, iw,
                           bucket_cnt, bucket_vals, cap, fp, hs_dev, seq);
}

// ---------------------------------------------------------------------------
// p write-out
// ---------------------------------------------------------------------------
LS_DEV float lap_cdf_f(float x) {
    const float e = 0.5f * __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    return x < 0.0f ? e : 1.0f - e;
}

template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void k_probs(const float* __restrict__ r, long long n, double inv_t,
                                                           float* __restrict__ p, Ctl* ctl, double* part) {
    __shared__ double s_red[kStreamThreads / 64];
    __shared__ int s_last;
    const double b = ctl->b;
    const int tid = threadIdx.x;
    double sum = 0.0;
    const long long stride = (long long)gridDim.x * kStreamThreads;
    const long long gt = (long long)blockIdx.x * kStreamThreads + tid;
    auto one = [&](float v) -> float {
        const float x = (float)(((double)v - b) * inv_t);
        const float q = lap_cdf_f(x);
        sum += (double)q;
        return q;
    };
    if (VEC) {
        const long long n4 = n >> 2;
        const float4* r4 = reinterpret_cast<const float4*>(r);
        float4* p4 = reinterpret_cast<float4*>(p);
        long long i = gt;
        for (; i + 3 * stride < n4; i += 4 * stride) {
            const float4 q0 = r4[i], q1 = r4[i + stride], q2 = r4[i + 2 * stride], q3 = r4[i + 3 * stride];
            p4[i] = make_float4(one(q0.x), one(q0.y), one(q0.z), one(q0.w));
            p4[i + stride] = make_float4(one(q1.x), one(q1.y), one(q1.z), one(q1.w));
            p4[i + 2 * stride] = make_float4(one(q2.x), one(q2.y), one(q2.z), one(q2.w));
            p4[i + 3 * stride] = make_float4(one(q3.x), one(q3.y), one(q3.z), one(q3.w));
        }
        for (; i < n4; i += stride) {
            const float4 q = r4[i];
            p4[i] = make_float4(one(q.x), one(q.y), one(q.z), one(q.w));
        }
        if (blockIdx.x == 0) {
            const long long j = (n4 << 2) + tid;
            if (tid < 4 && j < n) p[j] = one(r[j]);
        }
    } else {
        for (long long i = gt; i < n; i += stride) p[i] = one(r[i]);
    }
    const double tot = block_sum<kStreamThreads>(sum, s_red);
    if (tid == 0) part[blockIdx.x] = tot;
    if (!last_block_ticket(&ctl->done[kDoneProbs], &s_last)) return;
    double a = 0.0;
    for (unsigned bb = tid; bb < gridDim.x; bb += kStreamThreads) a += part[bb];
    const double T = block_sum<kStreamThreads>(a, s_red);
    if (tid == 0) { ctl->sum_p = T; ctl->done[kDoneProbs] = 0u; }
}

void launch_probs(const float* r, long long n, double t, float* p, Ctl* ctl, double* part, hipStream_t st) {
    const int blocks = stream_blocks(n);
    const bool vec = ((reinterpret_cast<uintptr_t>(r) | reinterpret_cast<uintptr_t>(p)) & 15u) == 0u;
    if (vec)
        hipLaunchKernelGGL(k_probs<true>, dim3(blocks), dim3(kStreamThreads), 0, st, r, n, 1.0 / t, p, ctl, part);
    else
        hipLaunchKernelGGL(k_probs<false>, dim3(blocks), dim3(kStreamThreads), 0, st, r, n, 1.0 / t, p, ctl, part);
}

// ---------------------------------------------------------------------------
// VJP
// ---------------------------------------------------------------------------
LS_DEV float lap_pdf_f(float x) { return 0.5f * __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f); }

template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void k_vjp_reduce(const float* __restrict__ r, const float* __restrict__ g,
                                                                long long n, const double* bptr, double inv_t,
                                                                Ctl* ctl, double* part) {
    __shared__ double s_red[kStreamThreads / 64];
    __shared__ int s_last;
    const double b = *bptr;
    const int tid = threadIdx.x;
    double sfg = 0.0, sf = 0.0;
    const long long stride = (long long)gridDim.x * kStreamThreads;
    const long long gt = (long long)blockIdx.x * kStreamThreads + tid;
    auto quad = [&](float4 q, float4 gg) {
        const float f0 = lap_pdf_f((float)(((double)q.x - b) * inv_t));
        const float f1 = lap_pdf_f((float)(((double)q.y - b) * inv_t));
        const float f2 = lap_pdf_f((float)(((double)q.z - b) * inv_t));
        const float f3 = lap_pdf_f((float)(((double)q.w - b) * inv_t));
        sfg += (double)(f0 * gg.x + f1 * gg.y) + (double)(f2 * gg.z + f3 * gg.w);
        sf += (double)((f0 + f1) + (f2 + f3));
    };
    if (VEC) {
        const long long n4 = n >> 2;
        const float4* r4 = reinterpret_cast<const float4*>(r);
        const float4* g4 = reinterpret_cast<const float4*>(g);
        long long i = gt;
        for (; i + 1 * stride < n4; i += 2 * stride) {
            const float4 q0 = r4[i], q1 = r4[i + stride];
            const float4 h0 = g4[i], h1 = g4[i + stride];
            quad(q0, h0); quad(q1, h1);
        }
        for (; i < n4; i += stride) quad(r4[i], g4[i]);
        if (blockIdx.x == 0) {
            const long long j = (n4 << 2) + tid;
            if (tid < 4 && j < n) {
                const float f = lap_pdf_f((float)(((double)r[j] - b) * inv_t));
                sfg += (double)(f * g[j]); sf += (double)f;
            }
        }
    } else {
        for (long long i = gt; i < n; i += stride) {
            const float f = lap_pdf_f((float)(((double)r[i] - b) * inv_t));
            sfg += (double)(f * g[i]); sf += (double)f;
        }
    }
    const double t0 = block_sum<kStreamThreads>(sfg, s_red);
    const double t1 = block_sum<kStreamThreads>(sf, s_red);
    if (tid == 0) { part[2 * blockIdx.x] = t0; part[2 * blockIdx.x + 1] = t1; }
    if (!last_block_ticket(&ctl->done[kDoneVjp], &s_last)) return;
    double a0 = 0.0, a1 = 0.0;
    for (unsigned bb = tid; bb < gridDim.x; bb += kStreamThreads) { a0 += part[2 * bb]; a1 += part[2 * bb + 1]; }
    const double T0 = block_sum<kStreamThreads>(a0, s_red);
    const double T1 = block_sum<kStreamThreads>(a1, s_red);
    if (tid == 0) {
        ctl->sumfg = T0; ctl->sumf = T1; ctl->c = T0 / T1;
        ctl->done[kDoneVjp] = 0u;
    }
}

// f/t = e^{-|x|}/(2t) evaluated as one exp2 with log2(1/(2t)) folded into the
// exponent (f itself underflows fp32, |x| > ~87, long before f/t does when
// t < 1), and carried at 2^32 times its value until after the product with
// (g - c): the hardware exp2 returns 0 below 2^-126, the final exact scaling
// by 2^-32 does not.
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void k_vjp_apply(const float* __restrict__ r, const float* __restrict__ g,
                                                               long long n, const double* bptr, double inv_t,
                                                               float log2_inv_2t, const Ctl* ctl,
                                                               float* __restrict__ grad) {
    const double b = *bptr;
    const float c = (float)ctl->c;
    const long long stride = (long long)gridDim.x * kStreamThreads;
    const long long gt = (long long)blockIdx.x * kStreamThreads + threadIdx.x;
    auto one = [&](float v, float gv) -> float {
        const float x = (float)(((double)v - b) * inv_t);
        const float f_over_t_2p32 = __builtin_amdgcn_exp2f(fmaf(-fabsf(x), 1.4426950408889634f, log2_inv_2t));
        return (f_over_t_2p32 * (gv - c)) * 0x1p-32f;
    };
    if (VEC) {
        const long long n4 = n >> 2;
        const float4* r4 = reinterpret_cast<const float4*>(r);
        const float4* g4 = reinterpret_cast<const float4*>(g);
        float4* o4 = reinterpret_cast<float4*>(grad);
        long long i = gt;
        for (; i + 1 * stride < n4; i += 2 * stride) {
            const float4 q0 = r4[i], q1 = r4[i + stride];
            const float4 h0 = g4[i], h1 = g4[i + stride];
            o4[i] = make_float4(one(q0.x, h0.x), one(q0.y, h0.y), one(q0.z, h0.z), one(q0.w, h0.w));
            o4[i + stride] = make_float4(one(q1.x, h1.x), one(q1.y, h1.y), one(q1.z, h1.z), one(q1.w, h1.w));
        }
        for (; i < n4; i += stride) {
            const float4 q = r4[i], h = g4[i];
            o4[i] = make_float4(one(q.x, h.x), one(q.y, h.y), one(q.z, h.z), one(q.w, h.w));
        }
        if (blockIdx.x == 0) {
            const long long j = (n4 << 2) + threadIdx.x;
            if (threadIdx.x < 4 && j < n) grad[j] = one(r[j], g[j]);
        }
    } else {
        for (long long i = gt; i < n; i += stride) grad[i] = one(r[i], g[i]);
    }
}

void launch_vjp(const float* r, const float* g, long long n, double t, const double* b, float* grad, Ctl* ctl,
                double* part, hipStream_t st, hipEvent_t* ev_mid) {
    const int blocks = stream_blocks(n);
    const bool vec = ((reinterpret_cast<uintptr_t>(r) | reinterpret_cast<uintptr_t>(g) |
                       reinterpret_cast<uintptr_t>(grad)) & 15u) == 0u;
    const double inv_t = 1.0 / t;
    if (vec) hipLaunchKernelGGL(k_vjp_reduce<true>, dim3(blocks), dim3(kStreamThreads), 0, st, r, g, n, b, inv_t, ctl, part);
    else hipLaunchKernelGGL(k_vjp_reduce<false>, dim3(blocks), dim3(kStreamThreads), 0, st, r, g, n, b, inv_t, ctl, part);
    if (ev_mid) (void)hipEventRecord(*ev_mid, st);
    const float l2 = (float)(std::log2(0.5 * inv_t) + 32.0);
    if (vec) hipLaunchKernelGGL(k_vjp_apply<true>, dim3(blocks), dim3(kStreamThreads), 0, st, r, g, n, b, inv_t, l2,
                                ctl, grad);
    else hipLaunchKernelGGL(k_vjp_apply<false>, dim3(blocks), dim3(kStreamThreads), 0, st, r, g, n, b, inv_t, l2,
                            ctl, grad);
}

// ---------------------------------------------------------------------------
// error outputs
// ---------------------------------------------------------------------------
__global__ void k_fill(float* p, long long n, float v) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}
__global__ void k_set_nan_b(Ctl* ctl, double* b_out) {
    const double nanv = __longlong_as_double(0x7ff8000000000000ll);
    ctl->b = nanv;
    if (b_out) *b_out = nanv;
}

void launch_fill(float* p, long long n, float v, hipStream_t st) {
    hipLaunchKernelGGL(k_fill, dim3(stream_blocks(n)), dim3(kStreamThreads), 0, st, p, n, v);
}
void launch_set_nan_b(Ctl* ctl, double* b_out, hipStream_t st) {
    hipLaunchKernelGGL(k_set_nan_b, dim3(1), dim3(1), 0, st, ctl, b_out);
}

}  // namespace lapsum
