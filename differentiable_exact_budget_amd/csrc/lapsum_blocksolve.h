// Workgroup-level building blocks of the Fast LapSum solver (gfx950):
//  * an LDS-resident LSD radix sort of up to NT*ITEMS keys, and
//  * the threshold solve over sorted segments: the stable prefix/suffix
//    "threshold curve" scan, the interval search and the closed-form root
//    (Fast LapSum paper, gist.science summary section 2.2, full-sort solver:
//    one stable prefix/suffix scan over the sorted scores, an index search
//    and a closed-form root in the interval where the budget balances).
//
// Notation.  Sorted scores v_0 <= ... <= v_{m-1} (the band, or all scores),
// plus optional tails from the streaming pass: c_R scores >= a_R folded
// into S_R = sum e^{(a_R - r)/t} and the scores < a_L folded into
// S_L = sum e^{(r - a_L)/t}.  Then, with every exponent <= 0,
//   P_j = sum_{i<=j} e^{(v_i - v_j)/t} + S_L e^{(a_L - v_j)/t}      (inclusive)
//   B_j = sum_{i>j}  e^{(v_j - v_i)/t} + S_R e^{(v_j - a_R)/t}      (exclusive)
//   G(v_j) = P_j/2 + (m - 1 - j) + c_R - B_j/2,
// and on [v_j, v_{j+1}) with w = e^{(x - v_j)/t}:
//   G(x) - k = P_j/(2w) + D - B_j w/2,   D = (m - 1 - j) + c_R - k,
// whose root is w = (D + sqrt(D^2 + P_j B_j))/B_j, evaluated in log space.
// The suffix is always carried as e^{-gap/t} (1 + B_{j+1}), never as a
// difference of inclusive sums.
#pragma once
#include "lapsum_device.h"

namespace lapsum {

// ---------------------------------------------------------------------------
// LDS radix sort (stable LSD, 8-bit digits, wave-level multisplit ranking)
// keys: LDS array holding the m keys to sort in place.
// cnt : LDS scratch of 256 * (NT/64) words.  scr: LDS scratch >= NT/64 + 2.
// Digits on which all keys agree are skipped.
// ---------------------------------------------------------------------------
template <int NT, int ITEMS>
__device__ void block_sort_lds(uint32_t* keys, int m, uint32_t* cnt, uint32_t* scr) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
    if (m <= 1) { __syncthreads(); return; }
    if (tid == 0) { scr[0] = 0u; scr[1] = 0xFFFFFFFFu; }
    __syncthreads();
    uint32_t kor = 0u, kand = 0xFFFFFFFFu;
    for (int i = tid; i < m; i += NT) { uint32_t k = keys[i]; kor |= k; kand &= k; }
    atomicOr(&scr[0], kor);
    atomicAnd(&scr[1], kand);
    __syncthreads();
    const uint32_t diff = scr[0] ^ scr[1];
    __syncthreads();

    uint32_t kr[ITEMS];
    uint32_t rk[ITEMS];
    volatile uint32_t* vc = cnt;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 8 * pass;
        if (((diff >> shift) & 0xFFu) == 0u) continue;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int idx = (w * ITEMS + i) * 64 + lane;
            kr[i] = idx < m ? keys[idx] : 0u;
        }
        for (int e = tid; e < 256 * NW; e += NT) cnt[e] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int idx = (w * ITEMS + i) * 64 + lane;
            const bool valid = idx < m;
            const unsigned long long act = ballot(valid);
            rk[i] = 0u;
            if (act != 0ull) {  // wave-uniform
                const uint32_t d = (kr[i] >> shift) & 0xFFu;
                const unsigned long long peers = match_digit8(d, act);
                const uint32_t base = vc[d * NW + w];
                rk[i] = base + (uint32_t)mbcnt(peers);
                if (valid && lane == 63 - __clzll(peers)) vc[d * NW + w] = base + (uint32_t)popc64(peers);
            }
        }
        __syncthreads();
        // exclusive scan over (digit, wave) in digit-major order: 4 entries per thread
        {
            constexpr int PER = 256 * NW / NT;  // = 4
            uint32_t loc[PER];
            uint32_t s = 0u;
#pragma unroll
            for (int q = 0; q < PER; ++q) { loc[q] = cnt[tid * PER + q]; s += loc[q]; }
            uint32_t ex = block_exclusive_scan<NT>(s, nullptr, scr + 2);
#pragma unroll
            for (int q = 0; q < PER; ++q) { cnt[tid * PER + q] = ex; ex += loc[q]; }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int idx = (w * ITEMS + i) * 64 + lane;
            if (idx < m) {
                const uint32_t d = (kr[i] >> shift) & 0xFFu;
                keys[cnt[d * NW + w] + rk[i]] = kr[i];
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// (position, value) carries of the threshold curve.
//   forward carry (k, v): v = sum over scores <= k of e^{(score - k)/t};
//   identity (-inf, 0).
//   backward carry (k, v): v = sum over scores >= k of e^{(k - score)/t};
//   identity (+inf, 0).
// ---------------------------------------------------------------------------
LS_DEV double ecoef(double x) { return exp(x); }  // fp64, x <= 0

LS_DEV void fwd_combine(float lk, double lv, float& k, double& v, double inv_t) {
    // left (lk, lv) followed by (k, v)
    if (v == 0.0 && k == -INFINITY) { k = lk; v = lv; return; }
    if (lv != 0.0) v += ecoef(((double)lk - (double)k) * inv_t) * lv;
}
LS_DEV void bwd_combine(float& k, double& v, float rk, double rv, double inv_t) {
    // (k, v) followed by right (rk, rv)
    if (v == 0.0 && k == INFINITY) { k = rk; v = rv; return; }
    if (rv != 0.0) v += ecoef(((double)k - (double)rk) * inv_t) * rv;
}

// exclusive scans over the NT threads of the workgroup (Hillis-Steele in LDS)
template <int NT>
LS_DEV void block_scan_fwd_excl(float& k, double& v, float* sk, double* sv, double inv_t) {
    const int tid = threadIdx.x;
    sk[tid] = k; sv[tid] = v;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
        float lk = -INFINITY; double lv = 0.0;
        const bool has = tid >= o;
        if (has) { lk = sk[tid - o]; lv = sv[tid - o]; }
        __syncthreads();
        if (has) fwd_combine(lk, lv, k, v, inv_t);
        sk[tid] = k; sv[tid] = v;
        __syncthreads();
    }
    float ek = -INFINITY; double ev = 0.0;
    if (tid > 0) { ek = sk[tid - 1]; ev = sv[tid - 1]; }
    __syncthreads();
    k = ek; v = ev;
}

template <int NT>
LS_DEV void block_scan_bwd_excl(float& k, double& v, float* sk, double* sv, double inv_t) {
    const int tid = threadIdx.x;
    sk[tid] = k; sv[tid] = v;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
        float rk = INFINITY; double rv = 0.0;
        const bool has = tid + o < NT;
        if (has) { rk = sk[tid + o]; rv = sv[tid + o]; }
        __syncthreads();
        if (has) bwd_combine(k, v, rk, rv, inv_t);
        sk[tid] = k; sv[tid] = v;
        __syncthreads();
    }
    float ek = INFINITY; double ev = 0.0;
    if (tid + 1 < NT) { ek = sk[tid + 1]; ev = sv[tid + 1]; }
    __syncthreads();
    k = ek; v = ev;
}

template <int NT>
LS_DEV int block_max_int(int x, int* s) {
    if (threadIdx.x == 0) *s = -1;
    __syncthreads();
    if (x >= 0) atomicMax(s, x);
    __syncthreads();
    int r = *s;
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// Threshold solve over sorted segments.
// ---------------------------------------------------------------------------
struct SegView {
    int nseg;
    const float* first;    // first (smallest) score of each segment
    const float* last;     // last (largest) score
    const double* P;       // sum_i e^{(v_i - last)/t} over the segment
    const double* Bx;      // sum_{i > first} e^{(first - v_i)/t} over the segment
    const uint32_t* cnt;   // scores in the segment (0 = empty)
    const uint32_t* off;   // offset of the segment's keys in `keys`
    const uint32_t* keys;  // sorted order-preserving keys (global or LDS)
};

struct Tails {
    float aL, aR;          // bracket ends (+-inf when open)
    double S_L, S_R;       // tail sums
    double m;              // scores in the segments
    double c_R;            // scores >= a_R
    double k, t, inv_t;
};

struct SolveScratch {      // global scratch
    float* pk; double* pv;     // per segment: forward carry before it
    float* bk; double* bv;     // per segment: backward carry after it
    double* bfx;               // per segment: exclusive suffix at its first score
    uint32_t* rank;            // per segment: sorted index of its first score
    double* eP; double* eB;    // per score of the root segment: P_j, B_j
};

struct SolveOut { double b; long long jstar; int ok; };

// log-space closed-form root of  A/(2w) + D - B w/2 = 0  (w > 0)
LS_DEV double log_root(double lnA, double lnB, double D) {
    const double AB = (lnA == -INFINITY || lnB == -INFINITY) ? 0.0 : exp(lnA + lnB);
    const double s = sqrt(D * D + AB);
    if (D > 0.0) return log(D + s) - lnB;
    if (D < 0.0) return lnA - log(s - D);
    return 0.5 * (lnA - lnB);
}

// Runs on all NT threads of one workgroup; result valid in thread 0.
template <int NT, int EMAX>
__device__ SolveOut segment_solve(const SegView sv, const Tails tl, const SolveScratch sc,
                                  float* s_k, double* s_v, int* s_int) {
    const int tid = threadIdx.x;
    const double inv_t = tl.inv_t;
    const int nseg = sv.nseg;
    const int per = (nseg + NT - 1) / NT;
    const int s0 = min(nseg, tid * per), s1 = min(nseg, s0 + per);

    // ---- phase 1: forward carries across segments, and segment ranks ----
    float ak = -INFINITY; double av = 0.0; uint32_t rc = 0u;
    for (int s = s0; s < s1; ++s) {
        const uint32_t c = sv.cnt[s];
        if (c) { float lk = ak; double lv = av; ak = sv.last[s]; av = sv.P[s]; fwd_combine(lk, lv, ak, av, inv_t); }
        rc += c;
    }
    uint32_t rbase = block_exclusive_scan<NT>(rc, nullptr, (uint32_t*)s_int);
    block_scan_fwd_excl<NT>(ak, av, s_k, s_v, inv_t);
    {   // the lower tail precedes everything
        float ck = ak; double cv = av;
        float tk = -INFINITY; double tv = 0.0;
        if (tl.S_L > 0.0 && tl.aL > -INFINITY) { tk = tl.aL; tv = tl.S_L; }
        ak = tk; av = tv;
        fwd_combine(ak, av, ck, cv, inv_t);  // (tail) then (threads before)
        ak = ck; av = cv;
    }
    for (int s = s0; s < s1; ++s) {
        const uint32_t c = sv.cnt[s];
        sc.pk[s] = ak; sc.pv[s] = av; sc.rank[s] = rbase;
        rbase += c;
        if (c) { float lk = ak; double lv = av; ak = sv.last[s]; av = sv.P[s]; fwd_combine(lk, lv, ak, av, inv_t); }
    }
    // ---- phase 2: backward carries across segments ----
    float bk = INFINITY; double bvv = 0.0;
    for (int s = s1 - 1; s >= s0; --s) {
        if (sv.cnt[s]) { float k2 = sv.first[s]; double v2 = 1.0 + sv.Bx[s]; bwd_combine(k2, v2, bk, bvv, inv_t); bk = k2; bvv = v2; }
    }
    block_scan_bwd_excl<NT>(bk, bvv, s_k, s_v, inv_t);
    {   // the upper tail follows everything
        if (tl.S_R > 0.0 && tl.aR < INFINITY) bwd_combine(bk, bvv, tl.aR, tl.S_R, inv_t);
    }
    for (int s = s1 - 1; s >= s0; --s) {
        sc.bk[s] = bk; sc.bv[s] = bvv;
        if (sv.cnt[s]) { float k2 = sv.first[s]; double v2 = 1.0 + sv.Bx[s]; bwd_combine(k2, v2, bk, bvv, inv_t); bk = k2; bvv = v2; }
    }
    __syncthreads();
    // ---- phase 3: G at every segment's first score; last segment with G >= k ----
    int cand = -1;
    for (int s = s0; s < s1; ++s) {
        if (!sv.cnt[s]) continue;
        const float f = sv.first[s];
        const double Pf = 1.0 + (sc.pv[s] != 0.0 ? ecoef(((double)sc.pk[s] - (double)f) * inv_t) * sc.pv[s] : 0.0);
        const double Bf = sv.Bx[s] + (sc.bv[s] != 0.0 ? ecoef(((double)f - (double)sc.bk[s]) * inv_t) * sc.bv[s] : 0.0);
        sc.bfx[s] = Bf;
        const double G = 0.5 * Pf + (tl.m - 1.0 - (double)sc.rank[s]) + tl.c_R - 0.5 * Bf;
        if (G >= tl.k) cand = s;
    }
    const int sstar = block_max_int<NT>(cand, s_int);
    __threadfence_block();
    __syncthreads();

    SolveOut out; out.b = 0.0; out.jstar = -1; out.ok = 1;
    int jl = -1;
    uint32_t cS = 0u, offS = 0u, rankS = 0u;
    if (sstar >= 0) {
        // ---- phase 4: per-score curve inside the root segment ----
        cS = sv.cnt[sstar]; offS = sv.off[sstar]; rankS = sc.rank[sstar];
        const int E = ((int)cS + NT - 1) / NT;
        const int e0 = min((int)cS, tid * E), e1 = min((int)cS, e0 + E);
        float vv[EMAX];
        double al[EMAX];   // al[q] = e^{(v_{j-1} - v_j)/t} for j = e0 + q (q > 0)
#pragma unroll
        for (int q = 0; q < EMAX; ++q) {
            const int j = e0 + q;
            vv[q] = (j < e1) ? key2f(sv.keys[offS + j]) : 0.0f;
        }
#pragma unroll
        for (int q = 1; q < EMAX; ++q) {
            al[q] = (e0 + q < e1) ? ecoef(((double)vv[q - 1] - (double)vv[q]) * inv_t) : 0.0;
        }
        al[0] = 0.0;
        // forward: local prefix then workgroup carry
        float fk = -INFINITY; double fv = 0.0;
#pragma unroll
        for (int q = 0; q < EMAX; ++q) {
            if (e0 + q < e1) { fv = 1.0 + (q > 0 ? al[q] * fv : 0.0); fk = vv[q]; }
        }
        block_scan_fwd_excl<NT>(fk, fv, s_k, s_v, inv_t);
        {   // carry from everything before the segment
            float pk0 = sc.pk[sstar]; double pv0 = sc.pv[sstar];
            float ck = fk; double cv = fv;
            fwd_combine(pk0, pv0, ck, cv, inv_t);
            fk = ck; fv = cv;
        }
        double Pj[EMAX];
#pragma unroll
        for (int q = 0; q < EMAX; ++q) {
            if (e0 + q < e1) {
                double carry = (q == 0) ? (fv != 0.0 ? ecoef(((double)fk - (double)vv[0]) * inv_t) * fv : 0.0)
                                        : al[q] * Pj[q - 1];
                Pj[q] = 1.0 + carry;
            }
        }
        // backward: local inclusive suffix then workgroup carry
        float rk2 = INFINITY; double rv2 = 0.0;
#pragma unroll
        for (int q = EMAX - 1; q >= 0; --q) {
            if (e0 + q < e1) {
                rv2 = 1.0 + (rv2 != 0.0 ? ecoef(((double)vv[q] - (double)rk2) * inv_t) * rv2 : 0.0);
                rk2 = vv[q];
            }
        }
        block_scan_bwd_excl<NT>(rk2, rv2, s_k, s_v, inv_t);
        {
            float bk0 = sc.bk[sstar]; double bv0 = sc.bv[sstar];
            bwd_combine(rk2, rv2, bk0, bv0, inv_t);
        }
        double Bj[EMAX];
        int myj = -1;
#pragma unroll
        for (int q = EMAX - 1; q >= 0; --q) {
            if (e0 + q < e1) {
                double bx;
                if (q + 1 < EMAX && e0 + q + 1 < e1) bx = al[q + 1] * (1.0 + Bj[q + 1]);
                else bx = (rv2 != 0.0) ? ecoef(((double)vv[q] - (double)rk2) * inv_t) * rv2 : 0.0;
                Bj[q] = bx;
            }
        }
#pragma unroll
        for (int q = 0; q < EMAX; ++q) {
            const int j = e0 + q;
            if (j < e1) {
                sc.eP[j] = Pj[q];
                sc.eB[j] = Bj[q];
                const double G = 0.5 * Pj[q] + (tl.m - 1.0 - (double)(rankS + (uint32_t)j)) + tl.c_R - 0.5 * Bj[q];
                if (G >= tl.k) myj = j;
            }
        }
        jl = block_max_int<NT>(myj, s_int);
        if (jl < 0) jl = 0;  // the segment's first score passed in phase 3
        __threadfence_block();
        __syncthreads();
    }

    if (tid == 0) {
        double ref, lnA, lnB, D, clo, chi;
        if (sstar >= 0) {
            const float lo = key2f(sv.keys[offS + jl]);
            ref = lo; clo = lo;
            lnA = log(sc.eP[jl]);
            const double J = (double)(rankS + (uint32_t)jl);
            D = (tl.m - 1.0 - J) + tl.c_R - tl.k;
            out.jstar = (long long)(rankS + (uint32_t)jl);
            float vnext = 0.0f; double Bnext = 0.0; bool has_next = false;
            if ((uint32_t)jl + 1u < cS) { vnext = key2f(sv.keys[offS + jl + 1]); Bnext = sc.eB[jl + 1]; has_next = true; }
            else {
                for (int s = sstar + 1; s < nseg; ++s)
                    if (sv.cnt[s]) { vnext = sv.first[s]; Bnext = sc.bfx[s]; has_next = true; break; }
            }
            if (has_next) { chi = vnext; lnB = ((double)lo - (double)vnext) * inv_t + log1p(Bnext); }
            else {
                chi = tl.aR;
                lnB = (tl.S_R > 0.0 && tl.aR < INFINITY) ? log(tl.S_R) + ((double)lo - (double)tl.aR) * inv_t : -INFINITY;
            }
        } else {
            int s0n = -1;
            for (int s = 0; s < nseg; ++s) if (sv.cnt[s]) { s0n = s; break; }
            D = tl.m + tl.c_R - tl.k;
            if (tl.aL > -INFINITY) {
                ref = tl.aL; clo = tl.aL;
                lnA = tl.S_L > 0.0 ? log(tl.S_L) : -INFINITY;
                if (s0n >= 0) { chi = sv.first[s0n]; lnB = ((double)tl.aL - chi) * inv_t + log1p(sc.bfx[s0n]); }
                else {
                    chi = tl.aR;
                    lnB = (tl.S_R > 0.0 && tl.aR < INFINITY) ? log(tl.S_R) + ((double)tl.aL - (double)tl.aR) * inv_t : -INFINITY;
                }
            } else {
                clo = -INFINITY; lnA = -INFINITY;
                if (s0n >= 0) { ref = sv.first[s0n]; chi = ref; lnB = log1p(sc.bfx[s0n]); }
                else { ref = tl.aR; chi = tl.aR; lnB = tl.S_R > 0.0 ? log(tl.S_R) : -INFINITY; }
            }
            out.jstar = -1;
        }
        const double lnw = log_root(lnA, lnB, D);
        double b = ref + tl.t * lnw;
        if (b < clo) b = clo;
        if (b > chi) b = chi;
        out.b = b;
        out.ok = (b == b) && (b > -INFINITY) && (b < INFINITY);
    }
    return out;
}

}  // namespace lapsum
