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
#include <type_traits>
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
    // each wave ranks a contiguous run of rpw rows of 64 keys: spreading the
    // rows over all waves keeps each wave's serial chain of counter updates
    // short when m is small
    const int rows = (m + 63) >> 6;
    const int rpw = (rows + NW - 1) / NW;  // <= ITEMS
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 8 * pass;
        if (((diff >> shift) & 0xFFu) == 0u) continue;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int idx = (w * rpw + i) * 64 + lane;
            kr[i] = (i < rpw && idx < m) ? keys[idx] : 0u;
        }
        for (int e = tid; e < 256 * NW; e += NT) cnt[e] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int idx = (w * rpw + i) * 64 + lane;
            const bool valid = i < rpw && idx < m;
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
            const int idx = (w * rpw + i) * 64 + lane;
            if (i < rpw && idx < m) {
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

// exclusive scans of carries over the NT threads of the workgroup: shuffles
// inside each wave, then the wave totals scanned by wave 0 through LDS
// (sk, sv: >= NT/64 entries)
template <int NT>
LS_DEV void block_scan_fwd_excl(float& k, double& v, float* sk, double* sv, double inv_t) {
    constexpr int NW = NT / 64;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    float ik = k; double iv = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float lk = __shfl_up(ik, o, 64);
        const double lv = __shfl_up(iv, o, 64);
        if (lane >= o) fwd_combine(lk, lv, ik, iv, inv_t);
    }
    float ek = __shfl_up(ik, 1, 64);
    double ev = __shfl_up(iv, 1, 64);
    if (lane == 0) { ek = -INFINITY; ev = 0.0; }
    if (NW > 1) {
        if (lane == 63) { sk[w] = ik; sv[w] = iv; }
        __syncthreads();
        if (w == 0) {
            float tk = lane < NW ? sk[lane] : -INFINITY;
            double tv = lane < NW ? sv[lane] : 0.0;
#pragma unroll
            for (int o = 1; o < NW; o <<= 1) {
                const float lk = __shfl_up(tk, o, 64);
                const double lv = __shfl_up(tv, o, 64);
                if (lane >= o) fwd_combine(lk, lv, tk, tv, inv_t);
            }
            float xk = __shfl_up(tk, 1, 64);
            double xv = __shfl_up(tv, 1, 64);
            if (lane == 0) { xk = -INFINITY; xv = 0.0; }
            if (lane < NW) { sk[lane] = xk; sv[lane] = xv; }
        }
        __syncthreads();
        const float pk = sk[w];
        const double pv = sv[w];
        fwd_combine(pk, pv, ek, ev, inv_t);
        __syncthreads();
    }
    k = ek; v = ev;
}

template <int NT>
LS_DEV void block_scan_bwd_excl(float& k, double& v, float* sk, double* sv, double inv_t) {
    constexpr int NW = NT / 64;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    float ik = k; double iv = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float rk = __shfl_down(ik, o, 64);
        const double rv = __shfl_down(iv, o, 64);
        if (lane + o < 64) bwd_combine(ik, iv, rk, rv, inv_t);
    }
    float ek = __shfl_down(ik, 1, 64);
    double ev = __shfl_down(iv, 1, 64);
    if (lane == 63) { ek = INFINITY; ev = 0.0; }
    if (NW > 1) {
        if (lane == 0) { sk[w] = ik; sv[w] = iv; }
        __syncthreads();
        if (w == 0) {
            float tk = lane < NW ? sk[lane] : INFINITY;
            double tv = lane < NW ? sv[lane] : 0.0;
#pragma unroll
            for (int o = 1; o < NW; o <<= 1) {
                const float rk = __shfl_down(tk, o, 64);
                const double rv = __shfl_down(tv, o, 64);
                if (lane + o < NW) bwd_combine(tk, tv, rk, rv, inv_t);
            }
            float xk = __shfl_down(tk, 1, 64);
            double xv = __shfl_down(tv, 1, 64);
            if (lane + 1 >= NW) { xk = INFINITY; xv = 0.0; }
            if (lane < NW) { sk[lane] = xk; sv[lane] = xv; }
        }
        __syncthreads();
        bwd_combine(ek, ev, sk[w], sv[w], inv_t);
        __syncthreads();
    }
    k = ek; v = ev;
}

// largest x >= -1 over the workgroup (all threads call it; s: >= NT/64
// words).  A wave maximum by lane exchanges, then one word per wave: no
// same-address LDS atomics, which serialize when many threads hold a value.
template <int NT>
LS_DEV int block_max_int(int x, int* s) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6;
    const int m = (int)wave_max_u32((uint32_t)(x + 1)) - 1;
    if (lane_id() == 0) s[w] = m;
    __syncthreads();
    int r = s[0];
#pragma unroll
    for (int q = 1; q < NW; ++q) r = max(r, s[q]);
    __syncthreads();
    return r;
}

// segment aggregates of sorted scores v_0..v_{c-1} held as keys in `keys`
// (LDS or global): P = sum e^{(v_i - v_last)/t}, Bx = sum_{i>0} e^{(v_0 - v_i)/t}.
// Argument in fp64 (exact difference), exponential in fp32, sums in fp64.
template <int NT>
__device__ void segment_aggregates(const uint32_t* keys, int c, double inv_t, float* first, float* last,
                                   double* P, double* Bx, double* scratch) {
    const float f = key2f(keys[0]);
    const float l = key2f(keys[c - 1]);
    double p = 0.0, bx = 0.0;
    for (int i = threadIdx.x; i < c; i += NT) {
        const double v = (double)key2f(keys[i]);
        p += (double)exp_neg((float)((v - (double)l) * inv_t));
        if (i > 0) bx += (double)exp_neg((float)(((double)f - v) * inv_t));
    }
    const double ps = block_sum<NT>(p, scratch);
    const double bs = block_sum<NT>(bx, scratch);
    if (threadIdx.x == 0) { *first = f; *last = l; *P = ps; *Bx = bs; }
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
    // when set, segments hold raw (unsorted) fp32 bit patterns and the root
    // segment is sorted into this LDS buffer (capacity kBucketCapMax)
    uint32_t* sortbuf;
};

struct Tails {
    float aL, aR;          // bracket ends (+-inf when open)
    double S_L, S_R;       // tail sums
    double m;              // scores in the segments
    double c_R;            // scores >= a_R
    double k, t, inv_t;
    // a range [fL, fH] holding every score and tail key (+-inf: unknown);
    // when it spans at most 600 t, all carries share one additive frame
    // with key fL (fL = aL whenever the lower tail is not empty)
    float fL, fH;
};

struct SolveScratch {      // global scratch
    float* pk; double* pv;     // per segment: forward carry before it
    float* bk; double* bv;     // per segment: backward carry after it
    double* bfx;               // per segment: exclusive suffix at its first score
    uint32_t* rank;            // per segment: sorted index of its first score
    double* eP; double* eB;    // per score of the root segment: P_j, B_j
};

// big: the root segment holds more scores than the LDS sort buffer; jstar is
// then the segment's index and b is not formed
struct SolveOut { double b; long long jstar; int ok; int big; };

// log-space closed-form root of  A/(2w) + D - B w/2 = 0  (w > 0)
LS_DEV double log_root(double lnA, double lnB, double D) {
    const double AB = (lnA == -INFINITY || lnB == -INFINITY) ? 0.0 : exp(lnA + lnB);
    const double s = sqrt(D * D + AB);
    if (D > 0.0) return log(D + s) - lnB;
    if (D < 0.0) return lnA - log(s - D);
    return 0.5 * (lnA - lnB);
}

// wave-level exclusive scans of curve carries (wave 0 of the workgroup)
LS_DEV void wave_scan_fwd_excl(float& k, double& v, double inv_t) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float lk = __shfl_up(k, o, 64);
        const double lv = __shfl_up(v, o, 64);
        if (lane >= o) fwd_combine(lk, lv, k, v, inv_t);
    }
    float ek = __shfl_up(k, 1, 64);
    double ev = __shfl_up(v, 1, 64);
    if (lane == 0) { ek = -INFINITY; ev = 0.0; }
    k = ek; v = ev;
}
LS_DEV void wave_scan_bwd_excl(float& k, double& v, double inv_t) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float rk = __shfl_down(k, o, 64);
        const double rv = __shfl_down(v, o, 64);
        if (lane + o < 64) bwd_combine(k, v, rk, rv, inv_t);
    }
    float ek = __shfl_down(k, 1, 64);
    double ev = __shfl_down(v, 1, 64);
    if (lane == 63) { ek = INFINITY; ev = 0.0; }
    k = ek; v = ev;
}

// Carries of one segment per thread.  A carry (K, V) stands for a sum over
// a set of scores v: forward, V = sum e^{(v - K)/t}; backward,
// V = sum e^{(K - v)/t}.  A wave works in an additive frame when its
// segments span at most 600 t: with ref its smallest score, every
// u = e^{(v - ref)/t} lies in [1, e^600], so its carries are plain prefix
// and suffix sums of U = sum u and W = sum 1/u (key ref, no exponential on
// the scan chain), and the carries from the other waves and the tails are
// put in the same frame.  When the whole band [a_L, a_R) spans at most
// 600 t (global frame), every wave uses ref = a_L and the waves' totals add
// up without exponentials too.  A wider wave scans (K, V) pairs with the
// exponential combine.  Keys rise with the segment index, so every combine
// and every later evaluation at a score of the segment has an exponent
// <= 0; the one exception, a backward carry in an additive frame, has a
// factor e^{(x - ref)/t} <= e^600 on a sum of terms e^{(ref - v)/t} with
// v >= x, so the product stays below the count: no overflow.
struct SegCarries {
    uint32_t rank;               // scores in earlier segments
    int frame;                   // 1: all four carries below have key ref
    double E;                    // frame: e^{(first - ref)/t} of this segment
    float kf_in, kb_in;          // earlier / later segments of this wave
    double vf_in, vb_in;
    float kf_w, kb_w;            // lower tail and earlier waves / upper tail and later waves
    double vf_w, vb_w;
    float kf_o, kb_o;            // the same before the move into the frame (keys: nearest scores)
    double vf_o, vb_o;
    float last_before, first_after;  // nearest segment scores outside the segment (+-inf: none)
};
// scratch: sk >= 8 NT/64 floats, sv >= 6 NT/64 doubles, su >= 3 NT/64 words;
// not written again before the caller's next barrier
template <int NT>
LS_DEV SegCarries block_seg_carries(uint32_t c, float f, float l, double P, double Bx, const Tails& tl, bool global,
                                    float* sk, double* sv, uint32_t* su) {
    constexpr int NW = NT / 64;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const double inv_t = tl.inv_t;
    const float fk = c ? f : INFINITY;
    const float lk = c ? l : -INFINITY;
    // the wave's score range decides its frame (wave-uniform)
    const float wmin = __uint_as_float(wave_min_f32_bits(fk)), wmax = __uint_as_float(wave_max_f32_bits(lk));
    const bool empty = !(wmax > -INFINITY);
    const bool wadd = global || empty || ((double)wmax - (double)wmin) * inv_t <= 600.0;
    const float ref = global ? tl.fL : (empty ? -INFINITY : wmin);
    SegCarries r;
    r.frame = wadd ? 1 : 0;
    r.E = 1.0;
    // in-wave scans: counts, largest last score before, smallest first score
    // after, and the carries (plain sums in a frame, (K, V) pairs otherwise)
    uint32_t ir = c;
    float il = lk, iF = fk;
    float ak = lk, bk = fk;
    double av = 0.0, bv = 0.0;
    if (wadd) {
        if (c) {
            const double rd = (double)ref;
            r.E = exp(((double)f - rd) * inv_t);
            av = P * exp(((double)l - rd) * inv_t);
            bv = (1.0 + Bx) / r.E;
        }
    } else if (c) {
        av = P;
        bv = 1.0 + Bx;
    }
    if (wadd) {
        // plain sums, maxima and minima: butterfly scans over lane exchanges
        // (wadd is wave-uniform, so every lane is here)
        ir = wave_inclusive_scan(ir);
        il = wave_scan_max_f32(il);
        iF = wave_rscan_min_f32(iF);
        av = wave_scan_add_incl(av, false);
        bv = wave_scan_add_incl(bv, true);
    } else {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t a2 = __shfl_up(ir, o, 64);
            const float il2 = __shfl_up(il, o, 64);
            const float iF2 = __shfl_down(iF, o, 64);
            const double lv2 = __shfl_up(av, o, 64);
            const double rv2 = __shfl_down(bv, o, 64);
            const float lk2 = __shfl_up(ak, o, 64);
            const float rk2 = __shfl_down(bk, o, 64);
            if (lane >= o) {
                ir += a2;
                il = fmaxf(il, il2);
                fwd_combine(lk2, lv2, ak, av, inv_t);
            }
            if (lane + o < 64) {
                iF = fminf(iF, iF2);
                bwd_combine(bk, bv, rk2, rv2, inv_t);
            }
        }
    }
    r.rank = __shfl_up(ir, 1, 64);
    if (lane == 0) r.rank = 0u;
    float el = __shfl_up(il, 1, 64);
    if (lane == 0) el = -INFINITY;
    float eF = __shfl_down(iF, 1, 64);
    if (lane == 63) eF = INFINITY;
    r.vf_in = __shfl_up(av, 1, 64);
    if (lane == 0) r.vf_in = 0.0;
    r.vb_in = __shfl_down(bv, 1, 64);
    if (lane == 63) r.vb_in = 0.0;
    float tfk, tbk;
    if (wadd) {
        r.kf_in = ref;
        r.kb_in = ref;
        tfk = ref;
        tbk = empty && !global ? INFINITY : ref;
    } else {
        r.kf_in = __shfl_up(ak, 1, 64);
        if (lane == 0) r.kf_in = -INFINITY;
        r.kb_in = __shfl_down(bk, 1, 64);
        if (lane == 63) r.kb_in = INFINITY;
        tfk = __shfl(ak, 63, 64);
        tbk = __shfl(bk, 0, 64);
    }
    const double tfv = __shfl(av, 63, 64), tbv = __shfl(bv, 0, 64);
    if (lane == 0) {
        sk[w] = tfk; sv[w] = tfv;
        sk[NW + w] = tbk; sv[NW + w] = tbv;
        sk[2 * NW + w] = wmax; sk[3 * NW + w] = wmin;
        sk[4 * NW + w] = ref;
        su[2 * NW + w] = (wadd && !empty) ? 1u : 0u;  // the wave's carries go in its frame
    }
    if (lane == 63) su[w] = ir;
    __syncthreads();
    if (global) {
        // one frame for the whole band: each thread adds the other waves'
        // totals itself, in wave order (no exponential, no second stage)
        uint32_t pcn = 0u;
        double pv = tl.S_L > 0.0 ? tl.S_L * exp(((double)tl.aL - (double)tl.fL) * inv_t) : 0.0, qv = 0.0;
        float pmx = -INFINITY, qmn = INFINITY;
        for (int x = 0; x < w; ++x) { pcn += su[x]; pv += sv[x]; pmx = fmaxf(pmx, sk[2 * NW + x]); }
        for (int x = NW - 1; x > w; --x) { qv += sv[NW + x]; qmn = fminf(qmn, sk[3 * NW + x]); }
        if (tl.S_R > 0.0) qv += tl.S_R * exp(((double)tl.fL - (double)tl.aR) * inv_t);
        r.rank += pcn;
        r.kf_w = r.kb_w = r.kf_o = r.kb_o = tl.fL;
        r.vf_w = r.vf_o = pv;
        r.vb_w = r.vb_o = qv;
        r.last_before = fmaxf(el, pmx);
        r.first_after = fminf(eF, qmn);
        __syncthreads();
        return r;
    }
    // Every wave forms its own carries from the other waves' totals at once:
    // lane y < NW stands for wave y, lane NW for the lower tail and lane
    // NW + 1 for the upper tail.  A chain of forward combines leaves the key
    // of its last non-empty member, K, and the sum over members j of
    // V_j e^{(K_j - K)/t}: keys rise with the wave index, so K is the largest
    // key and every exponent is <= 0; backward, the smallest key and
    // e^{(K - K_j)/t}.  One exponential per lane, no serial chain.
    const bool tailL = tl.S_L > 0.0 && tl.aL > -INFINITY;
    const bool tailR = tl.S_R > 0.0 && tl.aR < INFINITY;
    float xk = -INFINITY, yk = INFINITY, pm = -INFINITY, qm = INFINITY;
    double xv = 0.0, yv = 0.0;
    uint32_t pc = 0u;
    if (lane < NW && lane < w) { xk = sk[lane]; xv = sv[lane]; pm = sk[2 * NW + lane]; pc = su[lane]; }
    if (lane < NW && lane > w) { yk = sk[NW + lane]; yv = sv[NW + lane]; qm = sk[3 * NW + lane]; }
    if (lane == NW && tailL) { xk = tl.aL; xv = tl.S_L; }
    if (lane == NW + 1 && tailR) { yk = tl.aR; yv = tl.S_R; }
    const float Kf = __uint_as_float(wave_max_f32_bits(xk));
    const float Kb = __uint_as_float(wave_min_f32_bits(yk));
    const double Vf = wave_sum(xv != 0.0 ? xv * exp(((double)xk - (double)Kf) * inv_t) : 0.0);
    const double Vb = wave_sum(yv != 0.0 ? yv * exp(((double)Kb - (double)yk) * inv_t) : 0.0);
    r.kf_o = Kf; r.vf_o = Vf;
    r.kb_o = Kb; r.vb_o = Vb;
    if (wadd && !empty) {  // into the wave's own frame (key ref: every exponent <= 0)
        r.kf_w = ref; r.vf_w = Vf != 0.0 ? Vf * exp(((double)Kf - (double)ref) * inv_t) : 0.0;
        r.kb_w = ref; r.vb_w = Vb != 0.0 ? Vb * exp(((double)ref - (double)Kb) * inv_t) : 0.0;
    } else {
        r.kf_w = Kf; r.vf_w = Vf;
        r.kb_w = Kb; r.vb_w = Vb;
    }
    r.rank += (uint32_t)wave_sum_u64(pc);
    r.last_before = fmaxf(el, __uint_as_float(wave_max_f32_bits(pm)));
    r.first_after = fminf(eF, __uint_as_float(wave_min_f32_bits(qm)));
    return r;
}

// Storage slot of segment s when each of nt threads owns per consecutive
// segments (thread t: segments t*per .. t*per + per - 1): the q-th segment of
// thread t sits at q*nt + t, so that the threads' q-th loads form one
// contiguous run (with per consecutive segments per thread at consecutive
// addresses, every lane of a load touched a different cache line).  The
// identity when per == 1.  Every writer of segment aggregates for a solve
// with more segments than threads uses the same slots.
LS_DEV int seg_slot(int s, int per, int nt) { return per == 1 ? s : (s % per) * nt + s / per; }

// Runs on all NT threads of one workgroup; result valid in thread 0.
// Memory round trips are kept to a handful: each thread fetches its
// segments' aggregates with PB loads in flight (in seg_slot order, so the
// workgroup's loads coalesce), the root segment's scores are read once, and
// the root is taken by the thread that owns j* with its neighbour's values
// exchanged through LDS.
template <int NT, int EMAX>
__device__ __attribute__((always_inline)) SolveOut segment_solve(const SegView sv, const Tails tl, const SolveScratch sc,
                                  float* s_k, double* s_v, int* s_int) {
    constexpr int PB = 4;  // segments per batch of loads when a thread holds several
    const int tid = threadIdx.x;
    const double inv_t = tl.inv_t;
    const int nseg = sv.nseg;
    __shared__ double s_root[4];
    __shared__ int s_owner;
    // the root segment's count, offset, rank and carries (phases 1-3 to 4)
    __shared__ uint32_t s_seg[3];
    __shared__ float s_ck[2];
    __shared__ double s_cv[2];
    // Whole-array mode (no segment aggregates given, sv.P null): one segment
    // holding every score, no tails.  Phases 1-3 are skipped: phase 4 tests
    // G at every score itself, and when none passes the root lies below the
    // first score.
    const bool whole = sv.P == nullptr;
    // storage slot of segment s (see seg_slot): identity when nseg <= NT
    const int per_seg = (nseg + NT - 1) / NT;
    const auto slot = [&](int s) { return seg_slot(s, per_seg, NT); };
    int sstar = 0;
    if (!whole) {
        // ---- phases 1-3: carries before/after every segment, segment ranks, and
        // G at every segment's first score; each thread owns a contiguous run of
        // segments (one segment when nseg <= NT, kept in registers) ----
        const int per = (nseg + NT - 1) / NT;
        const int s0 = min(nseg, tid * per), s1 = min(nseg, s0 + per);
        float ak = -INFINITY, bk = INFINITY;
        double av = 0.0, bvv = 0.0;
        uint32_t rc = 0u;
        uint32_t c1 = 0u, o1 = 0u; float f1 = 0.0f; double Bx1 = 0.0;  // the one segment (per == 1)
        if (per == 1) {
            if (s0 < s1) {
                c1 = sv.cnt[slot(s0)];
                o1 = sv.off[slot(s0)];
                if (c1) {
                    f1 = sv.first[slot(s0)]; Bx1 = sv.Bx[slot(s0)];
                    ak = sv.last[slot(s0)]; av = sv.P[slot(s0)];
                    bk = f1; bvv = 1.0 + Bx1;
                }
                rc = c1;
            }
        } else {
            // several segments per thread: their aggregates are read PB at a
            // time, all loads of a batch in flight before the combines
            for (int sb = s0; sb < s1; sb += PB) {
                uint32_t cq[PB]; float lq[PB]; double Pq[PB];
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const int s = sb + q;
                    const bool in = s < s1;
                    cq[q] = in ? sv.cnt[slot(s)] : 0u; lq[q] = in ? sv.last[slot(s)] : 0.0f; Pq[q] = in ? sv.P[slot(s)] : 0.0;
                }
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    if (cq[q]) { float lk = ak; double lv = av; ak = lq[q]; av = Pq[q]; fwd_combine(lk, lv, ak, av, inv_t); }
                    rc += cq[q];
                }
            }
            for (int sb = s1 - 1; sb >= s0; sb -= PB) {
                uint32_t cq[PB]; float fq[PB]; double Bq[PB];
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const int s = sb - q;
                    const bool in = s >= s0;
                    cq[q] = in ? sv.cnt[slot(s)] : 0u; fq[q] = in ? sv.first[slot(s)] : 0.0f; Bq[q] = in ? sv.Bx[slot(s)] : 0.0;
                }
#pragma unroll
                for (int q = 0; q < PB; ++q)
                    if (cq[q]) { float k2 = fq[q]; double v2 = 1.0 + Bq[q]; bwd_combine(k2, v2, bk, bvv, inv_t); bk = k2; bvv = v2; }
            }
        }
        uint32_t rbase;
        SegCarries cr{};  // per == 1
        if (per == 1) {
            const bool global = tl.fL > -INFINITY && tl.fH < INFINITY && ((double)tl.fH - (double)tl.fL) * inv_t <= 600.0;
            __shared__ uint32_t s_su[3 * (NT / 64)];  // per-wave counts, prefixes and frame flags
            cr = block_seg_carries<NT>(c1, f1, ak, av, Bx1, tl, global, s_k, s_v, s_su);
            rbase = cr.rank;
        } else {
            rbase = block_exclusive_scan<NT>(rc, nullptr, reinterpret_cast<uint32_t*>(s_int));
            block_scan_fwd_excl<NT>(ak, av, s_k, s_v, inv_t);
            {   // the lower tail precedes everything
                float tk = -INFINITY; double tv = 0.0;
                if (tl.S_L > 0.0 && tl.aL > -INFINITY) { tk = tl.aL; tv = tl.S_L; }
                fwd_combine(tk, tv, ak, av, inv_t);
            }
            block_scan_bwd_excl<NT>(bk, bvv, s_k, s_v, inv_t);
            if (tl.S_R > 0.0 && tl.aR < INFINITY) bwd_combine(bk, bvv, tl.aR, tl.S_R, inv_t);
        }
        int cand = -1;
        auto g_test = [&](int s, double Pf, double Bf, uint32_t rank) {
            sc.bfx[slot(s)] = Bf;
            const double G = 0.5 * Pf + (tl.m - 1.0 - (double)rank) + tl.c_R - 0.5 * Bf;
            if (G >= tl.k) cand = max(cand, s);
        };
        auto g_at_first = [&](int s, float f, double Bx, float pk, double pv, float nk, double nv, uint32_t rank) {
            const double Pf = 1.0 + (pv != 0.0 ? ecoef(((double)pk - (double)f) * inv_t) * pv : 0.0);
            const double Bf = Bx + (nv != 0.0 ? ecoef(((double)f - (double)nk) * inv_t) * nv : 0.0);
            g_test(s, Pf, Bf, rank);
        };
        if (per == 1) {
            if (s0 < s1 && c1) {
                // the curve at the segment's first score from the four carries
                const double x = (double)f1;
                double Pf = 1.0, Bf = Bx1;
                if (cr.frame) {  // all four carries have key ref; E = e^{(x - ref)/t}
                    Pf += (cr.vf_in + cr.vf_w) / cr.E;
                    Bf += (cr.vb_in + cr.vb_w) * cr.E;
                } else {
                    if (cr.vf_in != 0.0) Pf += cr.vf_in * exp(((double)cr.kf_in - x) * inv_t);
                    if (cr.vf_w != 0.0) Pf += cr.vf_w * exp(((double)cr.kf_w - x) * inv_t);
                    if (cr.vb_in != 0.0) Bf += cr.vb_in * exp((x - (double)cr.kb_in) * inv_t);
                    if (cr.vb_w != 0.0) Bf += cr.vb_w * exp((x - (double)cr.kb_w) * inv_t);
                }
                g_test(s0, Pf, Bf, rbase);
            }
        } else {
            for (int sb = s0; sb < s1; sb += PB) {
                uint32_t cq[PB]; float lq[PB]; double Pq[PB];
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const int s = sb + q;
                    const bool in = s < s1;
                    cq[q] = in ? sv.cnt[slot(s)] : 0u; lq[q] = in ? sv.last[slot(s)] : 0.0f; Pq[q] = in ? sv.P[slot(s)] : 0.0;
                }
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const int s = sb + q;
                    if (s < s1) { sc.pk[slot(s)] = ak; sc.pv[slot(s)] = av; sc.rank[slot(s)] = rbase; }
                    rbase += cq[q];
                    if (cq[q]) { float lk = ak; double lv = av; ak = lq[q]; av = Pq[q]; fwd_combine(lk, lv, ak, av, inv_t); }
                }
            }
            for (int sb = s1 - 1; sb >= s0; sb -= PB) {
                uint32_t cq[PB], rq[PB]; float fq[PB], pkq[PB]; double Bq[PB], pvq[PB];
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const int s = sb - q;
                    const bool in = s >= s0;
                    cq[q] = in ? sv.cnt[slot(s)] : 0u; fq[q] = in ? sv.first[slot(s)] : 0.0f; Bq[q] = in ? sv.Bx[slot(s)] : 0.0;
                    pkq[q] = in ? sc.pk[slot(s)] : 0.0f; pvq[q] = in ? sc.pv[slot(s)] : 0.0; rq[q] = in ? sc.rank[slot(s)] : 0u;
                }
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    const int s = sb - q;
                    if (s >= s0) { sc.bk[slot(s)] = bk; sc.bv[slot(s)] = bvv; }
                    if (cq[q]) {
                        g_at_first(s, fq[q], Bq[q], pkq[q], pvq[q], bk, bvv, rq[q]);
                        float k2 = fq[q]; double v2 = 1.0 + Bq[q]; bwd_combine(k2, v2, bk, bvv, inv_t); bk = k2; bvv = v2;
                    }
                }
            }
        }
        __threadfence_block();
        sstar = block_max_int<NT>(cand, s_int);
        // the root segment's count, offset, rank and carries, published through
        // LDS by the thread that holds them (per == 1) or read back by thread 0
        if (sstar >= 0) {
            if (per == 1) {
                if (tid == sstar) {
                    // the carries in (nearest score, sum) form: key = the nearest
                    // score of another segment (else the tail's end), every
                    // exponent <= 0 (the in-wave backward carry of an additive
                    // wave: at most 600 t)
                    // (the carries from other waves in their form before the move
                    // into this wave's frame: their keys are scores of those waves)
                    if (cr.last_before > -INFINITY) {
                        ak = cr.last_before;
                        av = 0.0;
                        if (cr.vf_in != 0.0) av += cr.vf_in * exp(((double)cr.kf_in - (double)ak) * inv_t);
                        if (cr.vf_o != 0.0) av += cr.vf_o * exp(((double)cr.kf_o - (double)ak) * inv_t);
                    } else if (tl.S_L > 0.0 && tl.aL > -INFINITY) { ak = tl.aL; av = tl.S_L; }
                    else { ak = -INFINITY; av = 0.0; }
                    if (cr.first_after < INFINITY) {
                        bk = cr.first_after;
                        bvv = 0.0;
                        if (cr.vb_in != 0.0) bvv += cr.vb_in * exp(((double)bk - (double)cr.kb_in) * inv_t);
                        if (cr.vb_o != 0.0) bvv += cr.vb_o * exp(((double)bk - (double)cr.kb_o) * inv_t);
                    } else if (tl.S_R > 0.0 && tl.aR < INFINITY) { bk = tl.aR; bvv = tl.S_R; }
                    else { bk = INFINITY; bvv = 0.0; }
                    sc.pk[slot(s0)] = ak; sc.pv[slot(s0)] = av; sc.bk[slot(s0)] = bk; sc.bv[slot(s0)] = bvv; sc.rank[slot(s0)] = rbase;
                    s_seg[0] = c1; s_seg[1] = o1; s_seg[2] = rbase;
                    s_ck[0] = ak; s_cv[0] = av; s_ck[1] = bk; s_cv[1] = bvv;
                }
            } else if (tid == 0) {
                s_seg[0] = sv.cnt[slot(sstar)]; s_seg[1] = sv.off[slot(sstar)]; s_seg[2] = sc.rank[slot(sstar)];
                s_ck[0] = sc.pk[slot(sstar)]; s_cv[0] = sc.pv[slot(sstar)]; s_ck[1] = sc.bk[slot(sstar)]; s_cv[1] = sc.bv[slot(sstar)];
            }
        }
    } else if (tid == 0) {  // whole array: the one segment, rank 0, no carries
        s_seg[0] = *sv.cnt; s_seg[1] = *sv.off; s_seg[2] = 0u;
        s_ck[0] = -INFINITY; s_cv[0] = 0.0; s_ck[1] = INFINITY; s_cv[1] = 0.0;
    }
    __threadfence_block();
    __syncthreads();

    SolveOut out; out.b = 0.0; out.jstar = -1; out.ok = 1; out.big = 0;
    if (tid == 0) s_owner = -1;
    if (sstar >= 0) {
        // ---- phase 4: per-score curve inside the root segment ----
        const uint32_t cS = s_seg[0], offS = s_seg[1], rankS = s_seg[2];
        if (sv.sortbuf && cS > (uint32_t)kBucketCapMax) {
            out.big = 1;
            out.jstar = sstar;
        } else {
        const uint32_t* rk = sv.keys + offS;
        if (sv.sortbuf) {
            // unsorted segment: sort it in LDS first
            const int cp = max(next_pow2((int)cS), 64);
            for (int i = tid; i < cp; i += NT)
                sv.sortbuf[i] = i < (int)cS ? f2key(__uint_as_float(sv.keys[offS + i])) : 0xFFFFFFFFu;
            __syncthreads();
            sort_pow2_lds<NT>(sv.sortbuf, cp);
            rk = sv.sortbuf;
        }
        // the per-score arrays are sized by the thread's share of the segment,
        // instantiated for a few shares so a small segment costs one element
        // per thread
        auto phase4 = [&](auto em_tag) {
            constexpr int EMX = decltype(em_tag)::value;
            const int E = ((int)cS + NT - 1) / NT;
            const int e0 = min((int)cS, tid * E), e1 = min((int)cS, e0 + E);
            float vv[EMX];
    #pragma unroll
            for (int q = 0; q < EMX; ++q) {
                const int j = e0 + q;
                vv[q] = (j < e1) ? key2f(rk[j]) : 0.0f;
            }
            const float vfirst = key2f(rk[0]);
            const float vlast = key2f(rk[cS - 1]);
            const float pk0 = s_ck[0]; const double pv0 = s_cv[0];
            const float bk0 = s_ck[1]; const double bv0 = s_cv[1];
            double Pj[EMX], Bj[EMX];
            if (((double)vlast - (double)vfirst) * inv_t <= 600.0) {
                // additive form relative to ref = v_first: u_j = e^{(v_j - ref)/t} in [1, e^600]
                //   P_j = (carry_P + sum_{i<=j} u_i) / u_j,  B_j = u_j (carry_B + sum_{i>j} 1/u_i)
                const double ref = (double)vfirst;
                double u[EMX], Ul[EMX], Wl[EMX];
    #pragma unroll
                for (int q = 0; q < EMX; ++q) u[q] = (e0 + q < e1) ? ecoef(((double)vv[q] - ref) * inv_t) : 1.0;
                {
                    double ut = 0.0, wt = 0.0;
    #pragma unroll
                    for (int q = 0; q < EMX; ++q)
                        if (e0 + q < e1) { ut += u[q]; wt += 1.0 / u[q]; }
                    double U, W;
                    block_scan_add_excl2<NT>(ut, wt, U, W, s_v);
    #pragma unroll
                    for (int q = 0; q < EMX; ++q)
                        if (e0 + q < e1) { U += u[q]; Ul[q] = U; }
    #pragma unroll
                    for (int q = EMX - 1; q >= 0; --q)
                        if (e0 + q < e1) { Wl[q] = W; W += 1.0 / u[q]; }
                }
                const double pc = (pv0 != 0.0) ? pv0 * ecoef(((double)pk0 - ref) * inv_t) : 0.0;
                const double bc = (bv0 != 0.0) ? bv0 * ecoef((ref - (double)bk0) * inv_t) : 0.0;
    #pragma unroll
                for (int q = 0; q < EMX; ++q) {
                    Pj[q] = (pc + Ul[q]) / u[q];
                    Bj[q] = u[q] * (bc + Wl[q]);
                }
            } else {
                // wide segment: affine carries with every exponent <= 0
                double al[EMX];
    #pragma unroll
                for (int q = 1; q < EMX; ++q)
                    al[q] = (e0 + q < e1) ? ecoef(((double)vv[q - 1] - (double)vv[q]) * inv_t) : 0.0;
                al[0] = 0.0;
                float fk = -INFINITY; double fv = 0.0;
    #pragma unroll
                for (int q = 0; q < EMX; ++q)
                    if (e0 + q < e1) { fv = 1.0 + (q > 0 ? al[q] * fv : 0.0); fk = vv[q]; }
                block_scan_fwd_excl<NT>(fk, fv, s_k, s_v, inv_t);
                {
                    float pk = pk0; double pv = pv0;
                    float ck = fk; double cv = fv;
                    fwd_combine(pk, pv, ck, cv, inv_t);
                    fk = ck; fv = cv;
                }
    #pragma unroll
                for (int q = 0; q < EMX; ++q) {
                    if (e0 + q < e1) {
                        const double carry = (q == 0) ? (fv != 0.0 ? ecoef(((double)fk - (double)vv[0]) * inv_t) * fv : 0.0)
                                                      : al[q] * Pj[q - 1];
                        Pj[q] = 1.0 + carry;
                    }
                }
                float rk2 = INFINITY; double rv2 = 0.0;
    #pragma unroll
                for (int q = EMX - 1; q >= 0; --q) {
                    if (e0 + q < e1) {
                        rv2 = 1.0 + (rv2 != 0.0 ? ecoef(((double)vv[q] - (double)rk2) * inv_t) * rv2 : 0.0);
                        rk2 = vv[q];
                    }
                }
                block_scan_bwd_excl<NT>(rk2, rv2, s_k, s_v, inv_t);
                {
                    float bk = bk0; double bvv = bv0;
                    bwd_combine(rk2, rv2, bk, bvv, inv_t);
                }
    #pragma unroll
                for (int q = EMX - 1; q >= 0; --q) {
                    const int j = e0 + q;
                    if (j < e1) {
                        if (q + 1 < EMX && j + 1 < e1) Bj[q] = al[q + 1] * (1.0 + Bj[q + 1]);
                        else Bj[q] = (rv2 != 0.0) ? ecoef(((double)vv[q] - (double)rk2) * inv_t) * rv2 : 0.0;
                    }
                }
            }
            int myj = -1;
    #pragma unroll
            for (int q = 0; q < EMX; ++q) {
                const int j = e0 + q;
                if (j < e1) {
                    const double G = 0.5 * Pj[q] + (tl.m - 1.0 - (double)(rankS + (uint32_t)j)) + tl.c_R - 0.5 * Bj[q];
                    if (G >= tl.k) myj = j;
                }
            }
            // neighbour exchange: every thread publishes its first score and its B there
            s_k[tid] = vv[0];
            s_v[tid] = e0 < e1 ? Bj[0] : 0.0;
            int jl = block_max_int<NT>(myj, s_int);  // (has barriers; also orders the LDS writes above)
            if (jl < 0 && !whole) jl = 0;             // the segment's first score passed in phase 3
            if (jl >= e0 && jl < e1) {
                // this thread owns j*: lower end, P there, and the next score with its B
                const int q = jl - e0;
                double Pjs = 0.0, vlo = 0.0, vnx = 0.0, Bnx = 0.0;
                int has_next = 0;
    #pragma unroll
                for (int qq = 0; qq < EMX; ++qq) if (qq == q) { Pjs = Pj[qq]; vlo = (double)vv[qq]; }
                if (jl + 1 < e1) {
    #pragma unroll
                    for (int qq = 0; qq < EMX - 1; ++qq) if (qq == q) { vnx = (double)vv[qq + 1]; Bnx = Bj[qq + 1]; }
                    has_next = 1;
                } else if ((uint32_t)jl + 1u < cS) {
                    vnx = (double)s_k[tid + 1]; Bnx = s_v[tid + 1]; has_next = 1;
                }
                s_root[0] = Pjs; s_root[1] = vlo; s_root[2] = vnx; s_root[3] = Bnx;
                s_owner = has_next;
            }
            __syncthreads();
            if (tid == 0 && jl < 0) {
                // whole array, G(v_first) < k: b lies below every score, where
                // G(b) = n - w (1 + B_first)/2 with w = e^{(b - v_first)/t}, so
                // w = 2 (n - k)/(1 + B_first): the quadratic with A = 0.
                // Thread 0 holds B_first (its first element is score 0).
                const double ref = (double)vfirst;
                const double D = tl.m + tl.c_R - tl.k;
                const double lnw = log_root(-INFINITY, log1p(Bj[0]), D);
                double b = ref + tl.t * lnw;
                if (b > ref) b = ref;
                out.jstar = -1;
                out.b = b;
                out.ok = (b == b) && (b > -INFINITY) && (b < INFINITY);
            } else if (tid == 0) {
                const double lo = s_root[1];
                double lnA = log(s_root[0]), lnB, chi;
                const double J = (double)(rankS + (uint32_t)jl);
                const double D = (tl.m - 1.0 - J) + tl.c_R - tl.k;
                out.jstar = (long long)(rankS + (uint32_t)jl);
                const int has_next = s_owner;
                if (has_next) {
                    const double vnext = s_root[2], Bnext = s_root[3];
                    chi = vnext; lnB = (lo - vnext) * inv_t + log1p(Bnext);
                } else if (bv0 != 0.0) {
                    // the backward carry after the root segment: its position is the
                    // next score (first of a later segment, or a_R) and its value the
                    // sum of e^{(position - v)/t} over every score from there up
                    chi = (double)bk0; lnB = (lo - (double)bk0) * inv_t + log(bv0);
                } else {
                    chi = tl.aR; lnB = -INFINITY;
                }
                const double lnw = log_root(lnA, lnB, D);
                double b = lo + tl.t * lnw;
                if (b < lo) b = lo;
                if (b > chi) b = chi;
                out.b = b;
                out.ok = (b == b) && (b > -INFINITY) && (b < INFINITY);
            }
        };
        // A root segment of at most 64 scores: wave 0 alone, one score per
        // lane, with the same arithmetic as phase4 at one score per thread
        // (the cross-wave parts of its scans only add identities there) but
        // no barrier; the other waves go on to the caller.
        auto phase4_wave = [&]() {
            if (tid >= 64) return;
            const int l = tid;
            const bool in = l < (int)cS;
            const float vv = in ? key2f(rk[l]) : 0.0f;
            const float vfirst = key2f(rk[0]);
            const float vlast = key2f(rk[cS - 1]);
            const float pk0 = s_ck[0]; const double pv0 = s_cv[0];
            const float bk0 = s_ck[1]; const double bv0 = s_cv[1];
            double Pj = 0.0, Bj = 0.0;
            if (((double)vlast - (double)vfirst) * inv_t <= 600.0) {
                const double ref = (double)vfirst;
                const double u = in ? ecoef(((double)vv - ref) * inv_t) : 1.0;
                const double U = wave_excl_from_incl(wave_scan_add_incl(in ? u : 0.0, false), false);
                const double W = wave_excl_from_incl(wave_scan_add_incl(in ? 1.0 / u : 0.0, true), true);
                const double pc = (pv0 != 0.0) ? pv0 * ecoef(((double)pk0 - ref) * inv_t) : 0.0;
                const double bc = (bv0 != 0.0) ? bv0 * ecoef((ref - (double)bk0) * inv_t) : 0.0;
                Pj = (pc + (U + u)) / u;
                Bj = u * (bc + W);
            } else {
                float fk = in ? vv : -INFINITY;
                double fv = in ? 1.0 : 0.0;
                wave_scan_fwd_excl(fk, fv, inv_t);
                {
                    float pk = pk0; double pv = pv0;
                    fwd_combine(pk, pv, fk, fv, inv_t);
                }
                if (in) Pj = 1.0 + (fv != 0.0 ? ecoef(((double)fk - (double)vv) * inv_t) * fv : 0.0);
                float rk2 = in ? vv : INFINITY;
                double rv2 = in ? 1.0 : 0.0;
                wave_scan_bwd_excl(rk2, rv2, inv_t);
                {
                    float bk = bk0; double bvv = bv0;
                    bwd_combine(rk2, rv2, bk, bvv, inv_t);
                }
                if (in) Bj = (rv2 != 0.0) ? ecoef(((double)vv - (double)rk2) * inv_t) * rv2 : 0.0;
            }
            int myj = -1;
            if (in) {
                const double G = 0.5 * Pj + (tl.m - 1.0 - (double)(rankS + (uint32_t)l)) + tl.c_R - 0.5 * Bj;
                if (G >= tl.k) myj = l;
            }
            int jl = (int)wave_max_u32((uint32_t)(myj + 1)) - 1;
            if (jl < 0 && !whole) jl = 0;  // the segment's first score passed in phase 3
            const int js = jl < 0 ? 0 : jl, jn = min(js + 1, 63);
            const double Pjs = __shfl(Pj, js, 64), vlo = (double)__shfl(vv, js, 64);
            const double vnx = (double)__shfl(vv, jn, 64), Bnx = __shfl(Bj, jn, 64);
            if (tid == 0 && jl < 0) {
                // whole array, G(v_first) < k: b lies below every score (as in phase4)
                const double ref = (double)vfirst;
                const double D = tl.m + tl.c_R - tl.k;
                const double lnw = log_root(-INFINITY, log1p(Bj), D);
                double b = ref + tl.t * lnw;
                if (b > ref) b = ref;
                out.jstar = -1;
                out.b = b;
                out.ok = (b == b) && (b > -INFINITY) && (b < INFINITY);
            } else if (tid == 0) {
                const double lo = vlo;
                double lnA = log(Pjs), lnB, chi;
                const double J = (double)(rankS + (uint32_t)jl);
                const double D = (tl.m - 1.0 - J) + tl.c_R - tl.k;
                out.jstar = (long long)(rankS + (uint32_t)jl);
                if ((uint32_t)jl + 1u < cS) {
                    chi = vnx; lnB = (lo - vnx) * inv_t + log1p(Bnx);
                } else if (bv0 != 0.0) {
                    chi = (double)bk0; lnB = (lo - (double)bk0) * inv_t + log(bv0);
                } else {
                    chi = tl.aR; lnB = -INFINITY;
                }
                const double lnw = log_root(lnA, lnB, D);
                double b = lo + tl.t * lnw;
                if (b < lo) b = lo;
                if (b > chi) b = chi;
                out.b = b;
                out.ok = (b == b) && (b > -INFINITY) && (b < INFINITY);
            }
        };
        if ((int)cS <= 64) phase4_wave();
        else if ((int)cS <= NT) phase4(std::integral_constant<int, 1>{});
        else if constexpr (EMAX > 4) {
            if ((int)cS <= 4 * NT) phase4(std::integral_constant<int, 4>{});
            else phase4(std::integral_constant<int, EMAX>{});
        } else phase4(std::integral_constant<int, EMAX>{});
        }  // not a big root segment
    } else if (tid == 0) {
        // the root lies below the first score of the segments
        double ref, lnA, lnB, clo, chi;
        int s0n = -1;
        for (int s = 0; s < nseg; ++s) if (sv.cnt[slot(s)]) { s0n = s; break; }
        const double D = tl.m + tl.c_R - tl.k;
        if (tl.aL > -INFINITY) {
            ref = tl.aL; clo = tl.aL;
            lnA = tl.S_L > 0.0 ? log(tl.S_L) : -INFINITY;
            if (s0n >= 0) { chi = sv.first[slot(s0n)]; lnB = ((double)tl.aL - chi) * inv_t + log1p(sc.bfx[slot(s0n)]); }
            else {
                chi = tl.aR;
                lnB = (tl.S_R > 0.0 && tl.aR < INFINITY) ? log(tl.S_R) + ((double)tl.aL - (double)tl.aR) * inv_t : -INFINITY;
            }
        } else {
            clo = -INFINITY; lnA = -INFINITY;
            if (s0n >= 0) { ref = sv.first[slot(s0n)]; chi = ref; lnB = log1p(sc.bfx[slot(s0n)]); }
            else { ref = tl.aR; chi = tl.aR; lnB = tl.S_R > 0.0 ? log(tl.S_R) : -INFINITY; }
        }
        out.jstar = -1;
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
