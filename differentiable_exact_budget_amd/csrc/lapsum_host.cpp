// Host orchestration and C ABI of the Fast LapSum solver (MI355X / gfx950).
//
// Paths (Fast LapSum paper, gist.science summary section 2.2):
//  * full sort: sort, one stable prefix/suffix scan (the threshold curve),
//    interval search, closed-form root.  One workgroup when n <= 16384,
//    otherwise an LSD radix sort and per-tile curve aggregates.
//  * bracketing (n > 10^6 by default): kernel-noised sample, binomial
//    order statistics a_L = x_(l), a_R = x_(h), one streaming pass that
//    folds out-of-band scores into fp64 tail sums and buckets the band,
//    certification, band sort + solve.  A bracket that fails is widened
//    and tried again (section 2.2, step 4), and the full sort covers the
//    worst case the bracket cannot (the arxivdaily abstract names this
//    fallback).
//
// Certification.  The streaming pass returns S_L, S_R, the band sums
// B_L = sum_band e^{(a_L - v)/t}, B_R = sum_band e^{(v - a_R)/t} and the
// counts.  G at the bracket ends follows exactly from them:
//   G(a_L) = S_L/2 + m - B_L/2 + c_R - e^{(a_L - a_R)/t} S_R/2
//   G(a_R) = e^{(a_L - a_R)/t} S_L/2 + B_R/2 + c_R - S_R/2
// and the bracket holds iff G(a_L) >= k > G(a_R) (G is decreasing).  The
// host reads these totals once per attempt (a pinned-memory hand-off from
// the pass's last workgroup), so a failed bracket never costs a band sort.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "lapsum.h"
#include "lapsum_testing.h"
#include "lapsum_launch.h"

using namespace lapsum;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Scratch memory of one (device, stream).  A call holds `mu` from the moment
// it finds its workspace until it returns, so calls on one stream from
// several host threads take turns (their device work is ordered on the
// stream in the order they took the workspace), and a release waits for the
// call in flight.  Workspace objects are never deleted: a release frees
// their memory and the next call allocates it again.
struct Workspace {
    std::mutex mu;
    bool inject_internal = false;  // lapsum_test_inject_internal: mark the next solve failed
    int device = 0;
    hipStream_t stream = nullptr;
    long long n_cap = 0;
    char* base = nullptr;
    size_t bytes = 0;
    Ctl* ctl = nullptr;
    HostSummary* hs = nullptr;      // pinned host
    HostSummary* hs_dev = nullptr;  // device view of hs
    unsigned int seq = 0;
    double* part = nullptr;
    int probs_parts = 1;  // partials the last p pass left
    float* sample = nullptr;
    long long* sample_idx = nullptr;
    uint32_t* shist = nullptr;  // two sample histograms (kSelHistBins words each), used in turn
    uint32_t* swin = nullptr;   // the select's gathered window (kWinHdr + kWinMax words)
    unsigned int shist_turn = 0;
    float* sp = nullptr;
    float* iw = nullptr;
    uint32_t* bucket_cnt = nullptr;
    uint32_t* bucket_vals = nullptr;
    uint32_t* hoff = nullptr;   // per bucket: slot offset of an overflowed bucket's scores, or kNotHeavy
    uint32_t* hfill = nullptr;  // per bucket: scores placed in that slot
    HeavyArrays heavy{};        // the slots of overflowed buckets (laid out on the device)
    SegArrays seg{};
    SolveScratch sc{};
    uint32_t* keysA = nullptr;
    uint32_t* keysB = nullptr;
    uint32_t* hist_part = nullptr;
    uint32_t* goff = nullptr;
    unsigned long long* status = nullptr;
    size_t status_bytes = 0;
    uint32_t epoch = 1;
    bool status_dirty = false;  // the status region holds split-pass data
    std::vector<hipEvent_t> events;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace*> g_ws;

long long tiles_for(long long n) { return (n + kRadixTile - 1) / kRadixTile; }

// layout of one workspace for forwards up to n_cap scores
struct Layout {
    size_t ctl, part, sample, sample_idx, shist, swin, sp, iw, bcnt, bvals, hoff, hfill, hmin, hmax, hch0, hpart,
        seg_first, seg_last, seg_P, seg_Bx, seg_cnt, seg_off,
        sc_pk, sc_pv, sc_bk, sc_bv, sc_bfx, sc_rank, sc_eP, sc_eB, keysA, keysB, hist, goff, status, total;
    size_t status_bytes;
};

Layout make_layout(long long n_cap) {
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
    // segment slots: a whole number of kCurveRootThreads (the root reads
    // segment s of more than one per thread from seg_slot's slot)
    const long long nseg0 = std::max<long long>(std::max<long long>(kMaxBuckets, tiles_for(n_cap)), 1);
    const long long nseg = (nseg0 + kCurveRootThreads - 1) / kCurveRootThreads * kCurveRootThreads;
    const long long elem = std::max<long long>(kBucketCapMax, std::max(kRadixTile, kSmallMax));
    L.ctl = take(sizeof(Ctl));
    L.part = take(sizeof(double) * 2 * (size_t)kMaxStreamParts);
    L.sample = take(sizeof(float) * kSampleMax);
    L.sample_idx = take(sizeof(long long) * kSampleMax);
    L.shist = take(sizeof(uint32_t) * 2 * kSelHistBins);
    L.swin = take(sizeof(uint32_t) * (kWinHdr + kWinMax));
    L.sp = take(sizeof(float) * (kMaxBuckets + 1));
    L.iw = take(sizeof(float) * kMaxBuckets);
    L.bcnt = take(sizeof(uint32_t) * kMaxBuckets);
    L.bvals = take(sizeof(uint32_t) * (size_t)kMaxBuckets * kBucketCapMax);
    L.hoff = take(sizeof(uint32_t) * kMaxBuckets);
    L.hfill = take(sizeof(uint32_t) * kMaxBuckets);
    L.hmin = take(sizeof(uint32_t) * kMaxBuckets);
    L.hmax = take(sizeof(uint32_t) * kMaxBuckets);
    L.hch0 = take(sizeof(uint32_t) * kMaxBuckets);
    // overflowed buckets hold at most n_cap scores: at most n_cap / chunk + one
    // partial chunk per bucket
    L.hpart = take(sizeof(unsigned long long) * 4 *
                   (size_t)(std::max<long long>(n_cap, 1) / kHeavyChunk + kMaxBuckets + 1));
    L.seg_first = take(sizeof(float) * nseg);
    L.seg_last = take(sizeof(float) * nseg);
    L.seg_P = take(sizeof(double) * nseg);
    L.seg_Bx = take(sizeof(double) * nseg);
    L.seg_cnt = take(sizeof(uint32_t) * nseg);
    L.seg_off = take(sizeof(uint32_t) * nseg);
    L.sc_pk = take(sizeof(float) * nseg);
    L.sc_pv = take(sizeof(double) * nseg);
    L.sc_bk = take(sizeof(float) * nseg);
    L.sc_bv = take(sizeof(double) * nseg);
    L.sc_bfx = take(sizeof(double) * nseg);
    L.sc_rank = take(sizeof(uint32_t) * nseg);
    L.sc_eP = take(sizeof(double) * elem);
    L.sc_eB = take(sizeof(double) * elem);
    const long long nk = std::max<long long>(n_cap, 1);
    L.keysA = take(sizeof(uint32_t) * nk);
    L.keysB = take(sizeof(uint32_t) * nk);
    L.hist = take(sizeof(uint32_t) * kHistStride * kRadixHistBlocks);
    L.goff = take(sizeof(uint32_t) * 1024);
    L.status_bytes = sizeof(unsigned long long) * radix_status_words(n_cap);
    L.status = take(L.status_bytes);
    L.total = o;
    return L;
}

// frees a workspace's memory (the caller holds w->mu)
void free_ws_memory(Workspace* w) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(w->device);
    (void)hipStreamSynchronize(w->stream);
    for (hipEvent_t e : w->events) (void)hipEventDestroy(e);
    w->events.clear();
    if (w->base) (void)hipFree(w->base);
    if (w->hs) (void)hipHostFree(w->hs);
    w->base = nullptr;
    w->bytes = 0;
    w->n_cap = 0;
    w->hs = nullptr;
    w->hs_dev = nullptr;
    (void)hipSetDevice(cur);
}

lapsum_status_t alloc_ws(Workspace* w, long long n_cap) {
    Layout L = make_layout(n_cap);
    char* base = nullptr;
    if (hipMalloc(&base, L.total) != hipSuccess) return LAPSUM_ERR_OUT_OF_MEMORY;
    w->base = base;
    w->bytes = L.total;
    w->n_cap = n_cap;
    w->ctl = reinterpret_cast<Ctl*>(base + L.ctl);
    w->part = reinterpret_cast<double*>(base + L.part);
    w->sample = reinterpret_cast<float*>(base + L.sample);
    w->sample_idx = reinterpret_cast<long long*>(base + L.sample_idx);
    w->shist = reinterpret_cast<uint32_t*>(base + L.shist);
    w->swin = reinterpret_cast<uint32_t*>(base + L.swin);
    w->shist_turn = 0;
    w->sp = reinterpret_cast<float*>(base + L.sp);
    w->iw = reinterpret_cast<float*>(base + L.iw);
    w->bucket_cnt = reinterpret_cast<uint32_t*>(base + L.bcnt);
    w->bucket_vals = reinterpret_cast<uint32_t*>(base + L.bvals);
    w->hoff = reinterpret_cast<uint32_t*>(base + L.hoff);
    w->hfill = reinterpret_cast<uint32_t*>(base + L.hfill);

    w->seg = SegArrays{reinterpret_cast<float*>(base + L.seg_first), reinterpret_cast<float*>(base + L.seg_last),
                       reinterpret_cast<double*>(base + L.seg_P), reinterpret_cast<double*>(base + L.seg_Bx),
                       reinterpret_cast<uint32_t*>(base + L.seg_cnt), reinterpret_cast<uint32_t*>(base + L.seg_off)};
    w->sc = SolveScratch{reinterpret_cast<float*>(base + L.sc_pk), reinterpret_cast<double*>(base + L.sc_pv),
                         reinterpret_cast<float*>(base + L.sc_bk), reinterpret_cast<double*>(base + L.sc_bv),
                         reinterpret_cast<double*>(base + L.sc_bfx), reinterpret_cast<uint32_t*>(base + L.sc_rank),
                         reinterpret_cast<double*>(base + L.sc_eP), reinterpret_cast<double*>(base + L.sc_eB)};
    w->keysA = reinterpret_cast<uint32_t*>(base + L.keysA);
    w->keysB = reinterpret_cast<uint32_t*>(base + L.keysB);
    w->heavy.hoff = w->hoff;
    w->heavy.hfill = w->hfill;
    w->heavy.hmin = reinterpret_cast<uint32_t*>(base + L.hmin);
    w->heavy.hmax = reinterpret_cast<uint32_t*>(base + L.hmax);
    w->heavy.hch0 = reinterpret_cast<uint32_t*>(base + L.hch0);
    w->heavy.hpart = reinterpret_cast<unsigned long long*>(base + L.hpart);
    w->heavy.base_off = (unsigned long long)(w->keysB - w->bucket_vals);
    w->heavy.cap_total = (unsigned long long)std::max<long long>(n_cap, 1);
    w->hist_part = reinterpret_cast<uint32_t*>(base + L.hist);
    w->goff = reinterpret_cast<uint32_t*>(base + L.goff);
    w->status = reinterpret_cast<unsigned long long*>(base + L.status);
    w->status_bytes = L.status_bytes;
    w->epoch = 1;
    // the control block (tickets, counters) and the look-back words start at zero
    if (hipMemsetAsync(w->ctl, 0, sizeof(Ctl), w->stream) != hipSuccess) return LAPSUM_ERR_HIP;
    if (hipMemsetAsync(w->status, 0, w->status_bytes, w->stream) != hipSuccess) return LAPSUM_ERR_HIP;
    // both sample histograms and the window header start at zero
    if (hipMemsetAsync(w->shist, 0, sizeof(uint32_t) * 2 * kSelHistBins, w->stream) != hipSuccess)
        return LAPSUM_ERR_HIP;
    if (hipMemsetAsync(w->swin, 0, sizeof(uint32_t) * kWinHdr, w->stream) != hipSuccess) return LAPSUM_ERR_HIP;
    // the radix sort's global digit totals start (and are left) at zero
    if (hipMemsetAsync(w->hist_part, 0, sizeof(uint32_t) * kHistRegionWords, w->stream) != hipSuccess)
        return LAPSUM_ERR_HIP;
    return LAPSUM_OK;
}

// The workspace of (current device, stream), locked for the rest of the
// caller's call and grown to forwards of n scores if it is smaller.
struct WsGuard {
    Workspace* w = nullptr;
    std::unique_lock<std::mutex> lk;
};

lapsum_status_t get_ws(hipStream_t stream, long long n, WsGuard* g) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LAPSUM_ERR_HIP;
    Workspace* w = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto key = std::make_pair(dev, stream);
        auto it = g_ws.find(key);
        if (it == g_ws.end()) {
            w = new Workspace();
            w->device = dev;
            w->stream = stream;
            g_ws[key] = w;
        } else {
            w = it->second;
        }
    }
    std::unique_lock<std::mutex> lk(w->mu);
    if (!w->hs) {
        void* hp = nullptr;
        if (hipHostMalloc(&hp, sizeof(HostSummary), hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess)
            return LAPSUM_ERR_OUT_OF_MEMORY;
        std::memset(hp, 0, sizeof(HostSummary));
        w->hs = reinterpret_cast<HostSummary*>(hp);
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, hp, 0) != hipSuccess) dp = hp;
        w->hs_dev = reinterpret_cast<HostSummary*>(dp);
        w->seq = 0;
    }
    if (!w->base || w->n_cap < n) {
        if (w->base) {
            // grow: wait for this stream's work, then replace the device buffer
            (void)hipStreamSynchronize(stream);
            (void)hipFree(w->base);
            w->base = nullptr;
            w->n_cap = 0;
        }
        lapsum_status_t st = alloc_ws(w, std::max<long long>(n, 1 << 16));
        if (st != LAPSUM_OK) {
            if (w->base) (void)hipFree(w->base);
            w->base = nullptr;
            w->n_cap = 0;
            return st;
        }
    }
    g->w = w;
    g->lk = std::move(lk);
    return LAPSUM_OK;
}

// ---------------------------------------------------------------------------
// per-launch timing (options.profile)
// ---------------------------------------------------------------------------
struct Timer {
    Workspace* w;
    hipStream_t st;
    bool on;
    int used = 0;
    std::vector<const char*> names;
    hipEvent_t ev(int i) {
        while ((int)w->events.size() <= i) {
            hipEvent_t e;
            (void)hipEventCreate(&e);
            w->events.push_back(e);
        }
        return w->events[i];
    }
    void begin(const char* name) {
        if (!on || (int)names.size() >= LAPSUM_MAX_TIMED_KERNELS) return;
        (void)hipEventRecord(ev(2 * (int)names.size()), st);
        names.push_back(name);
    }
    void end() {
        if (!on || names.empty() || used >= (int)names.size()) return;
        (void)hipEventRecord(ev(2 * used + 1), st);
        ++used;
    }
    void collect(lapsum_stats_t* s) {
        if (!s) return;
        s->n_timed = 0;
        if (!on) return;
        for (int i = 0; i < used; ++i) {
            float ms = 0.0f;
            (void)hipEventElapsedTime(&ms, w->events[2 * i], w->events[2 * i + 1]);
            s->kernel_ms[i] = ms;
            s->kernel_name[i] = names[i];
        }
        s->n_timed = used;
    }
};

// ---------------------------------------------------------------------------
// binomial order-statistic ranks: Y ~ Bin(s, q) scores below b among s samples.
//   l = largest l with P(Y <= l - 1) <= delta   (0: a_L = -inf)
//   h = smallest h with P(Y >= h) <= delta      (s + 1: a_R = +inf)
// The pmf is evaluated from its mode outwards by the ratio recurrence, far
// enough that the neglected mass is below 1e-300.
// ---------------------------------------------------------------------------
void binomial_ranks(long long s, double q, double delta, long long* l_out, long long* h_out) {
    static std::mutex mu;
    static std::map<std::tuple<long long, double, double>, std::pair<long long, long long>> cache;
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(std::make_tuple(s, q, delta));
        if (it != cache.end()) { *l_out = it->second.first; *h_out = it->second.second; return; }
    }
    long long mode = (long long)std::floor((double)(s + 1) * q);
    if (mode > s) mode = s;
    if (mode < 0) mode = 0;
    const double lq = std::log(q), l1q = std::log1p(-q);
    const double lmode = std::lgamma((double)s + 1.0) - std::lgamma((double)mode + 1.0) -
                         std::lgamma((double)(s - mode) + 1.0) + (double)mode * lq + (double)(s - mode) * l1q;
    std::vector<double> lp(s + 1, -INFINITY);
    lp[mode] = lmode;
    const double odds = lq - l1q;  // ln(q / (1 - q))
    long long lo = mode, hi = mode;
    for (long long i = mode; i > 0; --i) {  // pmf(i-1) = pmf(i) * i / (s - i + 1) / odds
        lp[i - 1] = lp[i] + std::log((double)i) - std::log((double)(s - i + 1)) - odds;
        lo = i - 1;
        if (lp[i - 1] < -700.0) break;
    }
    for (long long i = mode; i < s; ++i) {  // pmf(i+1) = pmf(i) * (s - i) / (i + 1) * odds
        lp[i + 1] = lp[i] + std::log((double)(s - i)) - std::log((double)(i + 1)) + odds;
        hi = i + 1;
        if (lp[i + 1] < -700.0) break;
    }
    long long l = 0;
    double cdf = 0.0;
    for (long long y = 0; y <= s; ++y) {
        if (y >= lo && y <= hi) cdf += std::exp(lp[y]);
        if (cdf <= delta) l = y + 1; else break;
        if (y < lo) { y = lo - 1; }  // skip the negligible part in one step
    }
    long long h = s + 1;
    double tail = 0.0;
    for (long long i = s; i >= 0; --i) {
        if (i >= lo && i <= hi) tail += std::exp(lp[i]);
        if (tail <= delta) h = i; else break;
        if (i > hi) { i = hi + 1; }
    }
    *l_out = l;
    *h_out = h;
    std::lock_guard<std::mutex> lk(mu);
    // a bounded memo: a caller whose budget changes every call (a learned k)
    // would otherwise grow it without end
    if (cache.size() >= 64) cache.clear();
    cache[std::make_tuple(s, q, delta)] = std::make_pair(l, h);
}

lapsum_status_t hip_ok(hipError_t e) { return e == hipSuccess ? LAPSUM_OK : LAPSUM_ERR_HIP; }

// The sample histogram a call builds: the two buffers are used in turn, and
// the sampler clears the other one, so each call finds its own at zero
// without a clearing launch of its own (the widenings of one call reuse it).
uint32_t* next_sample_hist(Workspace* w) {
    w->shist_turn ^= 1u;
    return w->shist + (size_t)w->shist_turn * kSelHistBins;
}
uint32_t* other_sample_hist(Workspace* w, uint32_t* hist) {
    return hist == w->shist ? w->shist + kSelHistBins : w->shist;
}

lapsum_status_t wait_summary(Workspace* w, hipStream_t st, unsigned int seq) {
    volatile unsigned int* flag = &w->hs->seq;
    auto t0 = std::chrono::steady_clock::now();
    for (unsigned long it = 0;; ++it) {
        if (*flag == seq) { std::atomic_thread_fence(std::memory_order_acquire); return LAPSUM_OK; }
        // the stream is asked about its state only once the summary is late
        // (a query may put a marker into the stream, costing the device time)
        if ((it & 4095u) == 4095u && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) {
            hipError_t e = hipStreamQuery(st);
            if (e == hipSuccess) {
                if (*flag == seq) { std::atomic_thread_fence(std::memory_order_acquire); return LAPSUM_OK; }
                return LAPSUM_ERR_INTERNAL;
            }
            if (e != hipErrorNotReady) return LAPSUM_ERR_HIP;
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(120)) return LAPSUM_ERR_INTERNAL;
        }
    }
}

// `count` fresh epochs for the words a sort publishes (one per pass); the
// region is cleared when the epochs would run out or when split passes left
// raw counts in it
uint32_t next_epoch(Workspace* w, hipStream_t st, uint32_t count) {
    if (w->epoch + count + 8u >= (1u << 30) || w->status_dirty) {
        (void)hipMemsetAsync(w->status, 0, w->status_bytes, st);
        w->epoch = 1;
        w->status_dirty = false;
    }
    uint32_t e = w->epoch;
    w->epoch += count;
    return e;
}

// Radix sort of n fp32 scores (keys end in keysB).  The one-kernel passes
// read epoch-tagged status words; the split passes leave counts and offsets
// in the same region, which must not pass for status words: the region is
// cleared before the next sort that reads it.
// form: as launch_radix_sort (0 picks by size).
void sort_keys(Workspace* w, const float* r, long long n, hipStream_t st, int form = 0) {
    const uint32_t epoch = next_epoch(w, st, 4u);
    launch_radix_sort(r, n, w->keysA, w->keysB, w->hist_part, w->goff, w->status, epoch, w->ctl, st, form);
    if (form == 2 || !radix_uses_onesweep(n)) w->status_dirty = true;
}

void run_full(Workspace* w, const float* r, long long n, double k, double t, double* b_out, hipStream_t st, Timer& tm) {
    if (n <= kSmallMax) {
        tm.begin("small_solve");
        launch_small_solve(r, (int)n, k, t, w->ctl, w->sc, b_out, nullptr, st);
        tm.end();
        return;
    }
    tm.begin("radix_sort");
    sort_keys(w, r, n, st);
    tm.end();
    tm.begin("curve_solve");
    launch_curve_tiles(w->keysB, n, w->ctl, w->seg, w->sc, k, t, b_out, st);
    tm.end();
}

struct BracketResult {
    bool certified = false, overflow = false, nonfinite = false;
    double gL = 0.0, gR = 0.0;
    HostSummary h{};
};

// G(a_L), G(a_R) from the streaming pass's totals
// The filter's finalize kernel forms G(a_L), G(a_R) from its sums and the
// verdict; the host takes the device's verdict as it is, so that the kernels
// launched behind the filter (which test the same verdict) and the host agree.
void certify(const HostSummary& h, BracketResult* res) {
    res->gL = h.g_aL;
    res->gR = h.g_aR;
    res->certified = (h.flags & kFlagCertified) != 0;
}

lapsum_status_t check_args(const float* r, int64_t n, double k, float t, const void* p, const void* b) {
    if (!r || !p || !b) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (n < 1 || n > 0xFFFFFFFFll) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(k > 0.0) || !(k < (double)n) || !std::isfinite(k)) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(t > 0.0f) || !std::isfinite(t)) return LAPSUM_ERR_INVALID_ARGUMENT;
    return LAPSUM_OK;
}

// status of the device-side checks recorded in the control block's flags
lapsum_status_t device_status(int flags) {
    if (flags & kFlagNonFinite) return LAPSUM_ERR_NONFINITE_INPUT;
    if (flags & kFlagInternal) return LAPSUM_ERR_INTERNAL;
    return LAPSUM_OK;
}

// A test hook (lapsum_test_inject_internal): the next solve on the workspace
// ends with its control block marked as a failed consistency check.
void apply_injected(Workspace* w, hipStream_t st) {
    if (!w->inject_internal) return;
    w->inject_internal = false;
    launch_or_flags(w->ctl, kFlagInternal, st);
}

// Waits for the call's work, fills the stats and returns the device-side
// status (a call with stats reports what the device found)
lapsum_status_t fill_stats(Workspace* w, hipStream_t st, long long n, lapsum_stats_t* stats) {
    if (!stats) return LAPSUM_OK;
    launch_sum_p(w->ctl, w->part, w->probs_parts, st);
    if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
    Ctl c;
    if (hipMemcpy(&c, w->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return LAPSUM_ERR_HIP;
    stats->b = c.b;
    stats->sum_p = c.sum_p;
    stats->status = device_status(c.flags);
    return (lapsum_status_t)stats->status;
}

// Waits for the band solve's root summary (written when the host asked for
// it: the root may lie in a bucket too large for LDS).
lapsum_status_t wait_root(Workspace* w, hipStream_t st, unsigned int seq) {
    volatile unsigned int* flag = &w->hs->root_seq;
    auto t0 = std::chrono::steady_clock::now();
    for (unsigned long it = 0;; ++it) {
        if (*flag == seq) { std::atomic_thread_fence(std::memory_order_acquire); return LAPSUM_OK; }
        if ((it & 4095u) == 4095u && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) {
            hipError_t e = hipStreamQuery(st);
            if (e == hipSuccess) {
                if (*flag == seq) { std::atomic_thread_fence(std::memory_order_acquire); return LAPSUM_OK; }
                return LAPSUM_ERR_INTERNAL;
            }
            if (e != hipErrorNotReady) return LAPSUM_ERR_HIP;
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(120)) return LAPSUM_ERR_INTERNAL;
        }
    }
}

lapsum_status_t check_options(const lapsum_options_t& opt) {
    if (opt.path < LAPSUM_PATH_AUTO || opt.path > LAPSUM_PATH_FORCE_FALLBACK) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (opt.bucket_capacity < 1 || opt.bucket_capacity > kBucketCapMax || !(opt.sample_factor > 0.0) ||
        !(opt.delta > 0.0 && opt.delta < 0.5) || !(opt.margin_scale >= 0.0) || opt.max_widen < 0 ||
        opt.cert_mode < 0 || opt.cert_mode > 1)
        return LAPSUM_ERR_INVALID_ARGUMENT;
    return LAPSUM_OK;
}

// the forward solve on a workspace the caller holds (arguments checked)
lapsum_status_t forward_locked(Workspace* w, const float* r, int64_t n, double k, float t_f, float* p, double* b_out,
                               const lapsum_options_t& opt, lapsum_stats_t* stats, hipStream_t st) {
    const double t = (double)t_f;
    Timer tm{w, st, opt.profile != 0};
    if (stats) {
        std::memset(stats, 0, sizeof(*stats));
        stats->a_L = -INFINITY; stats->a_R = INFINITY;
    }
    int path = opt.path;
    if (path == LAPSUM_PATH_AUTO) path = (n > opt.auto_threshold) ? LAPSUM_PATH_BRACKET : LAPSUM_PATH_FULL;

    if (path == LAPSUM_PATH_FULL) {
        run_full(w, r, n, k, t, b_out, st, tm);
        tm.begin("probs");
        w->probs_parts = launch_probs(r, n, t, p, w->ctl, w->part, st);
        tm.end();
        if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
        if (stats) {
            stats->path_taken = 1;
            stats->band_size = n;
            apply_injected(w, st);
            lapsum_status_t fs = fill_stats(w, st, n, stats);
            tm.collect(stats);
            return fs;
        }
        apply_injected(w, st);
        return LAPSUM_OK;
    }

    // ---- bracketing ----
    long long s = (long long)std::ceil(opt.sample_factor * std::sqrt((double)n));
    if (s < 1) s = 1;
    if (s > kSampleMax) s = kSampleMax;
    const double q = 1.0 - k / (double)n;
    long long l0, h0;
    binomial_ranks(s, q, opt.delta, &l0, &h0);
    const double c0 = (double)s * q;
    long long l = (long long)std::llround(c0 - opt.margin_scale * (c0 - (double)l0));
    long long h = (long long)std::llround(c0 + opt.margin_scale * ((double)h0 - c0));
    if (l < 0) l = 0;
    if (h > s + 1) h = s + 1;
    if (l > s) l = s;
    if (h < 1) h = 1;
    if (opt.margin_scale == 1.0) { l = l0; h = h0; }
    const int cap = opt.bucket_capacity;

    uint32_t* shist = next_sample_hist(w);
    tm.begin("sample");
    launch_sample(r, n, t, opt.seed, (int)s, w->sample, nullptr, st, shist, other_sample_hist(w, shist));
    tm.end();
    BracketResult br;
    int widen = 0;
    for (;;) {
        tm.begin("select");
        launch_select(w->sample, (int)s, l, h, cap, w->ctl, w->sp, w->iw, w->bucket_cnt, st, shist, w->swin);
        tm.end();
        const unsigned int seq = ++w->seq;
        tm.begin("filter");
        const int fparts = launch_filter_pass(r, n, t, w->ctl, w->sp, w->iw, w->bucket_cnt, w->bucket_vals, cap,
                                              w->part, st);
        tm.end();
        tm.begin("finalize");
        launch_filter_finalize(n, t, w->ctl, w->bucket_cnt, cap, w->part, fparts, w->hs_dev, seq, st, k, &w->heavy,
                               opt.cert_mode == 1);
        tm.end();
        if (opt.cert_mode == 1) {
            // the pages' certification: one more linear pass sums G(a_L) and
            // G(a_R) directly, and its verdict decides
            tm.begin("cert");
            launch_cert(r, n, t, w->ctl, w->part, w->hs_dev, seq, k, st);
            tm.end();
        }
        if (path != LAPSUM_PATH_FORCE_FALLBACK) {
            // launched before the host has the verdict: they run only when the
            // finalize kernel opened the gate (certified, every band score
            // stored), so the device never waits for the host on this path
            tm.begin("bucket_solve");
            launch_bucket_solve(w->bucket_vals, w->bucket_cnt, cap, kMaxBuckets, w->ctl, w->seg, w->sc, k, t, b_out,
                                st, nullptr, &w->ctl->gate);
            tm.end();
            tm.begin("probs");
            w->probs_parts = launch_probs(r, n, t, p, w->ctl, w->part, st, &w->ctl->gate);
            tm.end();
        }
        if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
        lapsum_status_t ws = wait_summary(w, st, seq);
        if (ws != LAPSUM_OK) return ws;
        br.h = *const_cast<HostSummary*>(w->hs);
        br.nonfinite = (br.h.flags & kFlagNonFinite) != 0;
        br.overflow = (br.h.flags & kFlagOverflow) != 0;
        if (br.nonfinite) break;
        certify(br.h, &br);  // overflow leaves the counts and sums exact
        if (br.certified || path == LAPSUM_PATH_FORCE_FALLBACK) break;
        if (widen >= opt.max_widen) break;
        // widen the failing side: double its distance from s q
        if (br.gL < k) {
            const double d = std::max(1.0, 2.0 * (c0 - (double)l));
            l = (long long)std::floor(c0 - d);
            if (l < 0) l = 0;
        } else {
            const double d = std::max(1.0, 2.0 * ((double)h - c0));
            h = (long long)std::ceil(c0 + d);
            if (h > s + 1) h = s + 1;
        }
        ++widen;
    }
    if (stats) {
        stats->widenings = widen;
        stats->certified = br.certified ? 1 : 0;
        stats->count_below = (int64_t)br.h.c_L;
        stats->band_size = (int64_t)br.h.m;
        stats->count_above = (int64_t)br.h.c_R;
        stats->sample_size = s;
        stats->rank_lo = l;
        stats->rank_hi = h;
        stats->buckets = br.h.nb;
        stats->a_L = br.h.aL;
        stats->a_R = br.h.aR;
        stats->g_aL = br.gL;
        stats->g_aR = br.gR;
        stats->g_aL_direct = br.h.g_aL_direct;
        stats->g_aR_direct = br.h.g_aR_direct;
        stats->tail_S_L = br.h.S_L; stats->tail_S_R = br.h.S_R;
        stats->band_B_L = br.h.B_L; stats->band_B_R = br.h.B_R;
    }
    if (br.nonfinite) {
        launch_set_nan_b(w->ctl, b_out, st);
        launch_fill(p, n, std::numeric_limits<float>::quiet_NaN(), st);
        if (stats) { fill_stats(w, st, n, stats); stats->status = LAPSUM_ERR_NONFINITE_INPUT; tm.collect(stats); }
        return LAPSUM_ERR_NONFINITE_INPUT;
    }
    bool fallback = !br.certified || path == LAPSUM_PATH_FORCE_FALLBACK;
    if (!fallback && !br.overflow) {
        // the gate was open: the band solve and p pass launched behind the filter did the work
        if (stats) {
            stats->path_taken = 2;
            apply_injected(w, st);
            lapsum_status_t fs = fill_stats(w, st, n, stats);
            tm.collect(stats);
            return fs;
        }
        apply_injected(w, st);
        return LAPSUM_OK;
    }
    // Overflowed buckets: the finalize kernel laid out a slot for each (flag
    // kFlagHeavy) unless they would not fit; one more pass over r fills the
    // slots and sums their aggregates in chunks, with no host round trip.
    long long max_heavy = 0;
    bool heavy = false;
    if (!fallback && br.overflow) {
        if (br.h.flags & kFlagHeavy) {
            heavy = true;
            max_heavy = (long long)br.h.max_bucket;
            tm.begin("heavy_collect");
            launch_heavy_collect(r, n, w->ctl, w->sp, w->iw, w->heavy, w->bucket_vals, br.h.hchunks, t, st);
            tm.end();
        } else {
            fallback = true;
        }
    }
    if (fallback) {
        run_full(w, r, n, k, t, b_out, st, tm);
    } else {
        // the root may lie in a bucket too large for the LDS sort: then the
        // band root hands it over (flag, carries as tails, slot offset) and
        // the host sorts that bucket and solves over it
        const bool may_be_big = heavy && max_heavy > kBucketCapMax;
        const unsigned int rseq = may_be_big ? ++w->seq : 0u;
        tm.begin("bucket_solve");
        launch_bucket_solve(w->bucket_vals, w->bucket_cnt, cap, br.h.nb, w->ctl, w->seg, w->sc, k, t, b_out, st,
                            heavy ? &w->heavy : nullptr, nullptr, may_be_big ? w->hs_dev : nullptr, rseq);
        tm.end();
        if (may_be_big) {
            if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
            lapsum_status_t rs = wait_root(w, st, rseq);
            if (rs != LAPSUM_OK) return rs;
            const int rflags = w->hs->root_flags;
            if (rflags & kFlagBigRoot) {
                const unsigned long long cnt = w->hs->root_m;
                const float* src = reinterpret_cast<const float*>(w->bucket_vals + w->hs->root_off);
                tm.begin("root_bucket_sort");
                sort_keys(w, src, (long long)cnt, st);
                tm.end();
                tm.begin("root_bucket_solve");
                launch_curve_tiles(w->keysB, (long long)cnt, w->ctl, w->seg, w->sc, k, t, b_out, st, true);
                tm.end();
            }
        }
    }
    tm.begin("probs");
    w->probs_parts = launch_probs(r, n, t, p, w->ctl, w->part, st);
    tm.end();
    if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
    if (stats) {
        stats->path_taken = fallback ? 3 : 2;
        apply_injected(w, st);
        lapsum_status_t fs = fill_stats(w, st, n, stats);
        tm.collect(stats);
        return fs;
    }
    apply_injected(w, st);
    return LAPSUM_OK;
}

// ---------------------------------------------------------------------------
// k-th and (k+1)-th largest scores (hard top-k threshold, DFTopK midpoint):
// the full sort up to the bracketing threshold, else a noiseless sample, the
// streaming filter and a count-based certification -- both order statistics
// are in the band iff c_R <= k - 1 and c_R + m >= k + 1 (>= n when k = n).
// Leaves the k-th largest in ctl->aR, the (k+1)-th in ctl->aL and their
// midpoint in ctl->b; tau_out (device fp64[2]) may be null.
// ---------------------------------------------------------------------------
lapsum_status_t order_stats_impl(Workspace* w, const float* r, long long n, long long k,
                                 const lapsum_options_t& opt, lapsum_stats_t* stats, hipStream_t st,
                                 double* tau_out) {
    Timer tm{w, st, opt.profile != 0};
    if (stats) {
        std::memset(stats, 0, sizeof(*stats));
        stats->a_L = -INFINITY; stats->a_R = INFINITY;
    }
    int path = opt.path;
    if (path == LAPSUM_PATH_AUTO) path = (n > opt.auto_threshold) ? LAPSUM_PATH_BRACKET : LAPSUM_PATH_FULL;
    auto full_sort = [&]() {
        if (n <= kSmallMax) {
            tm.begin("small_sort");
            launch_small_sort(r, (int)n, w->ctl, w->keysB, st);
            tm.end();
        } else {
            tm.begin("radix_sort");
            sort_keys(w, r, n, st);
            tm.end();
        }
        tm.begin("pick");
        launch_pick_sorted(w->keysB, n, k, w->ctl, tau_out, st);
        tm.end();
    };
    bool fallback = false, certified = false;
    int widen = 0;
    HostSummary h{};
    if (path == LAPSUM_PATH_FULL) {
        full_sort();
        if (stats) stats->path_taken = 1;
    } else {
        long long s = (long long)std::ceil(opt.sample_factor * std::sqrt((double)n));
        s = std::max<long long>(1, std::min<long long>(s, kSampleMax));
        const double q = 1.0 - (double)k / (double)n;
        long long l, hh;
        binomial_ranks(s, q, opt.delta, &l, &hh);
        const double c0 = (double)s * q;
        const int cap = opt.bucket_capacity;
        uint32_t* shist = next_sample_hist(w);
        tm.begin("sample");
        // no noise: the scores themselves
        launch_sample(r, n, 0.0, opt.seed, (int)s, w->sample, nullptr, st, shist, other_sample_hist(w, shist));
        tm.end();
        for (;;) {
            tm.begin("select");
            launch_select(w->sample, (int)s, l, hh, cap, w->ctl, w->sp, w->iw, w->bucket_cnt, st, shist, w->swin);
            tm.end();
            const unsigned int seq = ++w->seq;
            tm.begin("filter");
            launch_filter(r, n, 1.0, w->ctl, w->sp, w->iw, w->bucket_cnt, w->bucket_vals, cap, w->part,
                          w->hs_dev, seq, st, (double)k);
            tm.end();
            if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
            lapsum_status_t ws = wait_summary(w, st, seq);
            if (ws != LAPSUM_OK) return ws;
            h = *const_cast<HostSummary*>(w->hs);
            if (h.flags & kFlagNonFinite) {
                if (stats) { stats->status = LAPSUM_ERR_NONFINITE_INPUT; tm.collect(stats); }
                return LAPSUM_ERR_NONFINITE_INPUT;
            }
            const long long cR = (long long)h.c_R, m = (long long)h.m;
            const bool okR = cR <= k - 1;
            const bool okL = cR + m >= std::min<long long>(k + 1, n);
            if (h.flags & kFlagOverflow) { fallback = true; break; }
            if (okR && okL) { certified = true; break; }
            if (path == LAPSUM_PATH_FORCE_FALLBACK || widen >= opt.max_widen) { fallback = true; break; }
            if (!okR) {
                const double d = std::max(1.0, 2.0 * ((double)hh - c0));
                hh = std::min<long long>((long long)std::ceil(c0 + d), s + 1);
            }
            if (!okL) {
                const double d = std::max(1.0, 2.0 * (c0 - (double)l));
                l = std::max<long long>((long long)std::floor(c0 - d), 0);
            }
            ++widen;
        }
        if (path == LAPSUM_PATH_FORCE_FALLBACK) fallback = true;
        if (fallback) {
            full_sort();
        } else {
            tm.begin("bucket_pick");
            launch_bucket_pick(w->bucket_vals, w->bucket_cnt, cap, k, w->ctl, tau_out, st);
            tm.end();
        }
        if (stats) {
            stats->path_taken = fallback ? 3 : 2;
            stats->widenings = widen;
            stats->certified = certified ? 1 : 0;
            stats->count_below = (int64_t)h.c_L;
            stats->band_size = (int64_t)h.m;
            stats->count_above = (int64_t)h.c_R;
            stats->sample_size = s;
            stats->rank_lo = l;
            stats->rank_hi = hh;
            stats->buckets = h.nb;
            stats->a_L = h.aL;
            stats->a_R = h.aR;
        }
    }
    if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
    if (stats) {
        if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
        Ctl c;
        if (hipMemcpy(&c, w->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return LAPSUM_ERR_HIP;
        stats->b = c.b;
        stats->status = device_status(c.flags);
        tm.collect(stats);
        return (lapsum_status_t)stats->status;
    }
    return LAPSUM_OK;
}

lapsum_status_t check_topk_args(const float* r, int64_t n, int64_t k, long long kmax, const lapsum_options_t& o) {
    if (!r || n < 1 || n > 0xFFFFFFFFll) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (k < 1 || k > kmax) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (o.path < LAPSUM_PATH_AUTO || o.path > LAPSUM_PATH_FORCE_FALLBACK) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (o.bucket_capacity < 1 || o.bucket_capacity > kBucketCapMax || !(o.sample_factor > 0.0) ||
        !(o.delta > 0.0 && o.delta < 0.5) || o.max_widen < 0)
        return LAPSUM_ERR_INVALID_ARGUMENT;
    return LAPSUM_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

void lapsum_default_options(lapsum_options_t* opt) {
    if (!opt) return;
    std::memset(opt, 0, sizeof(*opt));
    opt->path = LAPSUM_PATH_AUTO;
    opt->max_widen = 2;
    opt->seed = 0x5EEDull;
    opt->sample_factor = 4.0;
    opt->delta = 1e-5;
    opt->margin_scale = 1.0;
    opt->auto_threshold = 1000000;
    opt->bucket_capacity = kBucketCapMax;
    opt->profile = 0;
    opt->cert_mode = 0;
}

const char* lapsum_status_string(lapsum_status_t s) {
    switch (s) {
        case LAPSUM_OK: return "ok";
        case LAPSUM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LAPSUM_ERR_NONFINITE_INPUT: return "non-finite score";
        case LAPSUM_ERR_OUT_OF_MEMORY: return "out of device memory";
        case LAPSUM_ERR_HIP: return "HIP runtime error";
        case LAPSUM_ERR_INTERNAL: return "internal consistency check failed";
    }
    return "unknown status";
}

lapsum_status_t lapsum_forward_ex(const float* scores, int64_t n, double k, float t, float* p_out, double* b_out,
                                  const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream) {
    lapsum_options_t o;
    if (opt) o = *opt; else lapsum_default_options(&o);
    lapsum_status_t a = check_args(scores, n, k, t, p_out, b_out);
    if (a != LAPSUM_OK) return a;
    if (check_options(o) != LAPSUM_OK) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, n, &wsg);
        if (gs != LAPSUM_OK) return gs;
        return forward_locked(wsg.w, scores, n, k, t, p_out, b_out, o, stats, st);
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}

lapsum_status_t lapsum_forward(const float* scores, int64_t n, double k, float t, float* p_out, double* b_out,
                               lapsum_stream_t stream) {
    return lapsum_forward_ex(scores, n, k, t, p_out, b_out, nullptr, nullptr, stream);
}

}  // extern "C"

namespace {
lapsum_status_t vjp_impl(const float* scores, const float* g, int64_t n, float t, const double* b, float* grad_out,
                         bool kt, double* dk_out, double* dt_out, const lapsum_options_t* opt,
                         lapsum_stats_t* stats, lapsum_stream_t stream) {
    if (!scores || !g || !b) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (n < 1 || n > 0xFFFFFFFFll) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(t > 0.0f) || !std::isfinite(t)) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, 0, &wsg);
        if (gs != LAPSUM_OK) return gs;
        Workspace* w = wsg.w;
        const bool prof = opt && opt->profile;
        if (stats) std::memset(stats, 0, sizeof(*stats));
        if (prof) {
            while (w->events.size() < 3) { hipEvent_t e; (void)hipEventCreate(&e); w->events.push_back(e); }
            (void)hipEventRecord(w->events[0], st);
        }
        launch_vjp(scores, g, n, (double)t, b, grad_out, w->ctl, w->part, st, prof ? &w->events[1] : nullptr, kt,
                   dk_out, dt_out);
        if (prof) (void)hipEventRecord(w->events[2], st);
        if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
        if (stats) {
            if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
            Ctl c;
            if (hipMemcpy(&c, w->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return LAPSUM_ERR_HIP;
            stats->vjp_c = c.c;
            stats->vjp_sum_f = c.sumf;
            if (prof) {
                float a = 0.0f, bms = 0.0f;
                (void)hipEventElapsedTime(&a, w->events[0], w->events[1]);
                (void)hipEventElapsedTime(&bms, w->events[1], w->events[2]);
                stats->kernel_ms[0] = a; stats->kernel_name[0] = "vjp_reduce";
                stats->n_timed = 1;
                if (grad_out) { stats->kernel_ms[1] = bms; stats->kernel_name[1] = "vjp_apply"; stats->n_timed = 2; }
            }
        }
        return LAPSUM_OK;
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}
}  // namespace

extern "C" {

lapsum_status_t lapsum_vjp_ex(const float* scores, const float* /*p*/, const float* g, int64_t n, float t,
                              const double* b, float* grad_out, const lapsum_options_t* opt,
                              lapsum_stats_t* stats, lapsum_stream_t stream) {
    if (!grad_out) return LAPSUM_ERR_INVALID_ARGUMENT;
    return vjp_impl(scores, g, n, t, b, grad_out, false, nullptr, nullptr, opt, stats, stream);
}

lapsum_status_t lapsum_vjp_kt(const float* scores, const float* g, int64_t n, float t, const double* b,
                              float* grad_out, double* dk_out, double* dt_out, const lapsum_options_t* opt,
                              lapsum_stats_t* stats, lapsum_stream_t stream) {
    if (!grad_out && !dk_out && !dt_out) return LAPSUM_ERR_INVALID_ARGUMENT;
    return vjp_impl(scores, g, n, t, b, grad_out, true, dk_out, dt_out, opt, stats, stream);
}

lapsum_status_t lapsum_vjp(const float* scores, const float* p, const float* g, int64_t n, float t, const double* b,
                           float* grad_out, lapsum_stream_t stream) {
    return lapsum_vjp_ex(scores, p, g, n, t, b, grad_out, nullptr, nullptr, stream);
}

void lapsum_release_workspaces(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_ws) {
        std::lock_guard<std::mutex> wl(kv.second->mu);  // waits for a call in flight on that stream
        free_ws_memory(kv.second);
    }
}

size_t lapsum_workspace_bytes(int64_t n, const lapsum_options_t* opt) {
    lapsum_options_t o;
    if (opt) o = *opt; else lapsum_default_options(&o);
    if (n < 1 || n > 0xFFFFFFFFll || check_options(o) != LAPSUM_OK) return 0;
    return make_layout(std::max<long long>(n, 1 << 16)).total;
}

lapsum_status_t lapsum_test_inject_internal(lapsum_stream_t stream) {
    try {
        WsGuard wsg;
        lapsum_status_t gs = get_ws(reinterpret_cast<hipStream_t>(stream), 0, &wsg);
        if (gs != LAPSUM_OK) return gs;
        wsg.w->inject_internal = true;
        return LAPSUM_OK;
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}

// ---------------------------------------------------------------------------
// stage entry points for parity tests
// ---------------------------------------------------------------------------
lapsum_status_t lapsum_test_binomial_ranks(int64_t s, double q, double delta, int64_t* l, int64_t* h) {
    if (!l || !h || s < 1 || !(q > 0.0 && q < 1.0) || !(delta > 0.0 && delta < 0.5)) return LAPSUM_ERR_INVALID_ARGUMENT;
    long long lo = 0, hi = 0;
    try {
        binomial_ranks(s, q, delta, &lo, &hi);
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
    *l = lo;
    *h = hi;
    return LAPSUM_OK;
}

lapsum_status_t lapsum_test_copy(const float* src, float* dst, int64_t n, lapsum_stream_t stream) {
    if (!src || !dst || n < 1) return LAPSUM_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return LAPSUM_ERR_INVALID_ARGUMENT;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    launch_copy(src, dst, n, st);
    return hip_ok(hipGetLastError());
}

lapsum_status_t lapsum_test_read(const float* src, int64_t n, float* sink, lapsum_stream_t stream) {
    if (!src || !sink || n < 1) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(src) & 15u) return LAPSUM_ERR_INVALID_ARGUMENT;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    launch_read(src, n, sink, st);
    return hip_ok(hipGetLastError());
}

lapsum_status_t lapsum_test_sort_form(const float* scores, int64_t n, float* out, int32_t form,
                                      lapsum_stream_t stream) {
    if (!scores || !out || n < 1 || n > 0xFFFFFFFFll || form < 0 || form > 2) return LAPSUM_ERR_INVALID_ARGUMENT;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsGuard wsg;
    lapsum_status_t gs = get_ws(st, n, &wsg);
    if (gs != LAPSUM_OK) return gs;
    Workspace* w = wsg.w;
    const double k = n > 1 ? 0.5 * (double)n : 0.5;
    if (n <= kSmallMax) {
        launch_small_solve(scores, (int)n, k, 1.0, w->ctl, w->sc, nullptr, w->keysB, st);
    } else {
        sort_keys(w, scores, n, st, form);
    }
    if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
    std::vector<uint32_t> keys((size_t)n);
    if (hipMemcpy(keys.data(), w->keysB, sizeof(uint32_t) * (size_t)n, hipMemcpyDeviceToHost) != hipSuccess)
        return LAPSUM_ERR_HIP;
    std::vector<float> vals((size_t)n);
    for (size_t i = 0; i < (size_t)n; ++i) {
        const uint32_t kk = keys[i];
        const uint32_t u = kk ^ ((kk >> 31) ? 0x80000000u : 0xFFFFFFFFu);
        std::memcpy(&vals[i], &u, 4);
    }
    return hip_ok(hipMemcpy(out, vals.data(), sizeof(float) * (size_t)n, hipMemcpyHostToDevice));
}

lapsum_status_t lapsum_test_sort(const float* scores, int64_t n, float* out, lapsum_stream_t stream) {
    return lapsum_test_sort_form(scores, n, out, 0, stream);
}

lapsum_status_t lapsum_test_sample(const float* scores, int64_t n, float t, uint64_t seed, int64_t s, float* x_out,
                                   int64_t* idx_out, lapsum_stream_t stream) {
    if (!scores || !x_out || n < 1 || s < 1 || s > kSampleMax || !(t > 0.0f)) return LAPSUM_ERR_INVALID_ARGUMENT;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    launch_sample(scores, n, (double)t, seed, (int)s, x_out, reinterpret_cast<long long*>(idx_out), st);
    return hip_ok(hipStreamSynchronize(st));
}

lapsum_status_t lapsum_test_select(const float* x, int64_t s, int64_t l, int64_t h, float* aL_host, float* aR_host,
                                   int32_t* nbuckets_host, lapsum_stream_t stream) {
    if (!x || s < 1 || s > kSampleMax || l < 0 || h > s + 1 || l > s || h < 1) return LAPSUM_ERR_INVALID_ARGUMENT;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsGuard wsg;
    lapsum_status_t gs = get_ws(st, 0, &wsg);
    if (gs != LAPSUM_OK) return gs;
    Workspace* w = wsg.w;
    // as in a forward: the sample histogram, then the gathered window
    uint32_t* shist = next_sample_hist(w);
    launch_key_hist(x, (int)s, shist, other_sample_hist(w, shist), st);
    launch_select(x, (int)s, l, h, kBucketCapMax, w->ctl, w->sp, w->iw, w->bucket_cnt, st, shist, w->swin);
    if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
    Ctl c;
    if (hipMemcpy(&c, w->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return LAPSUM_ERR_HIP;
    if (aL_host) *aL_host = c.aL;
    if (aR_host) *aR_host = c.aR;
    if (nbuckets_host) *nbuckets_host = c.nb;
    return LAPSUM_OK;
}

lapsum_status_t lapsum_test_filter(const float* scores, int64_t n, float t, float a_L, float a_R, int64_t* counts_host,
                                   double* sums_host, float* band_out, int64_t band_cap, int64_t* band_size_host,
                                   int32_t* nbuckets_host, int64_t* bucket_sizes_host, lapsum_stream_t stream) {
    if (!scores || n < 1 || n > 0xFFFFFFFFll || !(t > 0.0f) || !(a_L <= a_R)) return LAPSUM_ERR_INVALID_ARGUMENT;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsGuard wsg;
    lapsum_status_t gs = get_ws(st, n, &wsg);
    if (gs != LAPSUM_OK) return gs;
    Workspace* w = wsg.w;
    // a two-point "sample" whose order statistics are exactly a_L and a_R
    float two[2] = {a_L, a_R};
    if (hipMemcpy(w->sample, two, sizeof(two), hipMemcpyHostToDevice) != hipSuccess) return LAPSUM_ERR_HIP;
    const long long l = std::isinf(a_L) ? 0 : 1;
    const long long h = std::isinf(a_R) ? 3 : 2;
    launch_select(w->sample, 2, l, h, kBucketCapMax, w->ctl, w->sp, w->iw, w->bucket_cnt, st);
    const unsigned int seq = ++w->seq;
    launch_filter(scores, n, (double)t, w->ctl, w->sp, w->iw, w->bucket_cnt, w->bucket_vals, kBucketCapMax, w->part,
                  w->hs_dev, seq, st, 0.5 * (double)n);
    lapsum_status_t ws = wait_summary(w, st, seq);
    if (ws != LAPSUM_OK) return ws;
    HostSummary hsum = *const_cast<HostSummary*>(w->hs);
    if (counts_host) { counts_host[0] = (int64_t)hsum.c_L; counts_host[1] = (int64_t)hsum.m; counts_host[2] = (int64_t)hsum.c_R; }
    if (sums_host) { sums_host[0] = hsum.S_L; sums_host[1] = hsum.S_R; sums_host[2] = hsum.B_L; sums_host[3] = hsum.B_R; }
    if (hsum.flags & kFlagOverflow || (int64_t)hsum.m > band_cap) {
        if (band_size_host) *band_size_host = -1;
        return LAPSUM_OK;
    }
    // gather the band in bucket order (scores inside a bucket are unordered)
    if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
    std::vector<uint32_t> cnt(kMaxBuckets);
    if (hipMemcpy(cnt.data(), w->bucket_cnt, sizeof(uint32_t) * kMaxBuckets, hipMemcpyDeviceToHost) != hipSuccess)
        return LAPSUM_ERR_HIP;
    std::vector<float> band;
    band.reserve((size_t)hsum.m);
    std::vector<uint32_t> buf;
    if (nbuckets_host) *nbuckets_host = hsum.nb;
    for (int b = 0; b < hsum.nb; ++b) {
        if (bucket_sizes_host) bucket_sizes_host[b] = cnt[b];
        if (!cnt[b]) continue;
        buf.resize(cnt[b]);
        if (hipMemcpy(buf.data(), w->bucket_vals + (size_t)b * kBucketCapMax, sizeof(uint32_t) * cnt[b],
                      hipMemcpyDeviceToHost) != hipSuccess)
            return LAPSUM_ERR_HIP;
        for (uint32_t bits : buf) {
            float f;
            std::memcpy(&f, &bits, 4);
            band.push_back(f);
        }
    }
    if (band_size_host) *band_size_host = (int64_t)band.size();
    if (band_out && !band.empty())
        if (hipMemcpy(band_out, band.data(), sizeof(float) * band.size(), hipMemcpyHostToDevice) != hipSuccess)
            return LAPSUM_ERR_HIP;
    return LAPSUM_OK;
}


// ---------------------------------------------------------------------------
// order statistics, hard top-k, DFTopK
// ---------------------------------------------------------------------------
lapsum_status_t lapsum_topk_threshold(const float* scores, int64_t n, int64_t k, double* tau_out,
                                      const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream) {
    lapsum_options_t o;
    if (opt) o = *opt; else lapsum_default_options(&o);
    lapsum_status_t a = check_topk_args(scores, n, k, n, o);
    if (a != LAPSUM_OK || !tau_out) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, n, &wsg);
        if (gs != LAPSUM_OK) return gs;
        Workspace* w = wsg.w;
        return order_stats_impl(w, scores, n, k, o, stats, st, tau_out);
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}

lapsum_status_t lapsum_hard_topk(const float* scores, int64_t n, int64_t k, float* mask_out, double* tau_out,
                                 const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream) {
    lapsum_options_t o;
    if (opt) o = *opt; else lapsum_default_options(&o);
    lapsum_status_t a = check_topk_args(scores, n, k, n, o);
    if (a != LAPSUM_OK || !mask_out) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, n, &wsg);
        if (gs != LAPSUM_OK) return gs;
        Workspace* w = wsg.w;
        lapsum_status_t rs = order_stats_impl(w, scores, n, k, o, stats, st, tau_out);
        if (rs == LAPSUM_ERR_NONFINITE_INPUT) {
            launch_fill(mask_out, n, std::numeric_limits<float>::quiet_NaN(), st);
            return rs;
        }
        if (rs != LAPSUM_OK) return rs;
        launch_mask(scores, n, w->ctl, mask_out, st);
        return hip_ok(hipGetLastError());
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}

lapsum_status_t lapsum_dftopk(const float* scores, int64_t n, int64_t k, float t, float* p_out, double* b_out,
                              const lapsum_options_t* opt, lapsum_stats_t* stats, lapsum_stream_t stream) {
    lapsum_options_t o;
    if (opt) o = *opt; else lapsum_default_options(&o);
    lapsum_status_t a = check_topk_args(scores, n, k, n - 1, o);
    if (a != LAPSUM_OK || !p_out || !(t > 0.0f) || !std::isfinite(t)) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, n, &wsg);
        if (gs != LAPSUM_OK) return gs;
        Workspace* w = wsg.w;
        lapsum_status_t rs = order_stats_impl(w, scores, n, k, o, nullptr, st, nullptr);
        if (rs == LAPSUM_ERR_NONFINITE_INPUT) {
            launch_set_nan_b(w->ctl, b_out, st);
            launch_fill(p_out, n, std::numeric_limits<float>::quiet_NaN(), st);
            return rs;
        }
        if (rs != LAPSUM_OK) return rs;
        launch_copy_b(w->ctl, b_out, st);
        w->probs_parts = launch_probs(scores, n, (double)t, p_out, w->ctl, w->part, st);
        if (hipGetLastError() != hipSuccess) return LAPSUM_ERR_HIP;
        if (stats) {
            std::memset(stats, 0, sizeof(*stats));
            launch_sum_p(w->ctl, w->part, w->probs_parts, st);
            if (hipStreamSynchronize(st) != hipSuccess) return LAPSUM_ERR_HIP;
            Ctl c;
            if (hipMemcpy(&c, w->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return LAPSUM_ERR_HIP;
            stats->b = c.b;
            stats->sum_p = c.sum_p;
            stats->status = device_status(c.flags);
            return (lapsum_status_t)stats->status;
        }
        return LAPSUM_OK;
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}


// ---------------------------------------------------------------------------
// many independent rows
// ---------------------------------------------------------------------------
lapsum_status_t lapsum_forward_batched(const float* scores, int64_t rows, int64_t n, double k, const double* k_rows,
                                       float t, float* p_out, double* b_out, lapsum_stream_t stream) {
    if (!scores || !p_out || !b_out || rows < 1 || rows > 0x7FFFFFFFll || n < 1 || n > 0xFFFFFFFFll)
        return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!k_rows && !(k > 0.0 && k < (double)n && std::isfinite(k))) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(t > 0.0f) || !std::isfinite(t)) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        if (n <= kRowsLdsMax) {
            launch_rows_forward(scores, rows, (int)n, k_rows, k, (double)t, p_out, b_out, st);
            return hip_ok(hipGetLastError());
        }
        if (n <= rows_supported_max()) {
            // one workgroup per row, sorting through scratch of the stream's
            // workspace (its radix key buffer)
            WsGuard wsg;
            lapsum_status_t gs = get_ws(st, (long long)rows_long_scratch_words(rows, (int)n), &wsg);
            if (gs != LAPSUM_OK) return gs;
            launch_rows_forward_long(scores, rows, (int)n, k_rows, k, (double)t, p_out, b_out, wsg.w->keysA, st);
            return hip_ok(hipGetLastError());
        }
        // long rows: the single-vector solver, row by row
        std::vector<double> kh;
        if (k_rows) {
            kh.resize((size_t)rows);
            if (hipMemcpyAsync(kh.data(), k_rows, sizeof(double) * (size_t)rows, hipMemcpyDeviceToHost, st) !=
                    hipSuccess ||
                hipStreamSynchronize(st) != hipSuccess)
                return LAPSUM_ERR_HIP;
        }
        lapsum_options_t o;
        lapsum_default_options(&o);
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, n, &wsg);
        if (gs != LAPSUM_OK) return gs;
        Workspace* w = wsg.w;
        for (int64_t i = 0; i < rows; ++i) {
            const double ki = k_rows ? kh[(size_t)i] : k;
            const float* ri = scores + i * n;
            if (!(ki > 0.0 && ki < (double)n)) {
                launch_set_nan_b(w->ctl, b_out + i, st);
                launch_fill(p_out + i * n, n, std::numeric_limits<float>::quiet_NaN(), st);
                continue;
            }
            lapsum_status_t rs = forward_locked(w, ri, n, ki, t, p_out + i * n, b_out + i, o, nullptr, st);
            if (rs != LAPSUM_OK && rs != LAPSUM_ERR_NONFINITE_INPUT) return rs;
        }
        return hip_ok(hipGetLastError());
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}

lapsum_status_t lapsum_vjp_batched(const float* scores, const float* g, int64_t rows, int64_t n, float t,
                                   const double* b, float* grad_out, lapsum_stream_t stream) {
    if (!scores || !g || !b || !grad_out || rows < 1 || rows > 0x7FFFFFFFll || n < 1 || n > 0xFFFFFFFFll)
        return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(t > 0.0f) || !std::isfinite(t)) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        if (n <= rows_supported_max()) {
            launch_rows_vjp(scores, g, rows, (int)n, (double)t, b, grad_out, st);
            return hip_ok(hipGetLastError());
        }
        WsGuard wsg;
        lapsum_status_t gs = get_ws(st, 0, &wsg);
        if (gs != LAPSUM_OK) return gs;
        Workspace* w = wsg.w;
        for (int64_t i = 0; i < rows; ++i)
            launch_vjp(scores + i * n, g + i * n, n, (double)t, b + i, grad_out + i * n, w->ctl, w->part, st, nullptr,
                       false, nullptr, nullptr);
        return hip_ok(hipGetLastError());
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}

}  // extern "C"
