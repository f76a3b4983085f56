// lapsum_forward_noalloc: the forward solve of the full-sort path (Fast
// LapSum paper, gist.science summary section 2.2, full-sort solver) for
// callers that cannot allocate device memory.  Its scratch memory is a
// file-scope device array of fixed size, one per GPU, which lives as long as
// the process; the call itself allocates nothing.
//
// The kernels are the full-sort path's own: the one-workgroup solve up to
// 16384 scores, else the LSD radix sort in its split form (count, scan,
// scatter per digit: every word they read was written by the same sort, so
// nothing carries over from an earlier call), the per-tile curve aggregates
// and the one-workgroup root, then p.  The few words that must start at
// zero (the control block's last-workgroup tickets and the radix histogram
// totals) are cleared by a fill kernel at the start of every call.
#include <cmath>
#include <mutex>

#include "lapsum.h"
#include "lapsum_launch.h"

namespace lapsum {
namespace {

constexpr long long kNoAllocMaxN = 1LL << 20;  // scores per call

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// byte offsets into the scratch array, for up to kNoAllocMaxN scores
struct NoAllocLayout {
    static constexpr long long kTiles = (kNoAllocMaxN + kCurveTile - 1) / kCurveTile;          // curve segments
    static constexpr long long kSplitTiles = (kNoAllocMaxN + kSplitTileKeys - 1) / kSplitTileKeys;
    static constexpr long long kProbParts = (kNoAllocMaxN + 2047) / 2048 + 1;                 // p pass partials
    static constexpr size_t ctl = 0;
    static constexpr size_t hist = align256(ctl + sizeof(Ctl));
    static constexpr size_t goff = align256(hist + sizeof(uint32_t) * kHistRegionWords);
    static constexpr size_t part = align256(goff + sizeof(uint32_t) * 1024);
    static constexpr size_t keysA = align256(part + sizeof(double) * kProbParts);
    static constexpr size_t keysB = align256(keysA + sizeof(uint32_t) * kNoAllocMaxN);
    static constexpr size_t status = align256(keysB + sizeof(uint32_t) * kNoAllocMaxN);  // split counts + offsets
    static constexpr size_t seg = align256(status + sizeof(uint32_t) * 2 * 256 * kSplitTiles);
    // per segment: first, last (f32), P, Bx (f64), cnt, off (u32); solve:
    // pk, bk (f32), pv, bv, bfx (f64), rank (u32)
    static constexpr size_t seg_bytes = (size_t)kTiles * (4 + 4 + 8 + 8 + 4 + 4 + 4 + 4 + 8 + 8 + 8 + 4);
    static constexpr size_t total = align256(seg + seg_bytes + 64 * 12);
};

// The scratch memory.  In host code this name stands for the host-side
// shadow of the symbol, not a device address: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[NoAllocLayout::total];

std::mutex g_sym_mu;
void* g_scratch_ptr[64] = {};  // per device: the address of that device's copy of the array

// The device address of this device's scratch array (set-up on the first
// call on a device, with that device current).
lapsum_status_t scratch_for_device(int dev, unsigned char** out) {
    if (dev < 0 || dev >= 64) return LAPSUM_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lk(g_sym_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LAPSUM_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
    return LAPSUM_OK;
}

// zeroes n32 words at p (a kernel, not a memset: fits in a captured stream)
__global__ void k_zero_words(uint32_t* p, int n32) {
    for (int i = threadIdx.x; i < n32; i += blockDim.x) p[i] = 0u;
}

template <class T>
T* at(unsigned char* base, size_t off) { return reinterpret_cast<T*>(base + off); }

}  // namespace
}  // namespace lapsum

using namespace lapsum;

extern "C" lapsum_status_t lapsum_forward_noalloc(const float* scores, int64_t n, double k, float t, float* p_out,
                                                  double* b_out, lapsum_stream_t stream) {
    if (!scores || !p_out || !b_out) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (n < 1 || n > kNoAllocMaxN) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(k > 0.0) || !(k < (double)n) || !std::isfinite(k)) return LAPSUM_ERR_INVALID_ARGUMENT;
    if (!(t > 0.0f) || !std::isfinite(t)) return LAPSUM_ERR_INVALID_ARGUMENT;
    try {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return LAPSUM_ERR_HIP;
        unsigned char* base = nullptr;
        lapsum_status_t s = scratch_for_device(dev, &base);
        if (s != LAPSUM_OK) return s;
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        using Lay = NoAllocLayout;
        Ctl* ctl = at<Ctl>(base, Lay::ctl);
        uint32_t* hist = at<uint32_t>(base, Lay::hist);
        // the control block and the histogram totals start at zero
        hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(base),
                           (int)(Lay::goff / sizeof(uint32_t)));
        unsigned char* sg = base + Lay::seg;
        const size_t T = (size_t)Lay::kTiles;
        SegArrays seg{reinterpret_cast<float*>(sg), reinterpret_cast<float*>(sg + 4 * T),
                      reinterpret_cast<double*>(sg + 8 * T), reinterpret_cast<double*>(sg + 16 * T),
                      reinterpret_cast<uint32_t*>(sg + 24 * T), reinterpret_cast<uint32_t*>(sg + 28 * T)};
        unsigned char* sv = sg + 32 * T;
        SolveScratch sc{reinterpret_cast<float*>(sv), reinterpret_cast<double*>(sv + 8 * T),
                        reinterpret_cast<float*>(sv + 4 * T), reinterpret_cast<double*>(sv + 16 * T),
                        reinterpret_cast<double*>(sv + 24 * T), reinterpret_cast<uint32_t*>(sv + 32 * T),
                        nullptr, nullptr};
        const double td = (double)t;
        if (n <= kSmallMax) {
            launch_small_solve(scores, (int)n, k, td, ctl, sc, b_out, nullptr, st);
        } else {
            uint32_t* keysA = at<uint32_t>(base, Lay::keysA);
            uint32_t* keysB = at<uint32_t>(base, Lay::keysB);
            launch_radix_sort(scores, n, keysA, keysB, hist, at<uint32_t>(base, Lay::goff),
                              at<unsigned long long>(base, Lay::status), 1u, ctl, st, 2);
            launch_curve_tiles(keysB, n, ctl, seg, sc, k, td, b_out, st);
        }
        launch_probs(scores, n, td, p_out, ctl, at<double>(base, Lay::part), st);
        return hipGetLastError() == hipSuccess ? LAPSUM_OK : LAPSUM_ERR_HIP;
    } catch (...) {
        return LAPSUM_ERR_INTERNAL;
    }
}
