// Plain streaming kernels that set the achievable HBM ceilings the solver's
// streaming kernels are compared with, and calibrate the hardware traffic
// counters against a transfer of known size.  No arithmetic beyond what keeps
// the loads alive: one tile of kStreamThreads * V float4 per workgroup, the
// fastest plain shape measured for each pattern.
#include <algorithm>

#include "lapsum_launch.h"
#include "lapsum_streamio.h"

namespace lapsum {

constexpr int kCopyV = 1, kReadV = 2;

__global__ __launch_bounds__(kStreamThreads) void k_copy(const float* __restrict__ a, float* __restrict__ b,
                                                          long long n) {
    const long long n4 = n / 4;
    float4* b4 = reinterpret_cast<float4*>(b);
    auto f = [&](const float4& v, long long i) { st4<true>(b4 + i, v); };
    tile_f4<kCopyV, true>(reinterpret_cast<const float4*>(a), n4, false, f, f);
    if (blockIdx.x == 0)
        for (long long j = n4 * 4 + threadIdx.x; j < n; j += kStreamThreads) b[j] = a[j];
}

__global__ __launch_bounds__(kStreamThreads) void k_read(const float* __restrict__ a, long long n,
                                                          float* __restrict__ sink) {
    const long long n4 = n / 4;
    float acc = 0.0f;
    auto f = [&](const float4& v, long long) { acc += (v.x + v.y) + (v.z + v.w); };
    tile_f4<kReadV, true>(reinterpret_cast<const float4*>(a), n4, false, f, f);
    if (blockIdx.x == 0)
        for (long long j = n4 * 4 + threadIdx.x; j < n; j += kStreamThreads) acc += a[j];
    // the sum is only consumed when it hits one exact value, which keeps every
    // load live without a reduction
    if (acc == -1.0f) sink[threadIdx.x] = acc;
}

void launch_copy(const float* a, float* b, long long n, hipStream_t st) {
    const long long g = std::max<long long>(1, stream_tiles<kCopyV>(n / 4));
    hipLaunchKernelGGL(k_copy, dim3((unsigned)std::min<long long>(g, 1 << 24)), dim3(kStreamThreads), 0, st, a, b, n);
}
void launch_read(const float* a, long long n, float* sink, hipStream_t st) {
    const long long g = std::max<long long>(1, stream_tiles<kReadV>(n / 4));
    hipLaunchKernelGGL(k_read, dim3((unsigned)std::min<long long>(g, 1 << 24)), dim3(kStreamThreads), 0, st, a, n, sink);
}

}  // namespace lapsum
