// Load pipeline of the streaming passes (gfx950): 16-byte loads, several in
// flight per thread, over one or two fp32 arrays.
#pragma once
#include "lapsum_device.h"

namespace lapsum {

// ---------------------------------------------------------------------------
// Grid-stride streaming over float4 elements [0, n4) with U loads in flight
// per thread: the next U loads are issued before the current U are consumed
// (software pipelining -- a single load in flight per wave leaves HBM idle
// while the wave computes).  The main loop's trip test uses the wave's last
// lane, so all 64 lanes iterate together (wave-wide ballots are safe inside
// main); leftover elements go to tail, one per lane.  reverse = true walks
// the array from its end, so a pass can start on the part of an array the
// previous pass read last (still in the memory-side cache).
// main(v, idx) / tail(v, idx): v = element idx.
// ---------------------------------------------------------------------------
typedef float f4v __attribute__((ext_vector_type(4)));

// 16-byte load, optionally non-temporal (streamed past the caches)
template <bool NT>
LS_DEV float4 ld4(const float4* p) {
    if (NT) {
        const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    }
    return *p;
}

// 16-byte store, optionally non-temporal: the streamed outputs (p, grad) are
// not read back by this step, and keeping them out of the caches leaves the
// latency-bound kernels of the next step less dirty data to write back
template <bool NT>
LS_DEV void st4(float4* p, float4 v) {
    if (NT) {
        const f4v t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f4v*>(p));
    } else {
        *p = v;
    }
}

template <int U, bool NT = false, class Main, class Tail>
LS_DEV void stream_f4(const float4* __restrict__ a, long long n4, bool reverse, Main&& main, Tail&& tail) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // logical position
    const long long last = 63 - (long long)lane_id();
    const long long step = reverse ? -stride : stride;                // physical step (wave-uniform)
    long long idx = reverse ? n4 - 1 - i : i;                         // physical index of i
    // the trip test is made explicitly wave-uniform; the prefetch offset is a
    // wave-uniform scalar (when there is no next batch the prefetch re-reads
    // the current one), so every load address is base + scalar and the
    // compiler keeps the prefetches in flight while the current batch is used
    auto uniform = [](bool c) { return __builtin_amdgcn_readfirstlane((int)c) != 0; };
    if (uniform(i + last + (long long)(U - 1) * stride < n4)) {
        float4 cur[U];
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = ld4<NT>(a + idx + u * step);
        while (true) {
            const bool hn = uniform(i + (long long)U * stride + last + (long long)(U - 1) * stride < n4);
            const long long poff = hn ? (long long)U * step : 0;
            float4 nx[U];
#pragma unroll
            for (int u = 0; u < U; ++u) nx[u] = ld4<NT>(a + idx + poff + u * step);
#pragma unroll
            for (int u = 0; u < U; ++u) main(cur[u], idx + u * step);
            i += (long long)U * stride;
            idx += (long long)U * step;
            if (!hn) break;
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nx[u];
        }
    }
    for (; i < n4; i += stride, idx += step) tail(a[idx], idx);
}

// the same over two arrays read in lockstep
template <int U, bool NT = false, class Main, class Tail>
LS_DEV void stream_f4x2(const float4* __restrict__ a, const float4* __restrict__ b, long long n4, bool reverse,
                        Main&& main, Tail&& tail) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long last = 63 - (long long)lane_id();
    const long long step = reverse ? -stride : stride;
    long long idx = reverse ? n4 - 1 - i : i;
    auto uniform = [](bool c) { return __builtin_amdgcn_readfirstlane((int)c) != 0; };
    if (uniform(i + last + (long long)(U - 1) * stride < n4)) {
        float4 ca[U], cb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) { ca[u] = ld4<NT>(a + idx + u * step); cb[u] = ld4<NT>(b + idx + u * step); }
        while (true) {
            const bool hn = uniform(i + (long long)U * stride + last + (long long)(U - 1) * stride < n4);
            const long long poff = hn ? (long long)U * step : 0;
            float4 na[U], nb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                na[u] = ld4<NT>(a + idx + poff + u * step);
                nb[u] = ld4<NT>(b + idx + poff + u * step);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) main(ca[u], cb[u], idx + u * step);
            i += (long long)U * stride;
            idx += (long long)U * step;
            if (!hn) break;
#pragma unroll
            for (int u = 0; u < U; ++u) { ca[u] = na[u]; cb[u] = nb[u]; }
        }
    }
    for (; i < n4; i += stride, idx += step) tail(a[idx], b[idx], idx);
}


// ---------------------------------------------------------------------------
// Tiled streaming over float4 elements [0, n4).  Tile j is the contiguous
// run [j*T, (j+1)*T) with T = kStreamThreads * V; thread t of a workgroup
// takes elements t + v*kStreamThreads of the tile, issuing all V loads before
// using any.  Workgroup b walks tiles b, b + gridDim.x, ... (from the last
// tile down when reverse), so with one tile per workgroup the hardware's
// in-order dispatch sweeps memory front to back, and with fewer workgroups
// each one walks tiles at a fixed stride.  main(v, idx) runs on full tiles
// (the test is workgroup-uniform, every lane active: wave-wide operations are
// safe); tail(v, idx) on the elements of a partial last tile.
// ---------------------------------------------------------------------------
template <int V>
__host__ __device__ inline long long stream_tiles(long long n4) {
    const long long T = (long long)kStreamThreads * V;
    return (n4 + T - 1) / T;
}

template <int V, bool NT, class Main, class Tail>
LS_DEV void tile_f4(const float4* __restrict__ a, long long n4, bool reverse, Main&& main, Tail&& tail) {
    constexpr long long T = (long long)kStreamThreads * V;
    const long long ntiles = stream_tiles<V>(n4);
    for (long long j = blockIdx.x; j < ntiles; j += gridDim.x) {
        const long long tile = reverse ? ntiles - 1 - j : j;
        const long long base = tile * T + threadIdx.x;
        if ((tile + 1) * T <= n4) {
            float4 x[V];
#pragma unroll
            for (int v = 0; v < V; ++v) x[v] = ld4<NT>(a + base + v * kStreamThreads);
#pragma unroll
            for (int v = 0; v < V; ++v) main(x[v], base + v * kStreamThreads);
        } else {
            for (int v = 0; v < V; ++v) {
                const long long i = base + v * kStreamThreads;
                if (i < n4) tail(a[i], i);
            }
        }
    }
}

// tile_f4 for workgroups that walk several tiles and compute a lot per
// element: the next tile's loads are issued before the current tile is
// consumed.  The prefetch is unconditional (a wave-uniform choice of tile: the
// next one when it is full, else the current one again, else tile 0), so the
// compiler keeps it in flight instead of waiting for all loads.
template <int V, bool NT, class Main, class Tail>
LS_DEV void tile_f4_pipelined(const float4* __restrict__ a, long long n4, Main&& main, Tail&& tail) {
    constexpr long long T = (long long)kStreamThreads * V;
    const long long ntiles = stream_tiles<V>(n4);
    if (n4 < T) {  // no full tile at all
        tile_f4<V, NT>(a, n4, false, main, tail);
        return;
    }
    long long j = blockIdx.x;
    if (j >= ntiles) return;
    auto full = [&](long long tile) { return (tile + 1) * T <= n4; };
    const long long tid = threadIdx.x;
    float4 x[V];
    {
        const long long first = full(j) ? j : 0;
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = ld4<NT>(a + first * T + tid + v * kStreamThreads);
    }
    while (true) {
        const long long jn = j + gridDim.x;
        const long long pf = (jn < ntiles && full(jn)) ? jn : (full(j) ? j : 0);
        float4 y[V];
#pragma unroll
        for (int v = 0; v < V; ++v) y[v] = ld4<NT>(a + pf * T + tid + v * kStreamThreads);
        if (full(j)) {
#pragma unroll
            for (int v = 0; v < V; ++v) main(x[v], j * T + tid + v * kStreamThreads);
        } else {
            for (int v = 0; v < V; ++v) {
                const long long i = j * T + tid + v * kStreamThreads;
                if (i < n4) tail(a[i], i);
            }
        }
        if (jn >= ntiles) break;
        j = jn;
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = y[v];
    }
}

// Wave tiles of 64 * V float4 handed out at run time inside a workgroup
// that owns tiles [t0, t1).  Wave w starts on tile t0 + w, issuing its loads
// before prologue() runs (the workgroup's set-up, which must end with a
// barrier and is called by every thread); every further tile comes from an
// LDS counter, claimed one tile ahead (the claim's latency hides behind the
// current tile) and prefetched before the current one is used.  The waves
// the CU serves faster take more tiles, so the workgroup's waves finish
// together.  prologue() must set *s_ctr to 0.  main(v, idx) runs on full
// tiles (every lane of the wave active); tail(v, idx) on the elements of a
// partial last tile; tile_end(j) after each tile j, by the whole wave (so
// that what depends on which wave met which tile can be settled per tile).
// Needs n4 >= 64 * V (a full tile 0 to fall back on).
template <int V, bool NT, class Main, class Tail, class Prologue, class TileEnd>
LS_DEV void wave_tiles_dynamic(const float4* __restrict__ a, long long n4, long long t0, long long t1,
                               unsigned int* s_ctr, Main&& main, Tail&& tail, Prologue&& prologue,
                               TileEnd&& tile_end) {
    constexpr long long T = 64LL * V;
    const long long lane = lane_id();
    const long long nw = blockDim.x >> 6;
    auto claim = [&]() -> unsigned int {
        unsigned int c = 0u;
        if (lane == 0) c = atomicAdd(s_ctr, 1u);
        return c;
    };
    auto full = [&](long long t) { return (t + 1) * T <= n4; };
    long long j = t0 + (long long)(threadIdx.x >> 6);
    float4 x[V];
    {
        const long long src = (j < t1 && full(j)) ? j : 0;  // a partial tile is read in the tail path
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = ld4<NT>(a + src * T + lane + v * 64);
    }
    prologue();
    if (j >= t1) return;
    unsigned int cn = claim();  // the tile after j
    while (true) {
        const long long jn = t0 + nw + (long long)__builtin_amdgcn_readfirstlane(cn);
        const bool more = jn < t1;  // wave-uniform
        if (more) cn = claim();
        const long long pf = (more && full(jn)) ? jn : (full(j) ? j : 0);
        float4 y[V];
#pragma unroll
        for (int v = 0; v < V; ++v) y[v] = ld4<NT>(a + pf * T + lane + v * 64);
        if (full(j)) {
#pragma unroll
            for (int v = 0; v < V; ++v) main(x[v], j * T + lane + v * 64);
        } else {
            for (int v = 0; v < V; ++v) {
                const long long i = j * T + lane + v * 64;
                if (i < n4) tail(a[i], i);
            }
        }
        tile_end(j);
        if (!more) break;
        j = jn;
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = y[v];
    }
}

// the same over two arrays read in lockstep
template <int V, bool NT, class Main, class Tail>
LS_DEV void tile_f4x2(const float4* __restrict__ a, const float4* __restrict__ b, long long n4, bool reverse,
                      Main&& main, Tail&& tail) {
    constexpr long long T = (long long)kStreamThreads * V;
    const long long ntiles = stream_tiles<V>(n4);
    for (long long j = blockIdx.x; j < ntiles; j += gridDim.x) {
        const long long tile = reverse ? ntiles - 1 - j : j;
        const long long base = tile * T + threadIdx.x;
        if ((tile + 1) * T <= n4) {
            float4 x[V], y[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                x[v] = ld4<NT>(a + base + v * kStreamThreads);
                y[v] = ld4<NT>(b + base + v * kStreamThreads);
            }
#pragma unroll
            for (int v = 0; v < V; ++v) main(x[v], y[v], base + v * kStreamThreads);
        } else {
            for (int v = 0; v < V; ++v) {
                const long long i = base + v * kStreamThreads;
                if (i < n4) tail(a[i], b[i], i);
            }
        }
    }
}

}  // namespace lapsum
