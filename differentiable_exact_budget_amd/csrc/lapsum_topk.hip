// Order statistics from the top: the k-th and (k+1)-th largest scores, the
// hard top-k mask and the DFTopK threshold (Fast LapSum paper, gist.science
// summary section 2.3: DFTopK puts the threshold at the midpoint of those two
// order statistics; it is LapSum's zero-temperature limit).
//
// They reuse the solver's machinery: the full sort for n <= the bracketing
// threshold, else a noiseless sample, the streaming filter (its counts and
// value-ordered buckets; its exp-sums go unused) and a count-based
// certification -- both order statistics lie in the band when
// c_R <= k - 1 and c_R + m >= k + 1 -- after which only the bucket(s) holding
// ranks k and k+1 from the top are sorted.
//
//  k_small_sort   n <= 16384: sort in LDS, write the sorted keys
//  k_pick_sorted  pick from a fully sorted key array
//  k_bucket_pick  one workgroup: locate ranks k, k+1 in the buckets, sort
//                 those buckets in LDS, pick
//  k_mask         mask_i = 1 where r_i >= the k-th largest
#include "lapsum_launch.h"
#include "lapsum_streamio.h"

namespace lapsum {

constexpr int kPickThreads = 1024;

__global__ __launch_bounds__(kPickThreads) void k_small_sort(const float* __restrict__ r, int n, Ctl* ctl,
                                                              uint32_t* keys_out) {
    __shared__ uint32_t keys[kSmallMax];
    __shared__ int s_bad;
    const int tid = threadIdx.x;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    const int np = max(next_pow2(n), 64);
    int bad = 0;
    for (int i = tid; i < np; i += kPickThreads) {
        if (i < n) {
            const float v = r[i];
            bad |= !finite_f(v);
            keys[i] = f2key(v);
        } else {
            keys[i] = 0xFFFFFFFFu;  // above every finite key: stays past the end
        }
    }
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    sort_pow2_lds<kPickThreads>(keys, np);
    for (int i = tid; i < n; i += kPickThreads) keys_out[i] = keys[i];
    if (tid == 0) ctl->flags = s_bad ? kFlagNonFinite : 0;
}

LS_DEV void write_order_stats(Ctl* ctl, double tk, double tk1, double* tau_out) {
    ctl->aL = (float)tk1;  // (k+1)-th largest
    ctl->aR = (float)tk;   // k-th largest
    ctl->b = 0.5 * (tk + tk1);
    if (tau_out) { tau_out[0] = tk; tau_out[1] = tk1; }
}

__global__ void k_pick_sorted(const uint32_t* keys, long long n, long long k, Ctl* ctl, double* tau_out) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const double tk = (double)key2f(keys[n - k]);
    const double tk1 = k < n ? (double)key2f(keys[n - k - 1]) : -INFINITY;
    write_order_stats(ctl, tk, tk1, tau_out);
}

// Ranks k and k+1 from the top, in the band: j = k - c_R and j + 1.  With
// per-bucket counts and the buckets in ascending value order, the bucket that
// holds the j-th largest band score is the one where the count of scores in
// higher buckets, above, satisfies above < j <= above + cnt.
__global__ __launch_bounds__(kPickThreads) void k_bucket_pick(const uint32_t* bucket_vals, const uint32_t* bucket_cnt,
                                                               int cap, long long k, Ctl* ctl, double* tau_out) {
    __shared__ uint32_t sortbuf[kBucketCapMax];
    __shared__ uint32_t scr[kPickThreads / 64 + 2];
    __shared__ int s_bkt[2];
    __shared__ uint32_t s_above[2];
    __shared__ double s_val[2];
    const int tid = threadIdx.x;
    const int nb = ctl->nb;
    const long long cR = (long long)ctl->c_R, m = (long long)ctl->m;
    const long long j1 = k - cR;  // >= 1 (certified)
    const bool want2 = k + 1 - cR <= m;
    // bucket tid counted from the top: reversed exclusive scan of the counts
    const int rb = nb - 1 - tid;  // this thread's bucket, visited top-down
    const uint32_t c = (tid < nb) ? min(bucket_cnt[rb], (uint32_t)cap) : 0u;
    const uint32_t above = block_exclusive_scan<kPickThreads>(c, nullptr, scr);
    if (tid == 0) { s_bkt[0] = -1; s_bkt[1] = -1; }
    __syncthreads();
    if (tid < nb && c > 0u) {
        if ((long long)above < j1 && j1 <= (long long)above + c) { s_bkt[0] = rb; s_above[0] = above; }
        if (want2 && (long long)above < j1 + 1 && j1 + 1 <= (long long)above + c) { s_bkt[1] = rb; s_above[1] = above; }
    }
    __syncthreads();
    for (int q = 0; q < 2; ++q) {
        const int bkt = s_bkt[q];
        if (q == 1 && (!want2 || bkt == s_bkt[0])) break;  // uniform
        if (bkt < 0) {
            if (tid == 0) atomicOr(&ctl->flags, kFlagInternal);
            break;
        }
        const int cnt = (int)min(bucket_cnt[bkt], (uint32_t)cap);
        const int np = max(next_pow2(cnt), 64);
        for (int i = tid; i < np; i += kPickThreads)
            sortbuf[i] = i < cnt ? f2key(__uint_as_float(bucket_vals[(size_t)bkt * (size_t)cap + i])) : 0xFFFFFFFFu;
        __syncthreads();
        sort_pow2_lds<kPickThreads>(sortbuf, np);
        if (tid == 0) {
            // ascending position of the j-th largest of this bucket
            const long long jj = (q == 0 ? j1 : j1 + 1) - (long long)s_above[q];
            s_val[q] = (double)key2f(sortbuf[cnt - jj]);
            if (q == 0 && want2 && s_bkt[1] == bkt) s_val[1] = (double)key2f(sortbuf[cnt - jj - 1]);
        }
        __syncthreads();
    }
    if (tid == 0) write_order_stats(ctl, s_val[0], want2 ? s_val[1] : -INFINITY, tau_out);
}

template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void k_mask(const float* __restrict__ r, long long n,
                                                          const Ctl* ctl, float* __restrict__ mask) {
    const float tk = ctl->aR;
    auto one = [&](float v) -> float { return v >= tk ? 1.0f : 0.0f; };
    if (VEC) {
        const long long n4 = n >> 2;
        float4* m4 = reinterpret_cast<float4*>(mask);
        auto body = [&](float4 q, long long idx) { m4[idx] = make_float4(one(q.x), one(q.y), one(q.z), one(q.w)); };
        tile_f4<2, true>(reinterpret_cast<const float4*>(r), n4, false, body, body);
        if (blockIdx.x == 0) {
            const long long j = (n4 << 2) + threadIdx.x;
            if (threadIdx.x < 4 && j < n) mask[j] = one(r[j]);
        }
    } else {
        const long long stride = (long long)gridDim.x * kStreamThreads;
        for (long long i = (long long)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride) mask[i] = one(r[i]);
    }
}

__global__ void k_copy_b(const Ctl* ctl, double* b_out) { *b_out = ctl->b; }
void launch_copy_b(const Ctl* ctl, double* b_out, hipStream_t st) {
    if (b_out) hipLaunchKernelGGL(k_copy_b, dim3(1), dim3(1), 0, st, ctl, b_out);
}

void launch_small_sort(const float* r, int n, Ctl* ctl, uint32_t* keys_out, hipStream_t st) {
    hipLaunchKernelGGL(k_small_sort, dim3(1), dim3(kPickThreads), 0, st, r, n, ctl, keys_out);
}

void launch_pick_sorted(const uint32_t* keys, long long n, long long k, Ctl* ctl, double* tau_out, hipStream_t st) {
    hipLaunchKernelGGL(k_pick_sorted, dim3(1), dim3(64), 0, st, keys, n, k, ctl, tau_out);
}

void launch_bucket_pick(const uint32_t* bucket_vals, const uint32_t* bucket_cnt, int cap, long long k, Ctl* ctl,
                        double* tau_out, hipStream_t st) {
    hipLaunchKernelGGL(k_bucket_pick, dim3(1), dim3(kPickThreads), 0, st, bucket_vals, bucket_cnt, cap, k, ctl,
                       tau_out);
}

void launch_mask(const float* r, long long n, const Ctl* ctl, float* mask, hipStream_t st) {
    const bool vec = ((reinterpret_cast<uintptr_t>(r) | reinterpret_cast<uintptr_t>(mask)) & 15u) == 0u;
    if (vec) {
        const long long g = std::max<long long>(1, std::min<long long>(stream_tiles<2>(n >> 2), 1 << 24));
        hipLaunchKernelGGL(k_mask<true>, dim3((unsigned)g), dim3(kStreamThreads), 0, st, r, n, ctl, mask);
    } else {
        hipLaunchKernelGGL(k_mask<false>, dim3(stream_blocks(n)), dim3(kStreamThreads), 0, st, r, n, ctl, mask);
    }
}

}  // namespace lapsum
