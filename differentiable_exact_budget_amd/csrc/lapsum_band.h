// Band buckets of the bracketing path: the filter and the heavy-bucket pass
// map a band score to its value-ordered bucket the same way.
#pragma once
#include "lapsum_device.h"

namespace lapsum {

struct FilterState {
    float aL, aR, ls;
    int ng, J, cap;
    const float* sp;
    const float* iw;
    uint32_t* bucket_cnt;
    uint32_t* bucket_vals;
};

// bucket of a band score: splitter gap by binary search, then equal-width
// sub-bucket inside a finite gap (monotone in v)
LS_DEV int band_bucket(const FilterState& fs, float v) {
    static_assert((kMaxBuckets & (kMaxBuckets - 1)) == 0, "the search below covers gaps < kMaxBuckets");
    int g = 0;
    for (int step = kMaxBuckets / 2; step > 0; step >>= 1)
        if (g + step < fs.ng && fs.sp[g + step] <= v) g += step;
    int sub = 0;
    const float iwg = fs.iw[g];
    if (fs.J > 1 && iwg > 0.0f) {
        const float f = (v - fs.sp[g]) * iwg;
        sub = f < (float)(fs.J - 1) ? (int)f : fs.J - 1;
    }
    return g * fs.J + sub;
}

}  // namespace lapsum
