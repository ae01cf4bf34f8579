// na_unfused_fast.hpp -- geometry of the unfused ops and their register-tiled
// kernels (fp32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "na_index.hpp"

namespace nu {

// One problem in (T, H, W) form; 2D problems have T = 1, k_t = 1, d_t = 1.
struct Geo {
    int ext[3], ker[3], dil[3];
    int tokens;  // per (batch, head)
    int K;       // prod(ker): entries per attention row
    int kw;      // ker[2]
    int khw;     // ker[1] * ker[2]
};

// Register-tiled paths; each returns false (launching nothing) when the
// problem is outside what it covers.
inline bool fast_qk(const Geo &, int64_t, int, const float *, const float *, float, float *,
                    hipStream_t) {
    return false;
}
inline bool fast_av(const Geo &, int64_t, int, const float *, const float *, float, float *,
                    hipStream_t) {
    return false;
}
inline bool fast_av_inverse(const Geo &, int64_t, int, const float *, const float *, float,
                            float *, hipStream_t) {
    return false;
}

}  // namespace nu
