// na_index.hpp -- window and inverse-window arithmetic of neighborhood
// attention on one axis, usable from host and device code.
//
// The window rule (NATTEN issue #161, "Backward pass is very slow towards much
// tokens and large kernels": windows of kernel_size keys around each query,
// kept at full size at the grid borders) is applied inside one residue class
// of a dilated axis, in sub-grid coordinates: an axis of extent L at dilation
// d splits into d classes r = 0..d-1, class r holding the n_r = ceil((L-r)/d)
// coordinates r, r+d, r+2d, ... Everything below works on the class index i.
//
// All arithmetic is int32: extents here are bounded by the token count of one
// batch element, which the host checks against INT32_MAX.
#pragma once

#if defined(__HIPCC__)
#define NA_HD __host__ __device__ __forceinline__
#else
#define NA_HD inline
#endif

namespace na {

// Number of positions of residue class r on an axis of extent L at dilation d.
NA_HD int class_size(int L, int d, int r) { return (L - r + d - 1) / d; }

// First key (class index) of the window of query class index i, for a class
// of n positions and window size k (1 <= k <= n): centered (floor(k/2) keys
// before the query), then shifted inward so the k keys stay in [0, n).
NA_HD int window_start(int i, int n, int k) {
    int s = i - k / 2;
    s = s < 0 ? 0 : s;
    int hi = n - k;
    return s > hi ? hi : s;
}

// Queries (class indices) whose window contains key j form one contiguous
// range [inverse_first, inverse_last]. window_start is non-decreasing in i
// and grows by at most one per step, so the range is found in closed form:
//  * the first query has window_start >= j - k + 1: that is 0 when
//    j - k + 1 <= 0, else the query whose centered start equals j - k + 1;
//  * the last query has window_start <= j: that is n - 1 when the window is
//    already pinned to the high border (j >= n - k), else j + floor(k/2).
NA_HD int inverse_first(int j, int n, int k) {
    (void)n;
    return (j - k + 1 <= 0) ? 0 : j - k + 1 + k / 2;
}
NA_HD int inverse_last(int j, int n, int k) { return (j >= n - k) ? n - 1 : j + k / 2; }

}  // namespace na
