// na_index.hpp -- window and inverse-window arithmetic of neighborhood
// attention on one axis, and the tile plan built on it; usable from host and
// device code.
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

// ----------------------------------------------------------------------------
// Tile plan along one axis. A tile spans `tile` points from `f` (clamped to
// the class), in patches of `p` points. Each patch walks `cnt` patches of the
// other side starting at its own start point; the staged box must hold every
// point any patch reads: from the tile's first start to the last patch's
// start plus cnt * p.

NA_HD int imin_hd(int a, int b) { return a < b ? a : b; }
NA_HD int imax_hd(int a, int b) { return a > b ? a : b; }

// Patches of p points that cover the union of the windows of p consecutive
// queries (that union is at most k + p - 1 long).
NA_HD int window_walk(int k, int p) { return (k + 2 * p - 2) / p; }

// Forward / dq: staged key box [start, start + extent) of the tile at f.
NA_HD void key_box(int f, int tile, int p, int n, int k, int *start, int *extent) {
    const int last_patch = imin_hd(f + tile - p, n - 1);
    const int lastq = imin_hd(f + tile - 1, n - 1);
    *start = window_start(f, n, k);
    const int reach = window_start(imin_hd(last_patch, n - 1), n, k) + window_walk(k, p) * p;
    const int union_end = window_start(lastq, n, k) + k;
    *extent = imax_hd(reach, union_end) - *start;
}

// dk/dv: patches of p queries covering the inverse windows of the p keys of
// the patch at first key f0 (last key f0 + p - 1, clamped).
NA_HD int inverse_walk(int f0, int p, int n, int k) {
    const int l0 = imin_hd(f0 + p - 1, n - 1);
    return (inverse_last(l0, n, k) - inverse_first(f0, n, k) + p) / p;
}

// Largest inverse_walk over the patches of the tile at f.
NA_HD int tile_inverse_walk(int f, int tile, int p, int n, int k) {
    int m = 1;
    for (int x = f; x < f + tile && x < n; x += p) m = imax_hd(m, inverse_walk(x, p, n, k));
    return m;
}

// dk/dv: staged query box of the tile at f, for a walk of cnt patches.
NA_HD void query_box(int f, int tile, int p, int n, int k, int cnt, int *start, int *extent) {
    const int last_patch = imin_hd(f + tile - p, n - 1);
    const int lastk = imin_hd(f + tile - 1, n - 1);
    *start = inverse_first(f, n, k);
    const int reach = inverse_first(last_patch, n, k) + cnt * p;
    const int union_end = inverse_last(lastk, n, k) + 1;
    *extent = imax_hd(reach, union_end) - *start;
}

}  // namespace na
