// na_mask.hip -- the window mask of the masked entry points built from an
// index tensor of attended tokens (na_window_mask_from_indices, include/na.h).
//
// NATTEN issue #161, "Backward pass is very slow towards much tokens and large
// kernels": for a time kernel that changes from frame to frame, the requester
// asks to pass the attended tokens of each query as an index tensor (to
// na3d_qk); the maintainer answers that a tiled kernel keeps the largest window
// and only masks inside it. So every listed token must lie in the query's
// window, and it becomes one byte of the query's mask row: the byte of its
// offset in the window (row-major over the window's (t, h, w) offsets), the
// layout the masked fused kernels and na_qk read.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "na.h"
#include "na_index.hpp"

namespace {

// Grid of one batch element, outermost axis first; a 2D grid has T = 1 with a
// window of 1 and dilation 1 along it.
struct MaskGrid {
    int ext[3], ker[3], dil[3];
    int tokens;  // T * H * W
    int K;       // prod(ker)
};

constexpr int kThreads = 256;

// Offset of key coordinate y in the window of query coordinate x along one
// axis (extent L, window k, dilation d), or -1 when y is outside that window:
// another residue class, or a class index outside [start, start + k).
__device__ __forceinline__ int axis_offset(int x, int y, int L, int k, int d) {
    const int r = x % d;
    if (y % d != r) return -1;
    const int s = na::window_start(x / d, na::class_size(L, d, r), k);
    const int j = y / d - s;
    return (unsigned)j < (unsigned)k ? j : -1;
}

// Clears n bytes: 16 per thread and grid-stride step, with one 16-byte store
// where the destination is 16-byte aligned and whole, bytes otherwise.
__global__ void __launch_bounds__(kThreads) clear_bytes_kernel(uint8_t *dst, int64_t n) {
    const bool vec = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
    const int64_t chunks = (n + 15) / 16;
    for (int64_t c = blockIdx.x * (int64_t)kThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kThreads) {
        const int64_t b = c * 16;
        if (vec && b + 16 <= n) {
            *reinterpret_cast<uint4 *>(dst + b) = make_uint4(0u, 0u, 0u, 0u);
        } else {
            for (int64_t i = b; i < n && i < b + 16; ++i) dst[i] = 0;
        }
    }
}

// One thread per query token x: each of its m slots holding a token of x's
// window sets that key's byte of x's (cleared) mask row; bad[x] = the number
// of slots that hold neither -1 nor a token of x's window. A thread writes
// only its own row and its own count, so no two threads touch one byte.
__global__ void __launch_bounds__(kThreads) mask_from_indices_kernel(MaskGrid g,
                                                                     const int64_t *indices,
                                                                     int m, uint8_t *mask,
                                                                     int32_t *bad) {
    const int64_t x = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (x >= g.tokens) return;
    const int xi = (int)x;
    const int hw = g.ext[1] * g.ext[2];
    const int xt = xi / hw, xh = (xi / g.ext[2]) % g.ext[1], xw = xi % g.ext[2];
    uint8_t *row = mask + x * g.K;
    const int64_t *slot = indices + x * m;
    int nbad = 0;
    for (int s = 0; s < m; ++s) {
        const int64_t y = slot[s];
        if (y == -1) continue;
        if (y < 0 || y >= g.tokens) {
            ++nbad;
            continue;
        }
        const int yi = (int)y;
        const int yt = yi / hw, yh = (yi / g.ext[2]) % g.ext[1], yw = yi % g.ext[2];
        const int jt = axis_offset(xt, yt, g.ext[0], g.ker[0], g.dil[0]);
        const int jh = axis_offset(xh, yh, g.ext[1], g.ker[1], g.dil[1]);
        const int jw = axis_offset(xw, yw, g.ext[2], g.ker[2], g.dil[2]);
        if (jt < 0 || jh < 0 || jw < 0) {
            ++nbad;
            continue;
        }
        row[(jt * g.ker[1] + jh) * g.ker[2] + jw] = 1;
    }
    bad[x] = nbad;
}

// The grid fields of a problem (extent, kernel, dilation; the other fields
// are not read): 2 or 3 axes, 1 <= kernel <= extent / dilation per axis, at
// most INT32_MAX tokens.
bool mask_grid(const na_problem *p, MaskGrid *g) {
    if (!p || (p->ndim != 2 && p->ndim != 3)) return false;
    const int nd = (int)p->ndim;
    MaskGrid r{};
    for (int a = 0; a < 3; ++a) r.ext[a] = r.ker[a] = r.dil[a] = 1;
    int64_t tokens = 1, K = 1;
    for (int a = 0; a < nd; ++a) {
        const int64_t L = p->extent[a], k = p->kernel[a], d = p->dilation[a];
        if (L < 1 || k < 1 || d < 1 || L > INT32_MAX || d > L || k > L / d) return false;
        tokens *= L;
        K *= k;
        if (tokens > INT32_MAX) return false;
        const int dst = a + (3 - nd);
        r.ext[dst] = (int)L;
        r.ker[dst] = (int)k;
        r.dil[dst] = (int)d;
    }
    r.tokens = (int)tokens;
    r.K = (int)K;
    *g = r;
    return true;
}

}  // namespace

extern "C" na_status na_window_mask_from_indices(const na_problem *p, const int64_t *indices,
                                                 int32_t m, uint8_t *mask, int32_t *bad,
                                                 void *hip_stream) {
    MaskGrid g;
    if (!mask_grid(p, &g) || m < 0 || !mask || !bad) return NA_ERR_INVALID_ARG;
    if ((m > 0 && !indices) || (reinterpret_cast<uintptr_t>(indices) & 7u) ||
        (reinterpret_cast<uintptr_t>(bad) & 3u))
        return NA_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    const int64_t nbytes = (int64_t)g.tokens * g.K;
    const int64_t clear_blocks = std::min<int64_t>((nbytes + 16 * kThreads - 1) / (16 * kThreads),
                                                   1 << 16);
    clear_bytes_kernel<<<dim3((unsigned)clear_blocks), dim3(kThreads), 0, st>>>(mask, nbytes);
    if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
    const int64_t blocks = ((int64_t)g.tokens + kThreads - 1) / kThreads;
    mask_from_indices_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(g, indices, m,
                                                                                mask, bad);
    return hipGetLastError() == hipSuccess ? NA_OK : NA_ERR_HIP;
}
