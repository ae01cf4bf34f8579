// na_api.hip -- the C ABI of libna (declared in include/na.h): problem
// validation on the host, workspace sizing, and kernel launches on the
// caller's stream. No allocation, no synchronization, no global state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstdint>
#include <initializer_list>
#include <type_traits>
#include <mutex>

#include "na.h"
#include "na_fast.hpp"
#include "na_host.hpp"
#include "na_kernels.hpp"
#include "na_mfma16.hpp"

namespace {

using na::bf16;
using na::f16;

constexpr int kThreads = 256;  // elementwise kernels

// (token, head) rows the static delta array of na_bwd_noalloc holds: 2^23
// fp32 values, 32 MiB per device.
constexpr int64_t kNoallocRows = NA_NOALLOC_MAX_ROWS;

#ifndef NA_SOURCE_SHA256
#define NA_SOURCE_SHA256 "unknown"
#endif

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Internal 3-axis form (T, H, W) of a validated problem.
struct Prob {
    int ext[3], ker[3], dil[3];
    int64_t batch, heads, head_dim;
    int64_t tokens;  // per batch element
    int64_t rows;    // batch * tokens * heads
    na_dtype dtype;
    float scale;
};

int max_union(const Prob &q, bool inverse, int (&mx)[3]);

na_status validate(const na_problem *p, Prob *out) {
    if (!p) return NA_ERR_INVALID_ARG;
    if (p->ndim != 2 && p->ndim != 3) return NA_ERR_INVALID_ARG;
    if (p->dtype != NA_F32 && p->dtype != NA_BF16 && p->dtype != NA_F16) return NA_ERR_INVALID_ARG;
    if (p->batch < 1 || p->heads < 1 || p->head_dim < 1) return NA_ERR_INVALID_ARG;
    if (!std::isfinite(p->scale)) return NA_ERR_INVALID_ARG;
    const int nd = (int)p->ndim;
    Prob q{};
    for (int a = 0; a < 3; ++a) {
        q.ext[a] = 1;
        q.ker[a] = 1;
        q.dil[a] = 1;
    }
    int64_t tokens = 1;
    for (int a = 0; a < nd; ++a) {
        const int64_t L = p->extent[a], k = p->kernel[a], d = p->dilation[a];
        if (L < 1 || k < 1 || d < 1) return NA_ERR_INVALID_ARG;
        if (L > INT32_MAX || d > L) return NA_ERR_INVALID_ARG;
        // the smallest residue class has floor(L / d) positions; the window must fit it
        if (k > L / d) return NA_ERR_INVALID_ARG;
        tokens *= L;
        if (tokens > INT32_MAX) return NA_ERR_INVALID_ARG;
        const int dst = a + (3 - nd);
        q.ext[dst] = (int)L;
        q.ker[dst] = (int)k;
        q.dil[dst] = (int)d;
    }
    // every offset fits comfortably in int64; keep batch*heads bounded for the wave id
    if (p->batch > INT32_MAX || p->heads > INT32_MAX) return NA_ERR_INVALID_ARG;
    if (p->head_dim != 16 && p->head_dim != 32 && p->head_dim != 64) return NA_ERR_UNSUPPORTED;
    // byte offsets within one row of tokens are 32-bit in the kernels
    const int64_t esize = p->dtype == NA_F32 ? 4 : 2;
    if (p->extent[nd - 1] * p->heads * p->head_dim * esize > INT32_MAX) return NA_ERR_UNSUPPORTED;
    q.batch = p->batch;
    q.heads = p->heads;
    q.head_dim = p->head_dim;
    q.tokens = tokens;
    q.rows = p->batch * tokens * p->heads;
    q.dtype = (na_dtype)p->dtype;
    q.scale = (float)p->scale;
    // the kernels keep per-axis validity masks of 32 bits over a patch walk.
    // The forward walk along an axis spans k + 1 or k + 2 points; the inverse
    // walk of a key near a border is longer (up to 2k points on short axes).
    // Windows up to 16 fit every extent, 17 to 21 all but a few class extents
    // between 33 and 42, and from 22 on only class extents below 33.
    int mx[3];
    if (max_union(q, false, mx) > 32 || max_union(q, true, mx) > 32) return NA_ERR_UNSUPPORTED;
    if (out) *out = q;
    return NA_OK;
}

// Largest box, per axis, that any tile stages: the keys its queries' walks
// read (forward, dq) or the queries its keys' walks read (dk/dv), over all
// tiles and residue classes (the same plan the kernels compute per tile).
// Also returns the longest walk (points along one axis a patch walks); the
// kernels keep per-axis validity masks of that many bits.
int max_union(const Prob &q, bool inverse, int (&mx)[3]) {
    int walk = 1;
    for (int a = 0; a < 3; ++a) {
        mx[a] = 1;
        const int k = q.ker[a], d = q.dil[a], tile = na::kTile[a], p = na::kPatch[a];
        for (int r = 0; r < d && r < q.ext[a]; ++r) {
            const int n = na::class_size(q.ext[a], d, r);
            for (int f = 0; f < n; f += tile) {
                int start, extent;
                if (inverse) {
                    const int cnt = na::tile_inverse_walk(f, tile, p, n, k);
                    na::query_box(f, tile, p, n, k, cnt, &start, &extent);
                    walk = std::max(walk, cnt * p);
                } else {
                    na::key_box(f, tile, p, n, k, &start, &extent);
                    walk = std::max(walk, na::window_walk(k, p) * p);
                }
                mx[a] = std::max(mx[a], extent);
            }
        }
    }
    return walk;
}

// Target LDS bytes for one workgroup's staged chunk: two workgroups per CU.
constexpr int kLdsTarget = 78 * 1024;
constexpr int kLdsTargetWide = 156 * 1024;
constexpr int kLdsMax = 160 * 1024;

// Tiling of the class grids and the LDS plan of one kernel kind; false when
// the problem does not fit (wave count overflow or LDS).
// h_chunks: when one plane along T of a box exceeds the LDS, cut chunks along
// H instead (all planes of a few rows at a time).
bool geometry(const Prob &q, bool inverse, int bytes_per_point, int merge_bytes,
              na::Geometry *g, int *lds_bytes, int target = 0, bool h_chunks = false) {
    int64_t n_tiles = q.batch * q.heads;
    int nres = 1;
    for (int a = 0; a < 3; ++a) {
        g->ext[a] = q.ext[a];
        g->ker[a] = q.ker[a];
        g->dil[a] = q.dil[a];
        const int nmax = na::class_size(q.ext[a], q.dil[a], 0);
        g->tiles[a] = (nmax + na::kTile[a] - 1) / na::kTile[a];
        n_tiles *= g->tiles[a];
        nres *= q.dil[a];
    }
    n_tiles *= nres;
    if (n_tiles > INT32_MAX) return false;
    g->heads = (int)q.heads;
    g->batch = (int)q.batch;
    g->head_dim = (int)q.head_dim;
    g->nres = nres;
    g->n_tiles = (int)n_tiles;
    // chunks of a staged box are cut along the outermost axis that has extent
    g->chunk_axis = q.ext[0] > 1 ? 0 : 1;
    int mx[3];
    if (max_union(q, inverse, mx) > 32) return false;  // 32-bit validity masks
    const int64_t full = (int64_t)mx[0] * mx[1] * mx[2] * bytes_per_point;
    if (h_chunks && g->chunk_axis == 0 && full / mx[0] > kLdsMax) g->chunk_axis = 1;
    const int64_t plane = full / mx[g->chunk_axis];
    // head_dim 64 kernels run one workgroup per CU (kSplitOccupancy): the CU's LDS
    if (target <= 0) target = q.head_dim >= 64 ? kLdsTargetWide : kLdsTarget;
    int64_t lds = std::min<int64_t>(full, target);
    lds = std::max<int64_t>(lds, plane);
    lds = std::max<int64_t>(lds, merge_bytes);
    if (lds > kLdsMax) return false;
    g->lds_budget = (int)lds;
    g->dq_lds_off = 0;
    *lds_bytes = (int)lds;
    return true;
}

// ----------------------------------------------------------------------------
// Register-resident kernels (na_fast.hpp): fp32, head_dim 16 or 32, square
// walks of C x C patches along H and W, one box plane within the LDS share of
// two workgroups per CU.

constexpr int kFastLdsMax = 80 * 1024;

struct FastPlan {
    na::fast::Geom g;
    int lds;
    int c;        // walk length the kernel is compiled for (along H; along W too when square)
    int cw;       // walk length along W
    bool t3;      // more than one plane along T
    bool pad;     // dq, dk/dv: padded points, one staging per tensor serves both read patterns
    int walk_lo;  // dk/dv: the launch takes tiles whose inverse walk lies in (walk_lo, c]
};

// Compiled walk lengths: 2 .. 5 patches per axis on single-plane grids, 2 .. 4
// with several planes along T (the per-lane rows and accumulators stay live
// across the plane loop there).
bool fast_walk_compiled(int c, bool t3) { return c >= 2 && c <= (t3 ? 4 : 5); }

// Border-only dk/dv kernels for longer walks, one workgroup per CU (head_dim
// 32; walks 6 and 7 on single-plane grids, 6 with the padded layout on grids
// with several planes): the whole LDS and register file of a CU.
constexpr int kBorderLdsMax = 160 * 1024;
bool border_walk_compiled(int c, bool t3, int head_dim) {
    return head_dim == 32 && (t3 ? c == 6 : (c == 6 || c == 7));
}

// dk/dv walks of ch x cw patches with ch != cw, for the border tiles that need
// the longer walk along one axis only: single-plane grids (one workgroup per
// CU, head_dim 32, fp32 and fp16) for windows of 7 and 9; grids with several
// planes (head_dim 32) for a window of 5 (fp32, two workgroups per CU) and of
// 7 (every type, one workgroup per CU, padded layout).
bool rect_walk_compiled(int ch, int cw, bool t3, int head_dim, int dtype) {
    if (head_dim != 32) return false;
    if (!t3)
        return (dtype == NA_F32 || dtype == NA_F16) &&
               ((ch == 7 && cw == 5) || (ch == 5 && cw == 7) || (ch == 6 && cw == 4) ||
                (ch == 4 && cw == 6));
    return (dtype == NA_F32 && ((ch == 4 && cw == 3) || (ch == 3 && cw == 4))) ||
           (ch == 6 && cw == 4) || (ch == 4 && cw == 6);
}

// Longest inverse walk (patches) along one axis (1: H, 2: W) of any 16-point
// tile of any residue class.
int max_axis_walk(const Prob &q, int a) {
    int m = 0;
    for (int r = 0; r < q.dil[a] && r < q.ext[a]; ++r) {
        const int n = na::class_size(q.ext[a], q.dil[a], r);
        for (int f = 0; f < n; f += 16) m = std::max(m, na::tile_inverse_walk(f, 16, 2, n, q.ker[a]));
    }
    return m;
}

// Longest inverse walk (patches) of any 16 x 16 tile of any residue class.
int max_tile_walk(const Prob &q) {
    int m = 0;
    for (int a = 1; a < 3; ++a)
        for (int r = 0; r < q.dil[a] && r < q.ext[a]; ++r) {
            const int n = na::class_size(q.ext[a], q.dil[a], r);
            for (int f = 0; f < n; f += 16)
                m = std::max(m, na::tile_inverse_walk(f, 16, 2, n, q.ker[a]));
        }
    return m;
}

// The 16 x 16 tiles whose inverse walk exceeds `done`, as border rows and
// columns (na::Border); false when they are not such a frame (dilation > 1
// has several residue classes of different sizes: launches then cover every
// tile and the others exit early).
bool border_of(const Prob &q, int done, na::Border *bd) {
    for (int a = 0; a < 3; ++a)
        if (q.dil[a] != 1) return false;
    int lo[3] = {0, 0, 0}, hi[3] = {0, 0, 0};
    for (int a = 1; a < 3; ++a) {
        const int n = q.ext[a], T = (n + 15) / 16;
        auto big = [&](int t) { return na::tile_inverse_walk(16 * t, 16, 2, n, q.ker[a]) > done; };
        while (lo[a] < T && big(lo[a])) ++lo[a];
        while (hi[a] < T - lo[a] && big(T - 1 - hi[a])) ++hi[a];
        for (int t = lo[a]; t < T - hi[a]; ++t)
            if (big(t)) return false;
    }
    const int R = (q.ext[1] + 15) / 16, C = (q.ext[2] + 15) / 16;
    bd->on = 1;
    bd->cls = 0;
    bd->rows_lo = lo[1];
    bd->rows_hi = hi[1];
    bd->cols_lo = lo[2];
    bd->cols_hi = hi[2];
    const int rb = lo[1] + hi[1], cb = lo[2] + hi[2];
    bd->per_plane = rb * C + (R - rb) * cb;
    return true;
}

// Divisors of the fast tile decode (na::fast::decode), from the geometry and
// the border set; call again after changing either.
void set_divisors(na::fast::Geom &g) {
    const int band = na::fast::kFastBand, last = g.tiles[2] % band;
    g.f_heads = na::make_fastdiv(g.heads);
    g.f_t = na::make_fastdiv(g.tiles[0]);
    g.f_plane = na::make_fastdiv(g.border.on ? g.border.per_plane : g.tiles[1] * g.tiles[2]);
    g.f_bandrows = na::make_fastdiv(band * g.tiles[1]);
    g.f_band = na::make_fastdiv(band);
    g.f_lastband = na::make_fastdiv(last ? last : band);
    g.f_nres = na::make_fastdiv(g.nres);
    const int cb = g.border.cols_lo + g.border.cols_hi;
    g.f_c = na::make_fastdiv(!g.border.on || g.border.cls == 0 ? g.tiles[2]
                             : (g.border.cls & 2)               ? std::max(1, cb)
                                                                : std::max(1, g.tiles[2] - cb));
    g.f_cb = na::make_fastdiv(std::max(1, g.border.cols_lo + g.border.cols_hi));
    for (int a = 0; a < 3; ++a) g.f_dil[a] = na::make_fastdiv(g.dil[a]);
    g.f_dil21 = na::make_fastdiv(g.dil[2] * g.dil[1]);
}

// kind 0: forward / dq (walk c = the window walk, exact);
// kind 1: dk/dv over the tiles whose inverse walk lies in (walk_lo, c], or
// with cw > 0 a walk of c patches along H and cw along W (border classes).
// pad: points one 16-byte slot apart (see dq_tile), for grids with several
// planes along T, whose plane boxes leave room for it.
// edge >= 0: the box only over the tiles of that border class (inverse walk
// along H above walk_lo exactly when bit 0 is set, along W when bit 1 is).
bool fast_plan(const Prob &q, int kind, int c, int walk_lo, FastPlan *pl, bool pad = false,
               int cw = 0, int edge = -1, bool one_layout = false) {
    // fp32 with head_dim 16 or 32; bf16 / fp16 (converted to fp32 while staged)
    // with head_dim 32
    if (q.dtype == NA_F32) {
        if (q.head_dim != 16 && q.head_dim != 32) return false;
    } else if (q.head_dim != 32) {
        return false;
    }
    const bool t3 = q.ext[0] > 1;
    if (cw <= 0) cw = c;
    bool wide;
    if (cw == c) {
        wide = kind == 1 && border_walk_compiled(c, t3, (int)q.head_dim);
        if (!fast_walk_compiled(c, t3) && !wide) return false;
    } else {
        if (kind != 1 || !rect_walk_compiled(c, cw, t3, (int)q.head_dim, q.dtype)) return false;
        wide = !t3 || std::max(c, cw) > 4;
    }
    if (pad && !t3) return false;
    if (wide && t3 && !pad) return false;  // the border kernels of such grids are padded
    const int PB = (int)q.head_dim * 4 + (pad ? 16 : 0);
    // largest plane box per axis over the tiles this launch runs
    int mx[3] = {1, 1, 1};
    for (int a = 1; a < 3; ++a)
        for (int r = 0; r < q.dil[a] && r < q.ext[a]; ++r) {
            const int n = na::class_size(q.ext[a], q.dil[a], r);
            for (int f = 0; f < n; f += 16) {
                int start, extent;
                if (kind == 0) {
                    na::key_box(f, 16, 2, n, q.ker[a], &start, &extent);
                } else {
                    const int ca = a == 1 ? c : cw;
                    const int wt = na::tile_inverse_walk(f, 16, 2, n, q.ker[a]);
                    if (wt > ca) continue;
                    if (edge >= 0 && (wt > walk_lo) != (((edge >> (a - 1)) & 1) != 0)) continue;
                    na::query_box(f, 16, 2, n, q.ker[a], ca, &start, &extent);
                }
                mx[a] = std::max(mx[a], extent);
            }
        }
    // row pitches: an odd number of 16-byte slots (A), 2 mod 4 slots (B; both
    // patterns when padded)
    const int slots = mx[2] * PB / 16;
    // one_layout (the backward's unpadded plans): both read patterns from the
    // A pitch, so a tensor the backward reads both ways is staged once (its
    // d-major reads then take bank conflicts; measured faster than a restaging)
    const int ra = pad ? (slots + ((2 - slots % 4) + 4) % 4) * 16 : (slots | 1) * 16;
    const int rb = pad || one_layout ? ra : (slots + ((2 - slots % 4) + 4) % 4) * 16;
    int64_t lds = (int64_t)mx[1] * std::max(ra, rb);
    na::fast::Geom &g = pl->g;
    g = na::fast::Geom{};
    g.rows_off = (int)lds;
    g.rows_pitch = mx[2];
    if (kind == 1) lds += (int64_t)mx[1] * mx[2] * 8;
    if (lds > (wide ? kBorderLdsMax : kFastLdsMax)) return false;
    int64_t n_tiles = q.batch * q.heads;
    int nres = 1;
    for (int a = 0; a < 3; ++a) {
        g.ext[a] = q.ext[a];
        g.ker[a] = q.ker[a];
        g.dil[a] = q.dil[a];
        const int nmax = na::class_size(q.ext[a], q.dil[a], 0);
        g.tiles[a] = a == 0 ? nmax : (nmax + 15) / 16;
        n_tiles *= g.tiles[a];
        nres *= q.dil[a];
    }
    n_tiles *= nres;
    if (n_tiles > INT32_MAX) return false;
    g.heads = (int)q.heads;
    g.batch = (int)q.batch;
    g.head_dim = (int)q.head_dim;
    g.nres = nres;
    g.n_tiles = (int)n_tiles;
    g.ra = ra;
    g.rb = rb;
    set_divisors(g);
    pl->lds = (int)lds;
    pl->c = c;
    pl->cw = cw;
    pl->t3 = t3;
    pl->pad = pad;
    pl->walk_lo = walk_lo;
    return true;
}

// Forward / dq: the register-resident kernels need a square walk. dq takes
// the padded layout where it fits.
bool fast_plan_fwd(const Prob &q, FastPlan *pl, bool try_pad = false) {
    const int c = na::window_walk(q.ker[1], 2);
    if (na::window_walk(q.ker[2], 2) != c) return false;
    return (try_pad && fast_plan(q, 0, c, 0, pl, true)) ||
           fast_plan(q, 0, c, 0, pl, false, 0, -1, try_pad);
}

template <typename Kern, typename Args>
na_status launch_fast(Kern kern, const FastPlan &pl, const Args &a, hipStream_t s) {
    if (!na_host::lds_limit_once((const void *)kern)) return NA_ERR_HIP;
    if (a.g.n_tiles == 0) return NA_OK;
    hipLaunchKernelGGL(kern, dim3(a.g.n_tiles), dim3(na::kThreads), pl.lds, s, a);
    return hipGetLastError() == hipSuccess ? NA_OK : NA_ERR_HIP;
}

// The compiled (head_dim, walk, several planes) combinations: fp32 below;
// the 16-bit types take the head_dim 32 ones.
#define NA_FAST_CASES(X)                                                                  \
    X(16, 2, false) X(16, 3, false) X(16, 4, false) X(16, 5, false)                      \
    X(32, 2, false) X(32, 3, false) X(32, 4, false) X(32, 5, false)                      \
    X(16, 2, true) X(16, 3, true) X(16, 4, true)                                         \
    X(32, 2, true) X(32, 3, true) X(32, 4, true)
#define NA_FAST_CASES16(X)                                                                \
    X(32, 2, false) X(32, 3, false) X(32, 4, false) X(32, 5, false)                      \
    X(32, 2, true) X(32, 3, true) X(32, 4, true)

// Window masks (a.mask) run on the register-resident kernels when the mask
// is 4-byte aligned (the forward and dq read it in aligned dwords), 16-bit
// tensors included (converted to fp32 while staged, as without a mask); the
// dk/dv walks that have no masked instantiation (fast_dkdv_masked) take the
// split kernels.
bool fast_mask_ok(const uint8_t *mask) { return (reinterpret_cast<uintptr_t>(mask) & 3u) == 0; }

template <typename T>
na_status fast_fwd(const FastPlan &pl, const na::fast::FwdArgsT<T> &a, hipStream_t s) {
    if (a.mask) {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return launch_fast(na::fast::fwd_kernel<T, D, C, C, T3, true>, pl, a, s);
        if constexpr (std::is_same<T, float>::value) {
            NA_FAST_CASES(X)
        } else {
            NA_FAST_CASES16(X)
        }
#undef X
        return NA_ERR_UNSUPPORTED;
    }
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return launch_fast(na::fast::fwd_kernel<T, D, C, C, T3>, pl, a, s);
    if constexpr (std::is_same<T, float>::value) {
        NA_FAST_CASES(X)
    } else {
        NA_FAST_CASES16(X)
    }
#undef X
    return NA_ERR_UNSUPPORTED;
}

template <typename T>
na_status fast_dq(const FastPlan &pl, const na::fast::BwdArgsT<T> &a, hipStream_t s) {
    if (a.mask) {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return pl.pad ? launch_fast(na::fast::dq_kernel<T, D, C, C, T3, T3, true>, pl, a, s) \
                      : launch_fast(na::fast::dq_kernel<T, D, C, C, T3, false, true>, pl, a, s);
        if constexpr (std::is_same<T, float>::value) {
            NA_FAST_CASES(X)
        } else {
            NA_FAST_CASES16(X)
        }
#undef X
        return NA_ERR_UNSUPPORTED;
    }
    if constexpr (std::is_same<T, float>::value) {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return pl.pad ? launch_fast(na::fast::dq_kernel<T, D, C, C, T3, T3>, pl, a, s)    \
                      : launch_fast(na::fast::dq_kernel<T, D, C, C, T3, false>, pl, a, s);
        NA_FAST_CASES(X)
#undef X
    } else {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return pl.pad ? launch_fast(na::fast::dq_kernel<T, D, C, C, T3, T3>, pl, a, s)    \
                      : launch_fast(na::fast::dq_kernel<T, D, C, C, T3, false>, pl, a, s);
        NA_FAST_CASES16(X)
#undef X
    }
    return NA_ERR_UNSUPPORTED;
}

// The masked dk/dv instantiations: the interior square walks at two
// workgroups per CU up to 5 patches on one plane and 3 on several (the walk of
// 4 spilled there); at head_dim 32 the longer walks of the border classes at
// one workgroup per CU: 7 x 5, 5 x 7, 6 x 4, 4 x 6, 6 x 6, 7 x 7 on one plane,
// 4 x 3, 3 x 4, 4 x 4 and (padded) 6 x 4, 4 x 6, 6 x 6 on several. The 16-bit
// types take the head_dim 32 ones.
#define NA_FAST_CASES_MASKED_DKDV(X)                                                      \
    X(16, 2, false) X(16, 3, false) X(16, 4, false) X(16, 5, false)                      \
    X(32, 2, false) X(32, 3, false) X(32, 4, false) X(32, 5, false)                      \
    X(16, 2, true) X(16, 3, true) X(32, 2, true) X(32, 3, true)
#define NA_FAST_CASES16_MASKED_DKDV(X)                                                    \
    X(32, 2, false) X(32, 3, false) X(32, 4, false) X(32, 5, false)                      \
    X(32, 2, true) X(32, 3, true)
bool fast_dkdv_masked(const FastPlan &pl) {
    const int ch = pl.c, cw = pl.cw;
    if (ch == cw && ch >= 2 && ch <= (pl.t3 ? 3 : 5))
        return pl.g.head_dim == 16 || pl.g.head_dim == 32;
    if (pl.g.head_dim != 32) return false;
    auto is = [&](int a, int b) { return ch == a && cw == b; };
    if (!pl.t3) return is(7, 5) || is(5, 7) || is(6, 4) || is(4, 6) || is(6, 6) || is(7, 7);
    return is(4, 3) || is(3, 4) || is(4, 4) ||
           (pl.pad && (is(6, 4) || is(4, 6) || is(6, 6)));
}

template <typename T>
na_status fast_dkdv(const FastPlan &pl, const na::fast::BwdArgsT<T> &a, hipStream_t s) {
    if (a.mask) {
        if (!fast_dkdv_masked(pl)) return NA_ERR_UNSUPPORTED;
        if (pl.cw == pl.c && pl.c <= (pl.t3 ? 3 : 5)) {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                               \
        return pl.pad ? launch_fast(na::fast::dkdv_kernel<T, D, C, C, T3, T3, true>, pl, a, s) \
                      : launch_fast(na::fast::dkdv_kernel<T, D, C, C, T3, false, true>, pl, a, s);
            if constexpr (std::is_same<T, float>::value) {
                NA_FAST_CASES_MASKED_DKDV(X)
            } else {
                NA_FAST_CASES16_MASKED_DKDV(X)
            }
#undef X
            return NA_ERR_UNSUPPORTED;
        }
#define X(CH, CW)                                                                        \
    if (pl.c == CH && pl.cw == CW && !pl.t3)                                         \
        return launch_fast(na::fast::dkdv_border_kernel<T, 32, CH, CW, false, false, true>, pl, a, s);
        X(7, 5) X(5, 7) X(6, 4) X(4, 6) X(6, 6) X(7, 7)
#undef X
#define X(CH, CW)                                                                        \
    if (pl.c == CH && pl.cw == CW && pl.t3)                                          \
        return pl.pad                                                                \
                   ? launch_fast(na::fast::dkdv_border_kernel<T, 32, CH, CW, true, true, true>, pl, a, s) \
                   : launch_fast(na::fast::dkdv_border_kernel<T, 32, CH, CW, true, false, true>, pl, a, s);
        X(4, 3) X(3, 4) X(4, 4)
#undef X
#define X(CH, CW)                                                                        \
    if (pl.c == CH && pl.cw == CW && pl.t3 && pl.pad)                                \
        return launch_fast(na::fast::dkdv_border_kernel<T, 32, CH, CW, true, true, true>, pl, a, s);
        X(6, 4) X(4, 6) X(6, 6)
#undef X
        return NA_ERR_UNSUPPORTED;
    }
    if (pl.cw != pl.c) {
        // border classes with a longer walk along one axis (rect_walk_compiled)
        if constexpr (!std::is_same<T, bf16>::value) {
#define X(CH, CW)                                                                        \
    if (a.g.head_dim == 32 && pl.c == CH && pl.cw == CW && !pl.t3)                       \
        return launch_fast(na::fast::dkdv_border_kernel<T, 32, CH, CW, false, false>, pl, a, s);
            X(7, 5) X(5, 7) X(6, 4) X(4, 6)
#undef X
        }
#define X(CH, CW)                                                                        \
    if (a.g.head_dim == 32 && pl.c == CH && pl.cw == CW && pl.t3 && pl.pad)              \
        return launch_fast(na::fast::dkdv_border_kernel<T, 32, CH, CW, true, true>, pl, a, s);
        X(6, 4) X(4, 6)
#undef X
        if constexpr (std::is_same<T, float>::value) {
#define X(CH, CW)                                                                        \
    if (a.g.head_dim == 32 && pl.c == CH && pl.cw == CW && pl.t3)                        \
        return pl.pad ? launch_fast(na::fast::dkdv_kernel<T, 32, CH, CW, true, true>, pl, a, s) \
                      : launch_fast(na::fast::dkdv_kernel<T, 32, CH, CW, true, false>, pl, a, s);
            X(4, 3) X(3, 4)
#undef X
        }
        return NA_ERR_UNSUPPORTED;
    }
    if constexpr (std::is_same<T, float>::value) {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return pl.pad ? launch_fast(na::fast::dkdv_kernel<T, D, C, C, T3, T3>, pl, a, s)  \
                      : launch_fast(na::fast::dkdv_kernel<T, D, C, C, T3, false>, pl, a, s);
        NA_FAST_CASES(X)
#undef X
    } else {
#define X(D, C, T3)                                                                       \
    if (a.g.head_dim == D && pl.c == C && pl.t3 == T3)                                   \
        return pl.pad ? launch_fast(na::fast::dkdv_kernel<T, D, C, C, T3, T3>, pl, a, s)  \
                      : launch_fast(na::fast::dkdv_kernel<T, D, C, C, T3, false>, pl, a, s);
        NA_FAST_CASES16(X)
#undef X
    }
#define X(D, C)                                                                          \
    if (a.g.head_dim == D && pl.c == C && !pl.t3)                                        \
        return launch_fast(na::fast::dkdv_border_kernel<T, D, C, C, false, false>, pl, a, s);
    X(32, 6) X(32, 7)
#undef X
    if (a.g.head_dim == 32 && pl.c == 6 && pl.t3 && pl.pad)
        return launch_fast(na::fast::dkdv_border_kernel<T, 32, 6, 6, true, true>, pl, a, s);
    return NA_ERR_UNSUPPORTED;
}

// ----------------------------------------------------------------------------
// 16-bit MFMA kernels (na_mfma16.hpp): bf16 and fp16 tensors with head_dim 32
// or 64. kind 0: forward, 1: dq, 2: dk/dv.

struct M16Plan {
    na::m16::Geom g;
    int lds;
};


// Columns a slab row must hold: the end of the last block any wave of any
// tile (4 << pcsh columns wide) walks, relative to its tile's box start (the
// same formulas the kernels evaluate), rounded to groups of four.
int m16_box_w(const Prob &q, bool inverse, int pcsh) {
    int bw = 4;
    const int k = q.ker[2], tw = 4 << pcsh;
    for (int r = 0; r < q.dil[2] && r < q.ext[2]; ++r) {
        const int n = na::class_size(q.ext[2], q.dil[2], r);
        for (int w0 = 0; w0 < n; w0 += tw) {
            const int U2 = inverse ? na::inverse_first(w0, n, k) : na::window_start(w0, n, k);
            for (int j = 0; j < (1 << pcsh) && w0 + 4 * j < n; ++j) {
                const int p0 = w0 + 4 * j, p1 = std::min(p0 + 3, n - 1);
                const int s0 = inverse ? na::inverse_first(p0, n, k) : na::window_start(p0, n, k);
                const int e1 = inverse ? na::inverse_last(p1, n, k) + 1
                                       : na::window_start(p1, n, k) + k;
                const int aw = (s0 - U2) & ~3;
                const int nbw = (e1 - U2 - aw + 3) >> 2;
                bw = std::max(bw, aw + 4 * nbw);
            }
        }
    }
    return bw;
}

// Sum over the tiles of one axis (tile extent te over the largest residue
// class) of the positions the tile's window union spans: planes (T) or
// 4-row slabs (H).
int64_t m16_union_sum(int n, int k, int te, bool inverse, bool slabs) {
    int64_t sum = 0;
    for (int o = 0; o < n; o += te) {
        const int l = std::min(o + te - 1, n - 1);
        const int a = inverse ? na::inverse_first(o, n, k) : na::window_start(o, n, k);
        const int b = inverse ? na::inverse_last(l, n, k) + 1 : na::window_start(l, n, k) + k;
        sum += slabs ? (b - a + 3) / 4 : b - a;
    }
    return sum;
}

// Tile shape of a 16-bit launch. The workgroup stages, per slab step, four rows
// of box_w points of one plane, and walks them; over the grid that is
// (T unions) x (H slabs) x (W tiles) steps. The shape taken is the one with the
// fewest staged points, each step counted with a fixed cost of kStepPoints
// points for its barrier and set-up. Several planes per tile only pay where a
// key plane serves several query planes (a window longer than one plane).
constexpr int kStepPoints = 16;
struct M16Shape {
    int tp, prsh, pcsh, box_w;
};
M16Shape m16_shape(const Prob &q, bool inverse) {
    static const int cand[][3] = {{1, 1, 2}, {2, 1, 1}, {2, 0, 2}, {4, 0, 1}};
    const int n0 = na::class_size(q.ext[0], q.dil[0], 0);
    const int n1 = na::class_size(q.ext[1], q.dil[1], 0);
    const int n2 = na::class_size(q.ext[2], q.dil[2], 0);
    M16Shape best{0, 0, 0, 0};
    double best_cost = 0.0;
    for (const auto &c : cand) {
        if (c[0] > 1 && (q.ker[0] == 1 || n0 == 1)) continue;
        const int bw = m16_box_w(q, inverse, c[2]);
        if (bw > 48) continue;
        const double steps = (double)m16_union_sum(n0, q.ker[0], c[0], inverse, false) *
                             (double)m16_union_sum(n1, q.ker[1], 4 << c[1], inverse, true) *
                             (double)((n2 + (4 << c[2]) - 1) / (4 << c[2]));
        const double cost = steps * (kStepPoints + bw);
        if (best.tp == 0 || cost < best_cost) {
            best = M16Shape{c[0], c[1], c[2], bw};
            best_cost = cost;
        }
    }
    return best;
}

bool m16_plan(const Prob &q, int kind, M16Plan *pl) {
    if (q.dtype != NA_BF16 && q.dtype != NA_F16) return false;
    if (q.head_dim != 32 && q.head_dim != 64) return false;
    const M16Shape sh = m16_shape(q, kind == 2);
    if (sh.tp == 0) return false;
    na::m16::Geom &g = pl->g;
    g = na::m16::Geom{};
    g.tp = sh.tp;
    g.prsh = sh.prsh;
    g.pcsh = sh.pcsh;
    int64_t n_tiles = q.batch * q.heads;
    int nres = 1;
    for (int a = 0; a < 3; ++a) {
        g.ext[a] = q.ext[a];
        g.ker[a] = q.ker[a];
        g.dil[a] = q.dil[a];
        const int nmax = na::class_size(q.ext[a], q.dil[a], 0);
        const int t = a == 0 ? sh.tp : a == 1 ? 4 << sh.prsh : 4 << sh.pcsh;
        g.tiles[a] = (nmax + t - 1) / t;
        n_tiles *= g.tiles[a];
        nres *= q.dil[a];
    }
    n_tiles *= nres;
    if (n_tiles > INT32_MAX) return false;
    g.heads = (int)q.heads;
    g.batch = (int)q.batch;
    g.nres = nres;
    g.n_tiles = (int)n_tiles;
    g.box_w = sh.box_w;
    // the kernels are compiled for slab rows of up to 24, 32 or 48 points
    // (static LDS: two buffers of two slabs each)
    g.wmax = g.box_w <= 24 ? 24 : g.box_w <= 32 ? 32 : 48;
    if (g.box_w > g.wmax) return false;
    pl->lds = 0;
    g.f_heads = na::make_fastdiv(g.heads);
    g.f_tw = na::make_fastdiv(g.tiles[2]);
    g.f_th = na::make_fastdiv(g.tiles[1]);
    g.f_t = na::make_fastdiv(g.tiles[0]);
    g.f_nres = na::make_fastdiv(g.nres);
    for (int a = 0; a < 3; ++a) g.f_dil[a] = na::make_fastdiv(g.dil[a]);
    g.f_dil21 = na::make_fastdiv(g.dil[2] * g.dil[1]);
    return true;
}

// kind 0: forward, 1: dq, 2: dk/dv (the kernels are built in na_m16.hip)
template <typename T, int D>
na_status launch_m16(int kind, const M16Plan &, const na::m16::Args<T> &a, hipStream_t s) {
    return na::m16::launch<T, D>(kind, a, s) == hipSuccess ? NA_OK : NA_ERR_HIP;
}

dim3 flat_grid(int64_t n) { return dim3((unsigned)((n + kThreads - 1) / kThreads)); }

na_status launched() { return hipGetLastError() == hipSuccess ? NA_OK : NA_ERR_HIP; }

template <typename T, int D>
na_status run_fwd(const Prob &pr, na::FwdArgs a, hipStream_t s) {
    constexpr int PB = D * (int)sizeof(T);
    if constexpr (!std::is_same<T, float>::value && (D == 32 || D == 64)) {
        M16Plan mp;
        if (!a.mask && m16_plan(pr, 0, &mp)) {
            na::m16::Args<T> ma{};
            ma.g = mp.g;
            ma.q = static_cast<const T *>(a.q);
            ma.k = static_cast<const T *>(a.k);
            ma.v = static_cast<const T *>(a.v);
            ma.o = static_cast<T *>(a.out);
            ma.lse_out = a.lse;
            ma.qscale = a.qscale;
            ma.frame = a.frame;
            ma.frame_axis = a.frame_axis;
            return launch_m16<T, D>(0, mp, ma, s);
        }
    }
    FastPlan pl;
    // window masks: the register-resident kernels, else the split kernels
    if ((!a.mask || fast_mask_ok(a.mask)) && fast_plan_fwd(pr, &pl)) {
        na::fast::FwdArgsT<T> fa{};
        fa.g = pl.g;
        fa.q = static_cast<const T *>(a.q);
        fa.k = static_cast<const T *>(a.k);
        fa.v = static_cast<const T *>(a.v);
        fa.out = static_cast<T *>(a.out);
        fa.lse = a.lse;
        fa.qscale = a.qscale;
        fa.frame = a.frame;
        fa.frame_axis = a.frame_axis;
        fa.mask = a.mask;
        fa.mask_k = a.mask_k;
        fa.mask_bytes = pr.tokens * a.mask_k;
        return fast_fwd<T>(pl, fa, s);
    }
    int lds;
    if (!geometry(pr, false, 2 * PB, na::kWaves * 64 * (D + 3) * 4, &a.g, &lds))
        return NA_ERR_UNSUPPORTED;
    auto kern = na::fwd_kernel<T, D>;
    if (!na_host::lds_limit_once((const void *)kern)) return NA_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3(a.g.n_tiles), dim3(na::kThreads), lds, s, a);
    return launched();
}

// Which kernels of the backward a call runs.
enum Phase { kPhaseDq = 1, kPhaseDkdv = 2, kPhaseBoth = 3 };

// Tile classes of the deterministic KV-parallel backward: per axis the
// smallest m such that any two tiles m (or more) apart along it have disjoint
// query boxes (box starts do not decrease along an axis, so checking tiles
// exactly m apart suffices). A tile's class is its tile index modulo m per
// axis; tiles of one class never add into the same element.
int kv_classes(const Prob &q, int (&m)[3]) {
    for (int a = 0; a < 3; ++a) {
        const int tile = na::kTile[a], p = na::kPatch[a], k = q.ker[a];
        auto box = [&](int n, int t, int *st, int *en) {
            const int f = t * tile;
            const int cnt = na::tile_inverse_walk(f, tile, p, n, k);
            int ex;
            na::query_box(f, tile, p, n, k, cnt, st, &ex);
            *en = *st + ex;
        };
        m[a] = 1;
        for (int r = 0; r < q.dil[a] && r < q.ext[a]; ++r) {
            const int n = na::class_size(q.ext[a], q.dil[a], r), T = (n + tile - 1) / tile;
            for (bool again = true; again;) {
                again = false;
                for (int t = 0; t + m[a] < T && !again; ++t) {
                    int s0, e0, s1, e1;
                    box(n, t, &s0, &e0);
                    box(n, t + m[a], &s1, &e1);
                    if (s1 < e0) {
                        ++m[a];
                        again = true;
                    }
                }
            }
        }
    }
    return m[0] * m[1] * m[2];
}

template <typename T, int D>
na_status run_bwd(const Prob &pr, na::BwdArgs a, int32_t variant, int32_t kv_splits, int phases,
                  hipStream_t s) {
    constexpr int PB = D * (int)sizeof(T);
    na::BwdArgs aq = a, ak = a;
    int lds_q = 0, lds_k = 0;
    if (!geometry(pr, false, 2 * PB, na::kWaves * 64 * (D + 1) * 4, &aq.g, &lds_q)) return NA_ERR_UNSUPPORTED;
    if (!geometry(pr, true, 2 * PB + 8, na::kWaves * 64 * (D + 1) * 4, &ak.g, &lds_k)) return NA_ERR_UNSUPPORTED;
    if constexpr (!std::is_same<T, float>::value && (D == 32 || D == 64)) {
        M16Plan mq, mk;
        if (variant == NA_BWD_GATHER && !a.mask && m16_plan(pr, 1, &mq) && m16_plan(pr, 2, &mk)) {
            na::m16::Args<T> ma{};
            ma.q = static_cast<const T *>(a.q);
            ma.k = static_cast<const T *>(a.k);
            ma.v = static_cast<const T *>(a.v);
            ma.out = static_cast<const T *>(a.out);
            ma.dout = static_cast<const T *>(a.dout);
            ma.lse = a.lse;
            ma.delta = a.delta;
            ma.dq = static_cast<T *>(a.dq);
            ma.dk = static_cast<T *>(a.dk);
            ma.dv = static_cast<T *>(a.dv);
            ma.qscale = a.qscale;
            ma.scale = a.scale;
            ma.frame = a.frame;
            ma.frame_axis = a.frame_axis;
            // dq (which also writes delta) strictly before dk/dv, which reads it
            if (phases & kPhaseDq) {
                ma.g = mq.g;
                const na_status st = launch_m16<T, D>(1, mq, ma, s);
                if (st != NA_OK) return st;
            }
            if (phases & kPhaseDkdv) {
                ma.g = mk.g;
                return launch_m16<T, D>(2, mk, ma, s);
            }
            return NA_OK;
        }
    }
    if (variant == NA_BWD_GATHER) {
        na::fast::BwdArgsT<T> fa{};
        fa.q = static_cast<const T *>(a.q);
        fa.k = static_cast<const T *>(a.k);
        fa.v = static_cast<const T *>(a.v);
        fa.out = static_cast<const T *>(a.out);
        fa.dout = static_cast<const T *>(a.dout);
        fa.lse = a.lse;
        fa.delta = a.delta;
        fa.dq = static_cast<T *>(a.dq);
        fa.dk = static_cast<T *>(a.dk);
        fa.dv = static_cast<T *>(a.dv);
        fa.qscale = a.qscale;
        fa.scale = a.scale;
        fa.frame = a.frame;
        fa.frame_axis = a.frame_axis;
        fa.edge = -1;  // dk/dv tiles by walk_lo (border classes set it per launch)
        // dq (which also writes delta) strictly before dk/dv, which reads it
        FastPlan pq, pk;
        fa.mask = a.mask;
        fa.mask_k = a.mask_k;
        fa.mask_bytes = pr.tokens * a.mask_k;
        const bool mask_fast = !a.mask || fast_mask_ok(a.mask);
        if (phases & kPhaseDq) {
            if (mask_fast && fast_plan_fwd(pr, &pq, true)) {
                fa.g = pq.g;
                const na_status st = fast_dq<T>(pq, fa, s);
                if (st != NA_OK) return st;
            } else {
                auto kern = na::dq_kernel<T, D>;
                if (!na_host::lds_limit_once((const void *)kern)) return NA_ERR_HIP;
                hipLaunchKernelGGL(kern, dim3(aq.g.n_tiles), dim3(na::kThreads), lds_q, s, aq);
                if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
            }
        }
        if (phases & kPhaseDkdv) {
            // the interior walk c (the window walk) over every tile, then the
            // shortest compiled longer walk over the border tiles that need
            // more; the split kernel takes whatever is left
            const int need = max_tile_walk(pr);
            const int c = std::max(na::window_walk(pr.ker[1], 2), na::window_walk(pr.ker[2], 2));
            int done = 0;  // tiles with inverse walk <= done are covered
            // with a window mask: the walks compiled with it (fast_dkdv_masked);
            // the split kernel takes the rest
            if (mask_fast &&
                (fast_plan(pr, 1, c, 0, &pk, true) ||
                 fast_plan(pr, 1, c, 0, &pk, false, 0, -1, true)) &&
                (!a.mask || fast_dkdv_masked(pk))) {
                fa.g = pk.g;
                fa.walk_lo = 0;
                const na_status st = fast_dkdv<T>(pk, fa, s);
                if (st != NA_OK) return st;
                done = c;
            }
            // border tiles by class: a longer walk along H only, along W only,
            // or along both (corners), each with the walk it needs, when all
            // the classes that occur have a compiled kernel
            if (done > 0 && done < need) {
                const int hm = max_axis_walk(pr, 1), wm = max_axis_walk(pr, 2);
                FastPlan cls[4];
                bool use[4] = {false, false, false, false}, all = true;
                for (int e = 1; e <= 3; ++e) {
                    if (((e & 1) && hm <= done) || ((e & 2) && wm <= done)) continue;  // no such tile
                    const int ch = (e & 1) ? hm : done, cw = (e & 2) ? wm : done;
                    use[e] = (fast_plan(pr, 1, ch, done, &cls[e], true, cw, e) ||
                              fast_plan(pr, 1, ch, done, &cls[e], false, cw, e, true)) &&
                             (!a.mask || fast_dkdv_masked(cls[e]));
                    all = all && use[e];
                }
                if (all) {
                    for (int e = 1; e <= 3; ++e) {
                        if (!use[e]) continue;
                        fa.g = cls[e].g;
                        fa.edge = e;
                        fa.walk_c = done;
                        na::Border &bd = fa.g.border;
                        if (border_of(pr, done, &bd)) {
                            // this class's tiles only, so every workgroup has work
                            const int rb = bd.rows_lo + bd.rows_hi, cb = bd.cols_lo + bd.cols_hi;
                            bd.cls = e;
                            bd.per_plane = ((e & 1) ? rb : fa.g.tiles[1] - rb) *
                                           ((e & 2) ? cb : fa.g.tiles[2] - cb);
                            fa.g.n_tiles =
                                (int)(pr.batch * pr.heads * fa.g.tiles[0] * bd.per_plane);
                            set_divisors(fa.g);
                        }
                        const na_status st = fast_dkdv<T>(cls[e], fa, s);
                        if (st != NA_OK) return st;
                    }
                    fa.edge = -1;
                    done = need;
                }
            }
            for (int cb = c + 1; done > 0 && done < need && cb <= need; ++cb) {
                if (!fast_plan(pr, 1, cb, done, &pk, true) &&
                    !fast_plan(pr, 1, cb, done, &pk, false, 0, -1, true))
                    continue;
                if (a.mask && !fast_dkdv_masked(pk)) continue;
                fa.g = pk.g;
                fa.walk_lo = done;
                if (border_of(pr, done, &fa.g.border)) {
                    fa.g.n_tiles = (int)(pr.batch * pr.heads * fa.g.tiles[0] * fa.g.border.per_plane);
                    set_divisors(fa.g);
                }
                const na_status st = fast_dkdv<T>(pk, fa, s);
                if (st != NA_OK) return st;
                done = cb;
            }
            if (done < need) {
                ak.skip_ch = done;  // 0: the split kernel takes every tile
                ak.skip_cw = done;
                if (done > 0 && border_of(pr, done, &ak.g.border))
                    ak.g.n_tiles = (int)(4 * pr.batch * pr.heads * ak.g.tiles[0] *
                                         ak.g.border.per_plane);
                auto kern = na::dkdv_kernel<T, D, 0>;
                if (!na_host::lds_limit_once((const void *)kern)) return NA_ERR_HIP;
                hipLaunchKernelGGL(kern, dim3(ak.g.n_tiles), dim3(na::kThreads), lds_k, s, ak);
                if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
            }
        }
        return NA_OK;
    }
    const int64_t n4 = pr.rows * D / 4;
    hipLaunchKernelGGL((na::delta_kernel<T, D>), flat_grid(pr.rows), dim3(kThreads), 0, s,
                       static_cast<const T *>(a.out), static_cast<const T *>(a.dout), a.delta,
                       pr.rows);
    if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
    if (kv_splits > 0) {
        // deterministic: classes of tiles with disjoint query boxes, run in rounds
        // of kv_splits classes, each class of a round adding into its own copy of
        // the accumulator; the copies are summed in order at the end
        int m[3];
        const int ncls = kv_classes(pr, m);
        const int ncopies = std::min<int>(kv_splits, ncls);
        const int64_t stride = (int64_t)pr.rows * D;
        const int64_t z4 = ncopies * stride / 4;
        hipLaunchKernelGGL(na::zero_kernel, flat_grid(z4), dim3(kThreads), 0, s, a.dq_acc, z4);
        if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
        na::BwdArgs ad = a;
        int lds_d = 0;
        if (!geometry(pr, true, 2 * PB + 8 + 8 * D, na::kWaves * 64 * (D + 1) * 4, &ad.g, &lds_d,
                      kLdsMax, true))
            return NA_ERR_UNSUPPORTED;
        auto kern = na::dkdv_kernel<T, D, 2>;
        if (!na_host::lds_limit_once((const void *)kern)) return NA_ERR_HIP;
        for (int a0 = 0; a0 < 3; ++a0) ad.cls_m[a0] = m[a0];
        ad.copy_stride = stride;
        for (int lo = 0; lo < ncls; lo += ncopies) {
            ad.cls_lo = lo;
            ad.cls_n = std::min(ncopies, ncls - lo);
            hipLaunchKernelGGL(kern, dim3(ad.g.n_tiles), dim3(na::kThreads), lds_d, s, ad);
            if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
        }
        hipLaunchKernelGGL((na::dq_copies_finalize_kernel<T>), flat_grid(n4), dim3(kThreads), 0, s,
                           a.dq_acc, ncopies, stride, static_cast<T *>(a.dq), a.scale, n4);
        return launched();
    }
    hipLaunchKernelGGL(na::zero_kernel, flat_grid(n4), dim3(kThreads), 0, s, a.dq_acc, n4);
    if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
    // dq contributions summed per workgroup in LDS over its query box when the
    // largest box fits beside the staging (one global atomic per box point and
    // channel instead of one per key block, query and channel)
    {
        int mx[3];
        max_union(pr, true, mx);
        const int64_t acc = (int64_t)mx[0] * mx[1] * mx[2] * (D + 1) * 4;
        const int off = (lds_k + 15) & ~15;
        if (off + acc <= kLdsMax) {
            ak.g.dq_lds_off = off;
            lds_k = (int)(off + acc);
        }
    }
    auto kern = na::dkdv_kernel<T, D, 1>;
    if (!na_host::lds_limit_once((const void *)kern)) return NA_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3(ak.g.n_tiles), dim3(na::kThreads), lds_k, s, ak);
    if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
    hipLaunchKernelGGL((na::dq_finalize_kernel<T>), flat_grid(n4), dim3(kThreads), 0, s,
                       a.dq_acc, static_cast<T *>(a.dq), a.scale, n4);
    return launched();
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

extern "C" {

na_status na_check_problem(const na_problem *p) { return validate(p, nullptr); }

const char *na_status_string(na_status s) {
    switch (s) {
        case NA_OK: return "NA_OK";
        case NA_ERR_INVALID_ARG: return "NA_ERR_INVALID_ARG: invalid problem or pointer";
        case NA_ERR_UNSUPPORTED:
            return "NA_ERR_UNSUPPORTED: no kernel for this problem (head_dim not 16, 32 or 64, a "
                   "window whose walk near a border exceeds 32 points, or a token row over 2 GiB)";
        case NA_ERR_WORKSPACE: return "NA_ERR_WORKSPACE: workspace missing or too small";
        case NA_ERR_HIP: return "NA_ERR_HIP: HIP runtime error at launch";
    }
    return "unknown na_status";
}

const char *na_source_sha256(void) { return NA_SOURCE_SHA256; }

int64_t na_window_start(int64_t extent, int64_t kernel, int64_t dilation, int64_t x) {
    if (extent < 1 || kernel < 1 || dilation < 1 || x < 0 || x >= extent || extent > INT32_MAX)
        return -1;
    if (kernel > extent / dilation) return -1;
    const int r = (int)(x % dilation);
    const int n = na::class_size((int)extent, (int)dilation, r);
    return r + dilation * na::window_start((int)(x / dilation), n, (int)kernel);
}

na_status na_inverse_window(int64_t extent, int64_t kernel, int64_t dilation, int64_t y,
                            int64_t *first, int64_t *last) {
    if (!first || !last) return NA_ERR_INVALID_ARG;
    if (extent < 1 || kernel < 1 || dilation < 1 || y < 0 || y >= extent || extent > INT32_MAX)
        return NA_ERR_INVALID_ARG;
    if (kernel > extent / dilation) return NA_ERR_INVALID_ARG;
    const int r = (int)(y % dilation);
    const int n = na::class_size((int)extent, (int)dilation, r);
    const int j = (int)(y / dilation);
    *first = r + dilation * na::inverse_first(j, n, (int)kernel);
    *last = r + dilation * na::inverse_last(j, n, (int)kernel);
    return NA_OK;
}

}  // extern "C"

namespace {

na_status fwd_common(const na_problem *p, const void *q, const void *k, const void *v, void *out,
                     float *lse, const int32_t *frame, void *hip_stream,
                     const uint8_t *mask = nullptr) {
    Prob pr;
    na_status st = validate(p, &pr);
    if (st != NA_OK) return st;
    if (!q || !k || !v || !out || !lse) return NA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
        return NA_ERR_INVALID_ARG;
    na::FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.qscale = pr.scale * na::kLog2e;
    a.frame = frame;
    a.frame_axis = p->ndim == 3 ? 0 : 1;
    a.mask = mask;
    a.mask_k = (int)(pr.ker[0] * pr.ker[1] * pr.ker[2]);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
#define NA_FWD_D(D)                                                   \
    case D:                                                           \
        if (pr.dtype == NA_F32) return run_fwd<float, D>(pr, a, s);   \
        if (pr.dtype == NA_BF16) return run_fwd<bf16, D>(pr, a, s);   \
        return run_fwd<f16, D>(pr, a, s);
    switch (pr.head_dim) { NA_FWD_D(16) NA_FWD_D(32) NA_FWD_D(64) }
#undef NA_FWD_D
    return NA_ERR_UNSUPPORTED;
}

bool frame_ok(const int32_t *frame) {
    return frame && (reinterpret_cast<uintptr_t>(frame) & 3u) == 0;
}

}  // namespace

extern "C" {

na_status na_fwd(const na_problem *p, const void *q, const void *k, const void *v, void *out,
                 float *lse, void *hip_stream) {
    return fwd_common(p, q, k, v, out, lse, nullptr, hip_stream);
}

na_status na_fwd_framed(const na_problem *p, const void *q, const void *k, const void *v,
                        void *out, float *lse, const int32_t *frame_kernel, void *hip_stream) {
    if (validate(p, nullptr) == NA_OK && !frame_ok(frame_kernel)) return NA_ERR_INVALID_ARG;
    return fwd_common(p, q, k, v, out, lse, frame_kernel, hip_stream);
}

na_status na_fwd_masked(const na_problem *p, const void *q, const void *k, const void *v,
                        void *out, float *lse, const uint8_t *mask, void *hip_stream) {
    if (validate(p, nullptr) == NA_OK && !mask) return NA_ERR_INVALID_ARG;
    return fwd_common(p, q, k, v, out, lse, nullptr, hip_stream, mask);
}

size_t na_bwd_workspace_bytes(const na_problem *p, int32_t variant, int32_t kv_splits) {
    Prob pr;
    if (validate(p, &pr) != NA_OK || kv_splits < 0) return 0;
    const size_t delta = round256((size_t)pr.rows * sizeof(float));
    if (variant == NA_BWD_GATHER) return delta;
    if (variant == NA_BWD_KVPARALLEL) {
        const size_t acc = (size_t)pr.rows * pr.head_dim * sizeof(float);
        return delta + round256(acc * (size_t)std::max(kv_splits, 1));
    }
    return 0;
}

namespace {

na_status bwd_common(const na_problem *p, const void *q, const void *k, const void *v,
                     const void *out, const void *dout, const float *lse, void *dq, void *dk,
                     void *dv, float *delta, float *dq_acc, int32_t variant, int32_t kv_splits,
                     int phases, void *hip_stream, const int32_t *frame = nullptr,
                     const uint8_t *mask = nullptr) {
    Prob pr;
    na_status st = validate(p, &pr);
    if (st != NA_OK) return st;
    na::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.dq_acc = dq_acc;
    a.qscale = pr.scale * na::kLog2e;
    a.scale = pr.scale;
    a.frame = frame;
    a.frame_axis = p->ndim == 3 ? 0 : 1;
    a.mask = mask;
    a.mask_k = (int)(pr.ker[0] * pr.ker[1] * pr.ker[2]);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
#define NA_BWD_D(D)                                                                 \
    case D:                                                                         \
        if (pr.dtype == NA_F32) return run_bwd<float, D>(pr, a, variant, kv_splits, phases, s); \
        if (pr.dtype == NA_BF16) return run_bwd<bf16, D>(pr, a, variant, kv_splits, phases, s); \
        return run_bwd<f16, D>(pr, a, variant, kv_splits, phases, s);
    switch (pr.head_dim) { NA_BWD_D(16) NA_BWD_D(32) NA_BWD_D(64) }
#undef NA_BWD_D
    return NA_ERR_UNSUPPORTED;
}

bool ptrs_ok(std::initializer_list<const void *> ptrs) {
    for (const void *ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return false;
    return true;
}

}  // namespace

namespace {

na_status bwd_entry(const na_problem *p, const void *q, const void *k, const void *v,
                    const void *out, const void *dout, const float *lse, void *dq, void *dk,
                    void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                    int32_t kv_splits, const int32_t *frame, void *hip_stream,
                    const uint8_t *mask = nullptr) {
    na_status st = validate(p, nullptr);
    if (st != NA_OK) return st;
    if (variant != NA_BWD_GATHER && variant != NA_BWD_KVPARALLEL) return NA_ERR_INVALID_ARG;
    if (kv_splits < 0) return NA_ERR_INVALID_ARG;
    if (!ptrs_ok({q, k, v, out, dout, lse, dq, dk, dv})) return NA_ERR_INVALID_ARG;
    const size_t need = na_bwd_workspace_bytes(p, variant, kv_splits);
    if (!workspace || workspace_bytes < need) return NA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NA_ERR_WORKSPACE;
    Prob pr;
    validate(p, &pr);
    float *delta = static_cast<float *>(workspace);
    float *dq_acc = variant == NA_BWD_KVPARALLEL
                        ? reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                    round256((size_t)pr.rows * sizeof(float)))
                        : nullptr;
    return bwd_common(p, q, k, v, out, dout, lse, dq, dk, dv, delta, dq_acc, variant, kv_splits,
                      kPhaseBoth, hip_stream, frame, mask);
}

}  // namespace

na_status na_bwd(const na_problem *p, const void *q, const void *k, const void *v,
                 const void *out, const void *dout, const float *lse, void *dq, void *dk,
                 void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                 int32_t kv_splits, void *hip_stream) {
    return bwd_entry(p, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes, variant,
                     kv_splits, nullptr, hip_stream);
}

na_status na_bwd_framed(const na_problem *p, const void *q, const void *k, const void *v,
                        const void *out, const void *dout, const float *lse, void *dq, void *dk,
                        void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                        int32_t kv_splits, const int32_t *frame_kernel, void *hip_stream) {
    if (validate(p, nullptr) == NA_OK && !frame_ok(frame_kernel)) return NA_ERR_INVALID_ARG;
    return bwd_entry(p, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes, variant,
                     kv_splits, frame_kernel, hip_stream);
}

na_status na_bwd_masked(const na_problem *p, const void *q, const void *k, const void *v,
                        const void *out, const void *dout, const float *lse, void *dq, void *dk,
                        void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                        int32_t kv_splits, const uint8_t *mask, void *hip_stream) {
    if (validate(p, nullptr) == NA_OK && !mask) return NA_ERR_INVALID_ARG;
    return bwd_entry(p, q, k, v, out, dout, lse, dq, dk, dv, workspace, workspace_bytes, variant,
                     kv_splits, nullptr, hip_stream, mask);
}

na_status na_bwd_dq(const na_problem *p, const void *q, const void *k, const void *v,
                    const void *out, const void *dout, const float *lse, void *dq, float *delta,
                    void *hip_stream) {
    na_status st = validate(p, nullptr);
    if (st != NA_OK) return st;
    if (!ptrs_ok({q, k, v, out, dout, lse, dq, delta})) return NA_ERR_INVALID_ARG;
    return bwd_common(p, q, k, v, out, dout, lse, dq, nullptr, nullptr, delta, nullptr,
                      NA_BWD_GATHER, 0, kPhaseDq, hip_stream);
}

na_status na_bwd_dkdv(const na_problem *p, const void *q, const void *k, const void *v,
                      const void *dout, const float *lse, const float *delta, void *dk, void *dv,
                      void *hip_stream) {
    na_status st = validate(p, nullptr);
    if (st != NA_OK) return st;
    if (!ptrs_ok({q, k, v, dout, lse, delta, dk, dv})) return NA_ERR_INVALID_ARG;
    return bwd_common(p, q, k, v, nullptr, dout, lse, nullptr, dk, dv, const_cast<float *>(delta),
                      nullptr, NA_BWD_GATHER, 0, kPhaseDkdv, hip_stream);
}

}  // extern "C"

// ----------------------------------------------------------------------------
// Backward without a caller workspace, for callers that cannot allocate device
// memory. Its one scratch buffer, the fp32 delta rows, is this file-scope
// array: every GPU the library runs on holds its own copy until the process
// ends. In host code the name `scratch` is only a host-side stand-in; the
// kernels get the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.

namespace {

static __device__ __align__(256) float scratch[kNoallocRows];

// Device address of `scratch` on the current device (nullptr on a HIP error
// or a device index past the table), kept in a fixed table: the lookup itself
// allocates nothing, host or device.
constexpr int kNoallocDevices = 64;

float *noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocDevices) return nullptr;
    static std::mutex mu;
    static float *ptrs[kNoallocDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev]) return ptrs[dev];
    float *ptr = nullptr;
    if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return nullptr;
    ptrs[dev] = ptr;
    return ptr;
}

}  // namespace

extern "C" {

na_status na_bwd_noalloc(const na_problem *p, const void *q, const void *k, const void *v,
                         const void *out, const void *dout, const float *lse, void *dq, void *dk,
                         void *dv, void *hip_stream) {
    Prob pr;
    na_status st = validate(p, &pr);
    if (st != NA_OK) return st;
    if (!ptrs_ok({q, k, v, out, dout, lse, dq, dk, dv})) return NA_ERR_INVALID_ARG;
    if (pr.rows > kNoallocRows) return NA_ERR_WORKSPACE;
    float *delta = noalloc_scratch();
    if (!delta) return NA_ERR_HIP;
    // delta is written in full by the dq kernel before dk/dv reads it: nothing
    // needs clearing between calls
    return bwd_common(p, q, k, v, out, dout, lse, dq, dk, dv, delta, nullptr, NA_BWD_GATHER, 0,
                      kPhaseBoth, hip_stream);
}

}  // extern "C"
