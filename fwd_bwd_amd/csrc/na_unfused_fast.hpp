// na_unfused_fast.hpp -- geometry of the unfused ops and their register-tiled
// kernels (fp32, head_dim 16 and 32).
//
// The unfused ops reuse the tile machinery of the fused kernels (na_fast.hpp):
// a workgroup of four waves owns a 16 x 16 tile of one residue class of one
// (batch, head) plane, one point per lane, the other side read from one
// staged box plane in LDS through the 4 x 4 x 1 MFMA blocks. A head-major
// tensor [B, heads, (T,) H, W, C] is the token-major layout of that machinery
// with one head and B * heads batch elements, so its decode and addressing
// apply unchanged. What differs is the attention array, which these ops read
// or write: its rows (K entries per point) pass through an LDS buffer so that
// global memory sees whole contiguous rows.
//
//   qk (QK, AGRAD): per window plane, scores of the lane's point against
//     its window (as the fused forward), then the plane's slice of the
//     attention rows of each wave's 8 x 8 points goes out through LDS;
//   av (AV, QGRAD): the slice comes in through LDS into the lane's registers,
//     then the weighted sum over the window (as the fused forward's P V);
//   av_inverse (KGRAD, VGRAD): the lane is a key; the attention entries of
//     the queries of its inverse window come in through LDS in chunks of box
//     rows, then the weighted sum over those queries (as the fused dk/dv).
//     Keys near the grid border have longer inverse windows: the compiled
//     walk covers them in several passes (offset walks), each adding to the
//     output of the previous one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "na_fast.hpp"
#include "na_host.hpp"
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

using namespace na;
using namespace na::fast;

struct UArgs {
    Geom g;
    const float *a;      // qk: the points' own vectors; av_inverse: the summed vectors
    const float *b;      // qk: the window vectors; av: the summed vectors
    const float *attn;   // av, av_inverse: the attention rows
    float *attn_out;     // qk: the attention rows
    float *out;          // av, av_inverse
    float alpha;
    int K, KP, kw;       // row length, one window plane's slice of it, window width
    FastDiv fKP;
    int rows_round;      // qk, av: rows of a wave's 8 x 8 points per LDS round (8, 4, 2, 1)
    int rows_full;       // qk on several planes: rows per LDS round of whole K-entry rows (0: off)
    FastDiv fK;
    int chunk_rows;      // av_inverse: box rows per attention chunk in LDS
    int oh, ow;          // av_inverse: walk offset of this pass, in patches
    int accumulate;      // av_inverse: add to out (passes after the first)
    const float *rpb;    // qk: relative positional bias [heads][2kt-1][2kh-1][2kw-1], or null
    int heads;           // qk with a bias: heads per batch element
    int rpb_off;         // qk with a bias: LDS byte offset of the bias table plane
    const uint8_t *mask; // qk: window mask [tokens][K] shared by every (batch, head) plane, or null
};

// Head of a tile's (batch, head) plane: planes are the batch elements of the
// head-major layout, base = plane * (tokens * head_dim) + class origin.
__device__ __forceinline__ int tile_head(const UArgs &a, const TileCtx &w) {
    const int64_t plane_elems = (int64_t)a.g.ext[0] * a.g.ext[1] * a.g.ext[2] * a.g.head_dim;
    return (int)((w.base / plane_elems) % a.heads);
}

// One window plane's slice (KP entries per point) of the attention rows of
// quarter rows [r0, r0 + rows_round) of a wave's 8 x 8 points, as one LDS
// array: point (row, col) of the round at buf + ((row - r0) * 8 + col) * KP.
// One quarter row at a time (its global base is wave-uniform), its 8 * KP
// elements taken by consecutive lanes; element e is entry e % KP of point
// column e / KP. With unit stride along W and a single window plane the
// row's slice is one contiguous run of global memory.
struct RowRun {
    int64_t base;     // global index of entry 0 of the row's first point
    int64_t cstride;  // global elements from one point of the row to the next
    int n;            // elements of the row inside the grid
    int kp;           // entries per point in the run: one window plane's slice, or (full) K
    FastDiv fkp;
    bool contiguous;
};

__device__ __forceinline__ RowRun row_run(const UArgs &a, const TileCtx &w, int t, int row,
                                          int col0, int cols, int it, bool full = false) {
    RowRun rr;
    const int c[3] = {t, row, col0};
    rr.kp = full ? a.K : a.KP;
    rr.fkp = full ? a.fK : a.fKP;
    rr.base = row_off(w, c) * a.K + it * rr.kp;
    rr.cstride = w.lst[2] * a.K;
    rr.n = imax(0, imin(cols, w.n[2] - col0)) * rr.kp;
    rr.contiguous = rr.cstride == rr.kp;
    return rr;
}

__device__ __forceinline__ int64_t run_index(const UArgs &, const RowRun &rr, int e) {
    if (rr.contiguous) return rr.base + e;
    const int col = fdiv(e, rr.fkp);
    return rr.base + col * rr.cstride + (e - col * rr.kp);
}

// Per-lane offsets of the elements e = lane + 64 m (m < kRunSteps) of a row
// run of `cols` points relative to its base: every row of a box has the same
// shape, so they are computed once per tile instead of once per element.
constexpr int kRunSteps = 16;

struct RunOffs {
    int off[kRunSteps];
    bool ok;  // the run fits kRunSteps steps of 64 lanes
};

__device__ __forceinline__ RunOffs run_offs(const UArgs &a, const TileCtx &w, int cols,
                                            bool full = false) {
    RunOffs ro;
    const int lane = threadIdx.x & 63;
    const int kp = full ? a.K : a.KP;
    const FastDiv fkp = full ? a.fK : a.fKP;
    const int n = cols * kp;
    ro.ok = n <= 64 * kRunSteps;
    const int cstride = (int)(w.lst[2] * a.K);
#pragma unroll
    for (int m = 0; m < kRunSteps; ++m) {
        const int e = lane + 64 * m;
        const int col = fdiv(e, fkp);
        ro.off[m] = col * cstride + (e - col * kp);
    }
    return ro;
}

// One row run, global -> LDS with direct loads (no register round trip, all in
// flight at once), by waves wv, wv + nw, ... of the workgroup, 64 lanes per
// step: 16-byte pieces when the run is contiguous and both ends are 16-byte
// aligned (vec), else 4-byte ones. Completion: stage_wait().
__device__ __forceinline__ void load_run(const UArgs &a, const RowRun &rr, const float *src,
                                         float *l, bool vec, int wv, int nw,
                                         const RunOffs *ro = nullptr) {
    const int lane = threadIdx.x & 63;
#if defined(__HIP_DEVICE_COMPILE__)
    if (vec) {
        const float *g = src + rr.base;
        const int n4 = rr.n >> 2;
        for (int b = 64 * wv; b < n4; b += 64 * nw)
            if (b + lane < n4)
                __builtin_amdgcn_global_load_lds(g + 4 * (b + lane), (lds_void *)(l + 4 * b), 16, 0, 0);
        for (int b = 4 * n4 + 64 * wv; b < rr.n; b += 64 * nw)
            if (b + lane < rr.n)
                __builtin_amdgcn_global_load_lds(g + b + lane, (lds_void *)(l + b), 4, 0, 0);
    } else if (ro && ro->ok && nw == 1) {
        const float *g = src + rr.base;
#pragma unroll
        for (int m = 0; m < kRunSteps; ++m)
            if (64 * m + lane < rr.n)
                __builtin_amdgcn_global_load_lds(g + ro->off[m], (lds_void *)(l + 64 * m), 4, 0, 0);
    } else {
        for (int b = 64 * wv; b < rr.n; b += 64 * nw)
            if (b + lane < rr.n)
                __builtin_amdgcn_global_load_lds(src + run_index(a, rr, b + lane), (lds_void *)(l + b),
                                                 4, 0, 0);
    }
#else
    (void)a; (void)rr; (void)src; (void)l; (void)vec; (void)wv; (void)nw; (void)lane; (void)ro;
#endif
}

__device__ __forceinline__ bool run_vec(const RowRun &rr, int lds_off) {
    return rr.contiguous && (rr.base & 3) == 0 && (lds_off & 3) == 0;
}

__device__ __forceinline__ void load_round(const UArgs &a, const TileCtx &w, int wave, int r0,
                                           int it, float *buf, const float *src,
                                           const RunOffs &ro) {
    const int qr0 = w.o[1] + 8 * (wave >> 1) + r0, qc0 = w.o[2] + 8 * (wave & 1);
    for (int row = 0; row < a.rows_round && qr0 + row < w.n[1]; ++row) {
        const RowRun rr = row_run(a, w, w.o[0], qr0 + row, qc0, 8, it);
        load_run(a, rr, src, buf + row * 8 * a.KP, run_vec(rr, row * 8 * a.KP), 0, 1, &ro);
    }
}

// A masked-out window entry: its score is -inf, so the softmax gives it no weight.
__device__ __forceinline__ float masked(const uint8_t *m, int64_t i, float v) {
    return m[i] ? v : -INFINITY;
}

// LDS -> global, one wave: 16-byte pieces where aligned, else 4-byte ones,
// four LDS reads in flight per lane. With a window mask, entry i of the
// attention array takes mask[i - mbase] (the mask indexes one plane). full:
// whole K-entry rows (rows_full per round) instead of one window plane's slice.
__device__ __forceinline__ void store_round(const UArgs &a, const TileCtx &w, int wave, int r0,
                                            int it, const float *buf, float *dst,
                                            const RunOffs &ro, int64_t mbase, bool use_mask,
                                            bool full = false) {
    const int lane = threadIdx.x & 63;
    const int qr0 = w.o[1] + 8 * (wave >> 1) + r0, qc0 = w.o[2] + 8 * (wave & 1);
    const uint8_t *mk = use_mask && a.mask ? a.mask - mbase : nullptr;
    const int rows = full ? a.rows_full : a.rows_round;
    for (int row = 0; row < rows && qr0 + row < w.n[1]; ++row) {
        const RowRun rr = row_run(a, w, w.o[0], qr0 + row, qc0, 8, it, full);
        const int kp = rr.kp;
        const float *brow = buf + row * 8 * kp;
        if (run_vec(rr, row * 8 * kp) &&
            (!mk || ((reinterpret_cast<uintptr_t>(mk + rr.base) & 3) == 0))) {
            const int n4 = rr.n >> 2;
            const float4 *l4 = reinterpret_cast<const float4 *>(brow);
            float4 *g4 = reinterpret_cast<float4 *>(dst + rr.base);
            if (mk) {
                const uchar4 *m4 = reinterpret_cast<const uchar4 *>(mk + rr.base);
                for (int b = lane; b < n4; b += 64) {
                    float4 v = l4[b];
                    const uchar4 m = m4[b];
                    v.x = m.x ? v.x : -INFINITY;
                    v.y = m.y ? v.y : -INFINITY;
                    v.z = m.z ? v.z : -INFINITY;
                    v.w = m.w ? v.w : -INFINITY;
                    g4[b] = v;
                }
                for (int e = 4 * n4 + lane; e < rr.n; e += 64)
                    dst[rr.base + e] = masked(mk, rr.base + e, brow[e]);
            } else {
                for (int b = lane; b < n4; b += 64) g4[b] = l4[b];
                for (int e = 4 * n4 + lane; e < rr.n; e += 64) dst[rr.base + e] = brow[e];
            }
            continue;
        }
        if (ro.ok) {
            float v[kRunSteps];
#pragma unroll
            for (int m = 0; m < kRunSteps; ++m)
                v[m] = 64 * m + lane < rr.n ? brow[64 * m + lane] : 0.f;
#pragma unroll
            for (int m = 0; m < kRunSteps; ++m)
                if (64 * m + lane < rr.n) {
                    const int64_t gi = rr.base + ro.off[m];
                    dst[gi] = mk ? masked(mk, gi, v[m]) : v[m];
                }
            continue;
        }
        for (int e0 = 0; e0 < rr.n; e0 += 4 * 64) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + 64 * u + lane;
                v[u] = e < rr.n ? brow[e] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + 64 * u + lane;
                if (e < rr.n) {
                    const int64_t gi = run_index(a, rr, e);
                    dst[gi] = mk ? masked(mk, gi, v[u]) : v[u];
                }
            }
        }
    }
}

// ============================================================================
// qk on grids with several planes, windows of at most rows_planes(CH * CW)
// planes: the scores of every window plane stay in the lane's registers, and
// the whole K-entry rows leave through LDS at the end. (Storing each plane's
// slice as it is formed writes runs of k_h * k_w entries K entries apart,
// partial lines that cost more than the scores: 1.8 ms of 2.9 ms for a
// 3 x 5 x 5 window on a 16 x 256 x 256 grid of 8 heads.)
constexpr int rows_planes(int ni) { return ni <= 4 ? 5 : ni <= 9 ? 3 : 0; }

template <int D, int CH, int CW, bool RPB>
__device__ __forceinline__ void qk_rows(const UArgs &a, const TileCtx &w, char *smem) {
    constexpr int PS = D * 4, NC = D / 4, NI = CH * CW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3, grp = lane >> 2;
    const Lane L = lane_geom(w, wave, lane);

    int us[3], lo[3], U[3], E[3];
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        us[x] = window_start(L.f[x], w.n[x], w.k[x]);
        lo[x] = window_start(L.p[x], w.n[x], w.k[x]) - us[x];
        key_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], &U[x], &E[x]);
    }
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    const int ra = a.g.ra;
    const char *baseA = smem + (us[1] - U[1] + (c >> 1)) * ra + (us[2] - U[2] + (c & 1)) * PS;
    const int64_t qo = elem_off(w, L.p);
    const int lr = 2 * (grp & 3) + (c >> 1), lc = 2 * (grp >> 2) + (c & 1);
    const int plane_tokens_k = w.k[1] * w.k[2];

    // bias: this head's whole table (2 k_t - 1 planes) in LDS past the staging
    // area and the row buffers, read when the rows are formed
    const int RH = 2 * w.k[1] - 1, RW = 2 * w.k[2] - 1;
    if constexpr (RPB) {
        const int n = (2 * w.k[0] - 1) * RH * RW;
        const float *src = a.rpb + (int64_t)tile_head(a, w) * n;
        float *dstl = reinterpret_cast<float *>(smem + a.rpb_off);
        for (int i = threadIdx.x; i < n; i += kThreads) dstl[i] = src[i];
    }

    constexpr int NP = rows_planes(NI);
    float s[NP][NI][4];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        if (j >= w.k[0]) break;
        const int tk = t0 + j;
        if (j > 0) __syncthreads();  // the previous plane is read no more
        stage_plane<float, D, PS>(a.b, w, tk, U[1], E[1], U[2], E[2], ra, smem);
        float qr[D];
        load_row<float, D>(a.a + qo + opaque_zero(), qr);
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] *= a.alpha;
        stage_wait();

        {
            f4 kb[2][NC / 2], z0, z1;
            pipelined<2 * NI>(
                [&](int jj, int bb) {
                    const int i = jj >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (jj & 1) * (NC / 2) * 16, kb[bb]);
                },
                [&](int jj, int bb) {
                    const int i = jj >> 1;
                    if ((jj & 1) == 0) z0 = z1 = f4{0.f, 0.f, 0.f, 0.f};
                    dot_half<NC / 2>(kb[bb], qr, (jj & 1) * (NC / 2), z0, z1);
                    if ((jj & 1) == 0) return;
                    const f4 z = z0 + z1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[j][i][e] = z[e];
                    pin4(s[j][i]);
                });
        }
    }
    __syncthreads();  // the staged planes are read no more: their LDS takes the rows

    const RunOffs ro = run_offs(a, w, 8, true);
    const int64_t plane_tokens = (int64_t)a.g.ext[0] * a.g.ext[1] * a.g.ext[2];
    const int64_t mbase = a.mask ? (w.lbase / plane_tokens) * plane_tokens * a.K : 0;
    float *buf = reinterpret_cast<float *>(smem) + wave * (a.rows_full * 8 * a.K);
    for (int r0 = 0; r0 < 8; r0 += a.rows_full) {
        if (lr >= r0 && lr < r0 + a.rows_full) {
            float *slot = buf + ((lr - r0) * 8 + lc) * a.K;
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                if (j >= w.k[0]) break;
                // bias of key plane t0 + j: the lane's entry for walk row h, column
                // wc at tbl + h * RW + wc (offset key - query + k - 1 per axis)
                const float *tbl = reinterpret_cast<const float *>(smem + a.rpb_off) +
                                   ((t0 + j - w.o[0] + w.k[0] - 1) * RH + us[1] - L.p[1] + w.k[1] - 1) * RW +
                                   (us[2] - L.p[2] + w.k[2] - 1);
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int h = 2 * (i / CW) + (e >> 1), wc = 2 * (i % CW) + (e & 1);
                        const int jh = h - lo[1], jw = wc - lo[2];
                        if ((unsigned)jh < (unsigned)w.k[1] && (unsigned)jw < (unsigned)w.k[2]) {
                            if constexpr (RPB)
                                slot[j * plane_tokens_k + jh * a.kw + jw] = s[j][i][e] + tbl[h * RW + wc];
                            else
                                slot[j * plane_tokens_k + jh * a.kw + jw] = s[j][i][e];
                        }
                    }
            }
        }
        __syncthreads();
        store_round(a, w, wave, r0, 0, buf, a.attn_out, ro, mbase, true, true);
        __syncthreads();
    }
}

// ============================================================================
// qk: attn[x][j] = alpha <a_x, b_{N(x)_j}>
// MODE 0: the scores. MODE 1 (single-plane grids): the window softmax of the
// scores, computed in the lane's registers (the whole window is there), so
// the probabilities leave instead of the scores. MODE 2 (single-plane grids):
// the scores are dP = <dout, v> (AGRAD); the lane's probabilities come in
// through LDS and dS = P (dP - sum_j P dP) leaves (the softmax backward).
template <int D, int CH, int CW, bool T3, bool RPB, int MODE>
__device__ __forceinline__ void qk_tile(const UArgs &a, int tile, char *smem) {
    static_assert(MODE == 0 || !T3, "the fused softmax needs the whole window in one plane");
    constexpr int PS = D * 4, NC = D / 4, NI = CH * CW;
    TileCtx w;
    if (!decode(a.g, tile, w)) return;
    if constexpr (T3 && MODE == 0 && rows_planes(NI) > 0) {
        // (rows_full is set only for windows of at most rows_planes(NI) planes)
        if (a.rows_full > 0) {
            qk_rows<D, CH, CW, RPB>(a, w, smem);
            return;
        }
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3, grp = lane >> 2;
    const Lane L = lane_geom(w, wave, lane);

    int us[3], lo[3], U[3], E[3];
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        us[x] = window_start(L.f[x], w.n[x], w.k[x]);
        lo[x] = window_start(L.p[x], w.n[x], w.k[x]) - us[x];
        key_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], &U[x], &E[x]);
    }
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    const int ra = a.g.ra;
    const char *baseA = smem + (us[1] - U[1] + (c >> 1)) * ra + (us[2] - U[2] + (c & 1)) * PS;
    const int64_t qo = elem_off(w, L.p);
    // the lane's point in its wave's 8 x 8 quarter, and the wave's LDS buffer
    const int lr = 2 * (grp & 3) + (c >> 1), lc = 2 * (grp >> 2) + (c & 1);
    float *buf = reinterpret_cast<float *>(smem) + wave * (a.rows_round * 8 * a.KP);
    // row-run offsets: formed once per tile for the plain scores; the softmax
    // modes form them after the window's scores, which they would otherwise
    // share the registers with (the bias variant spilled)
    RunOffs ro;
    if constexpr (MODE == 0) ro = run_offs(a, w, 8);
    // first attention entry of this tile's (batch, head) plane (the mask spans one plane)
    const int64_t plane_tokens = (int64_t)a.g.ext[0] * a.g.ext[1] * a.g.ext[2];
    const int64_t mbase = a.mask ? (w.lbase / plane_tokens) * plane_tokens * a.K : 0;

    const int nplanes = T3 ? w.k[0] : 1;
    for (int j = 0; j < nplanes; ++j) {
        const int tk = t0 + j;
        if (j > 0) __syncthreads();
        stage_plane<float, D, PS>(a.b, w, tk, U[1], E[1], U[2], E[2], ra, smem);
        float qr[D];
        load_row<float, D>(a.a + qo + opaque_zero(), qr);
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] *= a.alpha;
        stage_wait();

        // S_b[i][c] = <b_i, a_c> over the walk
        float s[NI][4];
        {
            f4 kb[2][NC / 2], z0, z1;
            pipelined<2 * NI>(
                [&](int jj, int bb) {
                    const int i = jj >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (jj & 1) * (NC / 2) * 16, kb[bb]);
                },
                [&](int jj, int bb) {
                    const int i = jj >> 1;
                    if ((jj & 1) == 0) z0 = z1 = f4{0.f, 0.f, 0.f, 0.f};
                    dot_half<NC / 2>(kb[bb], qr, (jj & 1) * (NC / 2), z0, z1);
                    if ((jj & 1) == 0) return;
                    const f4 z = z0 + z1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[i][e] = z[e];
                    pin4(s[i]);
                });
        }
        // bias: this head's table plane for the key plane tk in LDS (past the
        // staging area); the lane's entry for walk row h, column wc sits at
        // tbl + h * RW + wc (offset key - query + k - 1 per axis)
        const float *tbl = nullptr;
        if constexpr (RPB) {
            const int RH = 2 * w.k[1] - 1, RW = 2 * w.k[2] - 1;
            const float *src = a.rpb + ((int64_t)tile_head(a, w) * (2 * w.k[0] - 1) + tk - w.o[0] +
                                        w.k[0] - 1) * RH * RW;
            float *dstl = reinterpret_cast<float *>(smem + a.rpb_off);
            for (int i = threadIdx.x; i < RH * RW; i += kThreads) dstl[i] = src[i];
            tbl = dstl + (us[1] - L.p[1] + w.k[1] - 1) * RW + (us[2] - L.p[2] + w.k[2] - 1);
            // the softmax below reads entries other waves copied (the plain
            // scores read them only after the barrier that frees the staging)
            if constexpr (MODE == 1) __syncthreads();
        }
        if constexpr (MODE == 1) {
            // window softmax in registers: bias, window and mask decide the
            // entries; the others get zero weight
            const uint8_t *mrow = nullptr;
            if (a.mask) {
                const int c0[3] = {w.o[0], L.p[1], L.p[2]};
                mrow = a.mask + (row_off(w, c0) - (w.lbase / plane_tokens) * plane_tokens) * a.K;
            }
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int h = 2 * (i / CW) + (e >> 1), wc = 2 * (i % CW) + (e & 1);
                    const int jh = h - lo[1], jw = wc - lo[2];
                    bool ok = (unsigned)jh < (unsigned)w.k[1] && (unsigned)jw < (unsigned)w.k[2];
                    if (ok && mrow) ok = mrow[jh * a.kw + jw] != 0;
                    float v = s[i][e];
                    if constexpr (RPB) v += tbl[h * (2 * w.k[2] - 1) + wc];
                    s[i][e] = ok ? v : -INFINITY;
                    m = fmaxf(m, s[i][e]);
                }
            if (m == -INFINITY) m = 0.f;   // every entry masked out: zero weights
            float l = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s[i][e] = __expf(s[i][e] - m);
                    l += s[i][e];
                }
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[i][e] *= inv;
        }
        __syncthreads();  // the staged plane is read no more: its LDS takes the rows
        if constexpr (MODE != 0) ro = run_offs(a, w, 8);
        for (int r0 = 0; r0 < 8; r0 += a.rows_round) {
            const bool mine = lr >= r0 && lr < r0 + a.rows_round;
            float *slot = buf + ((lr - r0) * 8 + lc) * a.KP;
            if constexpr (MODE == 2) {
                // this round's probabilities into the slots, then dS in place
                load_round(a, w, wave, r0, j, buf, a.attn, ro);
                stage_wait();
                if (mine) {
                    float rs = 0.f;
#pragma unroll
                    for (int i = 0; i < NI; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int jh = 2 * (i / CW) + (e >> 1) - lo[1];
                            const int jw = 2 * (i % CW) + (e & 1) - lo[2];
                            if ((unsigned)jh < (unsigned)w.k[1] && (unsigned)jw < (unsigned)w.k[2])
                                rs += slot[jh * a.kw + jw] * s[i][e];
                        }
#pragma unroll
                    for (int i = 0; i < NI; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int jh = 2 * (i / CW) + (e >> 1) - lo[1];
                            const int jw = 2 * (i % CW) + (e & 1) - lo[2];
                            if ((unsigned)jh < (unsigned)w.k[1] && (unsigned)jw < (unsigned)w.k[2]) {
                                float *q = slot + jh * a.kw + jw;
                                *q = *q * (s[i][e] - rs);
                            }
                        }
                }
            } else if (mine) {
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int h = 2 * (i / CW) + (e >> 1), wc = 2 * (i % CW) + (e & 1);
                        const int jh = h - lo[1], jw = wc - lo[2];
                        if ((unsigned)jh < (unsigned)w.k[1] && (unsigned)jw < (unsigned)w.k[2]) {
                            if constexpr (RPB && MODE == 0)
                                slot[jh * a.kw + jw] = s[i][e] + tbl[h * (2 * w.k[2] - 1) + wc];
                            else
                                slot[jh * a.kw + jw] = s[i][e];
                        }
                    }
            }
            __syncthreads();
            store_round(a, w, wave, r0, j, buf, a.attn_out, ro, mbase, MODE == 0);
            __syncthreads();
        }
    }
}

// ============================================================================
// av: out_x = alpha sum_j attn[x][j] b_{N(x)_j}
template <int D, int CH, int CW, bool T3>
__device__ __forceinline__ void av_tile(const UArgs &a, int tile, char *smem) {
    constexpr int PS = D * 4, G = D / 4, NI = CH * CW;
    TileCtx w;
    if (!decode(a.g, tile, w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3, grp = lane >> 2;
    const Lane L = lane_geom(w, wave, lane);

    int us[3], lo[3], U[3], E[3];
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        us[x] = window_start(L.f[x], w.n[x], w.k[x]);
        lo[x] = window_start(L.p[x], w.n[x], w.k[x]) - us[x];
        key_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], &U[x], &E[x]);
    }
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    const int rb = a.g.rb;
    const char *baseB = smem + (us[1] - U[1]) * rb + (us[2] - U[2]) * PS + c * 16;
    const int lr = 2 * (grp & 3) + (c >> 1), lc = 2 * (grp >> 2) + (c & 1);
    float *buf = reinterpret_cast<float *>(smem) + wave * (a.rows_round * 8 * a.KP);

    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    const int nplanes = T3 ? w.k[0] : 1;
    for (int j = 0; j < nplanes; ++j) {
        const int tk = t0 + j;
        if (j > 0) __syncthreads();
        // this plane's weights into the registers of the walk (0 off the window)
        float s[NI][4];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[i][e] = 0.f;
        // row-run offsets: formed per plane so that they hold no registers
        // across the products
        const RunOffs ro = run_offs(a, w, 8);
        for (int r0 = 0; r0 < 8; r0 += a.rows_round) {
            load_round(a, w, wave, r0, j, buf, a.attn, ro);
            stage_wait();
            if (L.active && lr >= r0 && lr < r0 + a.rows_round) {
                const float *slot = buf + ((lr - r0) * 8 + lc) * a.KP;
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jh = 2 * (i / CW) + (e >> 1) - lo[1];
                        const int jw = 2 * (i % CW) + (e & 1) - lo[2];
                        if ((unsigned)jh < (unsigned)w.k[1] && (unsigned)jw < (unsigned)w.k[2])
                            s[i][e] = slot[jh * a.kw + jw];
                    }
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) pin4(s[i]);
        stage_plane<float, D, PS>(a.b, w, tk, U[1], E[1], U[2], E[2], rb, smem);
        stage_wait();

        // O_b[i][c] += b_e[dim(i, g)] * attn[c][e]
        {
            f4 vb[2][2][D / 16];
            pipelined<2 * NI>(
                [&](int jj, int bb) {
                    const int i = jj >> 1;
                    load_row_dmajor<D, PS>(baseB + (2 * (i / CW) + (jj & 1)) * rb,
                                           2 * (i % CW) * PS, vb[bb]);
                },
                [&](int jj, int bb) {
                    const int i = jj >> 1, h = jj & 1;
                    axpy_row<D>(vb[bb], s[i][2 * h], s[i][2 * h + 1], acc);
                });
        }
    }
    if (L.active) store_row<float, D>(a.out + elem_off(w, L.p), acc, a.alpha);
}

// ============================================================================
// av_inverse: out_y = alpha sum_{x : y in N(x)} attn[x][j(x, y)] a_x
template <int D, int CH, int CW, bool T3>
__device__ __forceinline__ void avi_tile(const UArgs &a, int tile, char *smem) {
    constexpr int PS = D * 4, G = D / 4, NI = CH * CW;
    TileCtx w;
    if (!decode(a.g, tile, w)) return;
    // this pass walks patches [oh, oh + CH) x [ow, ow + CW) of the inverse walks
    if (tile_inverse_walk(w.o[1], kTH, 2, w.n[1], w.k[1]) <= a.oh ||
        tile_inverse_walk(w.o[2], kTW, 2, w.n[2], w.k[2]) <= a.ow)
        return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3;
    const Lane L = lane_geom(w, wave, lane);  // keys

    int lo[3], U[3], E[3];
    unsigned vm[3];
    const int off[3] = {0, 2 * a.oh, 2 * a.ow};
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        const int cnt = off[x] / 2 + (x == 1 ? CH : CW);
        query_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], cnt, &U[x], &E[x]);
        U[x] += off[x];
        E[x] -= off[x];
        lo[x] = inverse_first(L.f[x], w.n[x], w.k[x]) + off[x];
        const int s0 = imax(0, inverse_first(L.p[x], w.n[x], w.k[x]) - lo[x]);
        const int s1 = imin(2 * (x == 1 ? CH : CW), inverse_last(L.p[x], w.n[x], w.k[x]) - lo[x] + 1);
        vm[x] = s1 > s0 ? bit_range(s0, s1 - s0) : 0u;
    }
    const int tq0 = inverse_first(w.o[0], w.n[0], w.k[0]);
    const int tq1 = inverse_last(w.o[0], w.n[0], w.k[0]);

    const int rb = a.g.rb;
    const int rel1 = lo[1] - U[1], rel2 = lo[2] - U[2];
    const char *baseB = smem + rel1 * rb + rel2 * PS + c * 16;
    float *abuf = reinterpret_cast<float *>(smem);

    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    const int nplanes = T3 ? tq1 - tq0 + 1 : 1;
    for (int j = 0; j < nplanes; ++j) {
        const int tq = tq0 + j;
        const int it = w.o[0] - window_start(tq, w.n[0], w.k[0]);  // window plane of the key
        float s[NI][4];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[i][e] = 0.f;
        // Formed per plane so that they hold no registers across the products:
        // the row-run offsets, and the LDS offsets (relative to the lane's
        // first walk point) of the entry of this lane's key in the attention
        // row of walk row h / column wc (the point's place in the box plus the
        // key's offset in that query's window)
        const RunOffs aro = run_offs(a, w, E[2]);
        int rowt[2 * CH], colt[2 * CW];
#pragma unroll
        for (int h = 0; h < 2 * CH; ++h)
            rowt[h] = h * E[2] * a.KP +
                      (L.p[1] - window_start(imin(lo[1] + h, w.n[1] - 1), w.n[1], w.k[1])) * a.kw;
#pragma unroll
        for (int h = 0; h < 2 * CW; ++h)
            colt[h] = h * a.KP + L.p[2] - window_start(imin(lo[2] + h, w.n[2] - 1), w.n[2], w.k[2]);
        // the box's attention entries of window plane it, a chunk of box rows
        // at a time: LDS element e = entry jj of box point pt = r * E2 + col
        for (int r0 = 0; r0 < E[1]; r0 += a.chunk_rows) {
            const int rows = imin(a.chunk_rows, E[1] - r0);
            if (j > 0 || r0 > 0) __syncthreads();
            for (int r = wave; r < rows && U[1] + r0 + r < w.n[1]; r += kWaves) {
                const RowRun rr = row_run(a, w, tq, U[1] + r0 + r, U[2], E[2], it);
                const int off = r * E[2] * a.KP;
                load_run(a, rr, a.attn, abuf + off, run_vec(rr, off), 0, 1, &aro);
            }
            stage_wait();
            // walk rows of this lane inside the chunk
            const int h0 = imax(0, r0 - rel1), h1 = imin(32, r0 - rel1 + rows);
            const unsigned rm = h1 > h0 ? vm[1] & bit_range(h0, h1 - h0) : 0u;
            const float *cb = abuf + ((rel1 - r0) * E[2] + rel2) * a.KP;
            if (rm) {
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int h = 2 * (i / CW) + (e >> 1), wc = 2 * (i % CW) + (e & 1);
                        if ((rm >> h) & (vm[2] >> wc) & 1u) s[i][e] = cb[rowt[h] + colt[wc]];
                    }
            }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) pin4(s[i]);
        __syncthreads();
        stage_plane<float, D, PS>(a.a, w, tq, U[1], E[1], U[2], E[2], rb, smem);
        stage_wait();

        // Out_b[i][c] += a_e[dim(i, g)] * attn[e][c]
        {
            f4 vb[2][2][D / 16];
            pipelined<2 * NI>(
                [&](int jj, int bb) {
                    const int i = jj >> 1;
                    load_row_dmajor<D, PS>(baseB + (2 * (i / CW) + (jj & 1)) * rb,
                                           2 * (i % CW) * PS, vb[bb]);
                },
                [&](int jj, int bb) {
                    const int i = jj >> 1, h = jj & 1;
                    axpy_row<D>(vb[bb], s[i][2 * h], s[i][2 * h + 1], acc);
                });
        }
        __syncthreads();
    }
    if (L.active) {
        float *dst = a.out + elem_off(w, L.p);
        if (a.accumulate) {
            // add the output of the earlier passes (same layout as store_row)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < D / 16; ++j) {
                    float o[4];
                    Io<float>::load4(dst + 4 * (i + 4 * j), o);
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[4 * j + t][i] = acc[4 * j + t][i] * a.alpha + o[t];
                }
            store_row<float, D>(dst, acc, 1.f);
        } else {
            store_row<float, D>(dst, acc, a.alpha);
        }
    }
}

template <int D, int CH, int CW, bool T3, bool RPB, int MODE>
__global__ void __launch_bounds__(kThreads, 2) qk_kernel(UArgs a) {
    extern __shared__ __align__(16) char smem[];
    qk_tile<D, CH, CW, T3, RPB, MODE>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

template <int D, int CH, int CW, bool T3>
__global__ void __launch_bounds__(kThreads, 2) av_kernel(UArgs a) {
    extern __shared__ __align__(16) char smem[];
    av_tile<D, CH, CW, T3>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

template <int D, int CH, int CW, bool T3>
__global__ void __launch_bounds__(kThreads, 2) avi_kernel(UArgs a) {
    extern __shared__ __align__(16) char smem[];
    avi_tile<D, CH, CW, T3>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

// ============================================================================
// Host planning.

constexpr int kLdsCap = 80 * 1024;  // two workgroups per CU

// Compiled walks: 2 .. 5 patches per axis on single-plane grids, 2 .. 4 with
// several planes along T, as for the fused kernels.
inline bool walk_compiled(int c, bool t3) { return c >= 2 && c <= (t3 ? 4 : 5); }

inline void set_divisors(Geom &g) {
    const int band = kFastBand, last = g.tiles[2] % band;
    g.f_heads = na::make_fastdiv(g.heads);
    g.f_t = na::make_fastdiv(g.tiles[0]);
    g.f_plane = na::make_fastdiv(g.tiles[1] * g.tiles[2]);
    g.f_bandrows = na::make_fastdiv(band * g.tiles[1]);
    g.f_band = na::make_fastdiv(band);
    g.f_lastband = na::make_fastdiv(last ? last : band);
    g.f_nres = na::make_fastdiv(g.nres);
    g.f_c = na::make_fastdiv(g.tiles[2]);
    g.f_cb = na::make_fastdiv(1);
    for (int a = 0; a < 3; ++a) g.f_dil[a] = na::make_fastdiv(g.dil[a]);
    g.f_dil21 = na::make_fastdiv(g.dil[2] * g.dil[1]);
}

struct UPlan {
    UArgs a;
    int lds;
    int c;
    bool t3;
};

// kind 0: qk / av; kind 1: av_inverse, one pass at walk offset (oh, ow).
inline bool plan(const Geo &geo, int64_t bh, int D, int kind, int oh, int ow, UPlan *pl) {
    if (D != 16 && D != 32) return false;
    const bool t3 = geo.ext[0] > 1;
    const int c = na::window_walk(geo.ker[1], 2);
    if (na::window_walk(geo.ker[2], 2) != c || !walk_compiled(c, t3)) return false;
    const int PB = D * 4;
    const int off[3] = {0, 2 * oh, 2 * ow};
    int mx[3] = {1, 1, 1};
    for (int a = 1; a < 3; ++a)
        for (int r = 0; r < geo.dil[a] && r < geo.ext[a]; ++r) {
            const int n = na::class_size(geo.ext[a], geo.dil[a], r);
            for (int f = 0; f < n; f += 16) {
                int start, extent;
                if (kind == 0) {
                    na::key_box(f, 16, 2, n, geo.ker[a], &start, &extent);
                } else {
                    if (na::tile_inverse_walk(f, 16, 2, n, geo.ker[a]) <= off[a] / 2) continue;
                    na::query_box(f, 16, 2, n, geo.ker[a], off[a] / 2 + c, &start, &extent);
                    extent -= off[a];
                }
                mx[a] = std::max(mx[a], extent);
            }
        }
    // row pitches as for the fused kernels: odd slot count (key-major reads),
    // 2 mod 4 slots (d-major reads)
    const int slots = mx[2] * PB / 16;
    const int rb = (slots + ((2 - slots % 4) + 4) % 4) * 16;
    const int ra = (slots | 1) * 16;
    int64_t lds = (int64_t)mx[1] * (kind == 0 ? std::max(ra, rb) : rb);
    UArgs &u = pl->a;
    u = UArgs{};
    u.K = geo.K;
    u.KP = geo.khw;
    u.fKP = na::make_fastdiv(geo.khw);
    u.kw = geo.kw;
    if (kind == 0) {
        // rows per LDS round of the wave buffers (four waves)
        int R = 8;
        while (R > 1 && (int64_t)4 * R * 8 * u.KP * 4 > std::max<int64_t>(lds, kLdsCap)) R /= 2;
        if ((int64_t)4 * R * 8 * u.KP * 4 > kLdsCap) return false;
        u.rows_round = R;
        lds = std::max<int64_t>(lds, (int64_t)4 * R * 8 * u.KP * 4);
    } else {
        const int64_t row_bytes = (int64_t)mx[2] * u.KP * 4;
        const int64_t room = std::max<int64_t>(lds, kLdsCap);
        if (row_bytes > room) return false;
        u.chunk_rows = (int)std::min<int64_t>(mx[1], room / row_bytes);
        lds = std::max<int64_t>(lds, u.chunk_rows * row_bytes);
    }
    if (lds > kLdsCap) return false;
    Geom &g = u.g;
    int64_t n_tiles = bh;
    int nres = 1;
    for (int a = 0; a < 3; ++a) {
        g.ext[a] = geo.ext[a];
        g.ker[a] = geo.ker[a];
        g.dil[a] = geo.dil[a];
        const int nmax = na::class_size(geo.ext[a], geo.dil[a], 0);
        g.tiles[a] = a == 0 ? nmax : (nmax + 15) / 16;
        n_tiles *= g.tiles[a];
        nres *= geo.dil[a];
    }
    n_tiles *= nres;
    if (n_tiles > INT32_MAX || bh > INT32_MAX) return false;
    g.heads = 1;  // head-major tensors: (batch, head) planes are batch elements
    g.batch = (int)bh;
    g.head_dim = D;
    g.nres = nres;
    g.n_tiles = (int)n_tiles;
    g.ra = ra;
    g.rb = rb;
    set_divisors(g);
    u.oh = oh;
    u.ow = ow;
    pl->lds = (int)lds;
    pl->c = c;
    pl->t3 = t3;
    return true;
}

template <typename Kern>
inline bool launch(Kern kern, const UPlan &pl, hipStream_t s) {
    if (!na_host::lds_limit_once((const void *)kern)) return false;
    if (pl.a.g.n_tiles > 0)
        hipLaunchKernelGGL(kern, dim3(pl.a.g.n_tiles), dim3(kThreads), pl.lds, s, pl.a);
    return true;
}

#define NU_CASES(X)                                                          \
    X(16, 2, false) X(16, 3, false) X(16, 4, false) X(16, 5, false)          \
    X(32, 2, false) X(32, 3, false) X(32, 4, false) X(32, 5, false)          \
    X(16, 2, true) X(16, 3, true) X(16, 4, true)                             \
    X(32, 2, true) X(32, 3, true) X(32, 4, true)

// Register-tiled paths; each returns false (launching nothing) when the
// problem is outside what they cover.
inline bool fast_qk(const Geo &geo, int64_t bh, int D, const float *a, const float *b, float alpha,
                    const float *rpb, const uint8_t *mask, int heads, float *attn, hipStream_t s) {
    UPlan pl;
    if (!plan(geo, bh, D, 0, 0, 0, &pl)) return false;
    pl.a.a = a;
    pl.a.b = b;
    pl.a.attn_out = attn;
    pl.a.alpha = alpha;
    pl.a.rpb = rpb;
    pl.a.mask = mask;
    pl.a.heads = heads;
    if (pl.t3 && geo.ker[0] <= rows_planes(pl.c * pl.c)) {
        // whole rows at the end: the four waves' round buffers of K-entry rows
        // share the LDS with the staging area
        int R = 8;
        while (R > 1 && (int64_t)4 * R * 8 * geo.K * 4 > std::max<int64_t>(pl.lds, kLdsCap)) R /= 2;
        const int64_t bytes = (int64_t)4 * R * 8 * geo.K * 4;
        if (bytes <= kLdsCap) {
            pl.a.rows_full = R;
            pl.a.fK = na::make_fastdiv(geo.K);
            pl.lds = (int)std::max<int64_t>(pl.lds, bytes);
        }
    }
    if (rpb) {
        // the bias table plane after the staging area; with whole rows, the
        // head's whole table after the row buffers
        pl.a.rpb_off = (pl.lds + 15) & ~15;
        pl.lds = pl.a.rpb_off + (pl.a.rows_full ? 2 * geo.ker[0] - 1 : 1) * (2 * geo.ker[1] - 1) *
                                    (2 * geo.ker[2] - 1) * 4;
        if (pl.lds > kLdsCap) return false;
    }
#define X(DD, C, T3)                                                                          \
    if (D == DD && pl.c == C && pl.t3 == T3)                                                  \
        return rpb ? launch(qk_kernel<DD, C, C, T3, true, 0>, pl, s)                          \
                   : launch(qk_kernel<DD, C, C, T3, false, 0>, pl, s);
    NU_CASES(X)
#undef X
    return false;
}

// The single-plane compiled cases (the fused softmax needs the whole window
// of a query in one plane).
#define NU_CASES2D(X)                                                        \
    X(16, 2) X(16, 3) X(16, 4) X(16, 5) X(32, 2) X(32, 3) X(32, 4) X(32, 5)

// Scores plus the window softmax in one kernel: probs (2D only).
inline bool fast_qk_softmax(const Geo &geo, int64_t bh, int D, const float *a, const float *b,
                            float alpha, const float *rpb, const uint8_t *mask, int heads,
                            float *probs, hipStream_t s) {
    UPlan pl;
    if (!plan(geo, bh, D, 0, 0, 0, &pl) || pl.t3) return false;
    pl.a.a = a;
    pl.a.b = b;
    pl.a.attn_out = probs;
    pl.a.alpha = alpha;
    pl.a.rpb = rpb;
    pl.a.mask = mask;
    pl.a.heads = heads;
    if (rpb) {
        pl.a.rpb_off = (pl.lds + 15) & ~15;
        pl.lds = pl.a.rpb_off + (2 * geo.ker[1] - 1) * (2 * geo.ker[2] - 1) * 4;
        if (pl.lds > kLdsCap) return false;
    }
#define X(DD, C)                                                                              \
    if (D == DD && pl.c == C)                                                                 \
        return rpb ? launch(qk_kernel<DD, C, C, false, true, 1>, pl, s)                       \
                   : launch(qk_kernel<DD, C, C, false, false, 1>, pl, s);
    NU_CASES2D(X)
#undef X
    return false;
}

// AGRAD plus the softmax backward in one kernel: dscores from dout, v, probs (2D only).
inline bool fast_qk_softmax_bwd(const Geo &geo, int64_t bh, int D, const float *dout,
                                const float *v, const float *probs, float *dscores,
                                hipStream_t s) {
    UPlan pl;
    if (!plan(geo, bh, D, 0, 0, 0, &pl) || pl.t3) return false;
    pl.a.a = dout;
    pl.a.b = v;
    pl.a.attn = probs;
    pl.a.attn_out = dscores;
    pl.a.alpha = 1.f;
#define X(DD, C) \
    if (D == DD && pl.c == C) return launch(qk_kernel<DD, C, C, false, false, 2>, pl, s);
    NU_CASES2D(X)
#undef X
    return false;
}

inline bool fast_av(const Geo &geo, int64_t bh, int D, const float *attn, const float *b,
                    float alpha, float *out, hipStream_t s) {
    UPlan pl;
    if (!plan(geo, bh, D, 0, 0, 0, &pl)) return false;
    pl.a.b = b;
    pl.a.attn = attn;
    pl.a.out = out;
    pl.a.alpha = alpha;
#define X(DD, C, T3) \
    if (D == DD && pl.c == C && pl.t3 == T3) return launch(av_kernel<DD, C, C, T3>, pl, s);
    NU_CASES(X)
#undef X
    return false;
}

// Longest inverse walk (patches) along axis a over every tile of every class.
inline int max_inverse_walk(const Geo &geo, int a) {
    int m = 1;
    for (int r = 0; r < geo.dil[a] && r < geo.ext[a]; ++r) {
        const int n = na::class_size(geo.ext[a], geo.dil[a], r);
        for (int f = 0; f < n; f += 16) m = std::max(m, na::tile_inverse_walk(f, 16, 2, n, geo.ker[a]));
    }
    return m;
}

inline bool fast_av_inverse(const Geo &geo, int64_t bh, int D, const float *attn, const float *a,
                            float alpha, float *out, hipStream_t s) {
    UPlan pl;
    if (!plan(geo, bh, D, 1, 0, 0, &pl)) return false;
    const int c = pl.c;
    const int wh = max_inverse_walk(geo, 1), ww = max_inverse_walk(geo, 2);
    // plan every pass first: launch nothing unless all of them fit
    const int ph = (wh + c - 1) / c, pw = (ww + c - 1) / c;
    if (ph * pw > 16) return false;
    UPlan plans[16];
    for (int i = 0; i < ph; ++i)
        for (int j = 0; j < pw; ++j)
            if (!plan(geo, bh, D, 1, i * c, j * c, &plans[i * pw + j])) return false;
    for (int p = 0; p < ph * pw; ++p) {
        UPlan &q = plans[p];
        q.a.a = a;
        q.a.attn = attn;
        q.a.out = out;
        q.a.alpha = alpha;
        q.a.accumulate = p > 0;
        bool ok = false;
#define X(DD, C, T3)                                                               \
    if (!ok && D == DD && q.c == C && q.t3 == T3) {                                \
        if (!launch(avi_kernel<DD, C, C, T3>, q, s)) return false;                 \
        ok = true;                                                                 \
    }
        NU_CASES(X)
#undef X
        if (!ok) return false;
    }
    return true;
}

}  // namespace nu
