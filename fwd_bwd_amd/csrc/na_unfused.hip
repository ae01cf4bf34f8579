// na_unfused.hip -- the unfused neighborhood-attention ops of libna (declared
// in include/na.h): window scores, the window softmax and the weighted sums
// over windows and inverse windows, on head-major tensors.
//
// NATTEN issue #161, "Backward pass is very slow towards much tokens and large
// kernels": the benchmark script's unfused method materializes the scores of
// every query against its window (na2d_qk / na3d_qk, shape [B, heads, (T,) H,
// W, K]), applies a softmax over the last axis and takes the weighted sum of
// the values (na2d_av / na3d_av); the maintainer's profiler tables list the
// backward of these ops as AGRAD and VGRAD (of av) and QGRAD and KGRAD (of
// qk). All six contractions are one of three maps:
//   qk          attn[x][j] = alpha <a_x, b_{N(x)_j}>                  QK, AGRAD
//   av          out_x = alpha sum_j attn[x][j] b_{N(x)_j}             AV, QGRAD
//   av_inverse  out_y = alpha sum_{x : y in N(x)} attn[x][j] a_x      KGRAD, VGRAD
// with j the position of the key in the window of x (row-major over the
// window's (t, h, w) offsets).
//
// Two implementations per map: register-tiled kernels for fp32 head_dim 16
// and 32 (na_unfused_fast.hpp), and plain per-element kernels for everything
// else. Both use the window arithmetic of na_index.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "na.h"
#include "na_index.hpp"
#include "na_unfused_fast.hpp"

namespace {

// ----------------------------------------------------------------------------
// Host-side problem description (head-major tensors).

struct UProb {
    nu::Geo g;
    int64_t heads;
    int64_t bh;     // batch * heads
    int64_t units;  // bh * tokens
    int D;
};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// need_dim: the op reads head_dim-long vectors (all but the two softmax ops).
na_status uvalidate(const na_problem *p, UProb *out, bool need_dim = true) {
    if (!p) return NA_ERR_INVALID_ARG;
    if (p->ndim != 2 && p->ndim != 3) return NA_ERR_INVALID_ARG;
    if (p->dtype != NA_F32 && p->dtype != NA_BF16) return NA_ERR_INVALID_ARG;
    if (p->batch < 1 || p->heads < 1 || p->head_dim < 1) return NA_ERR_INVALID_ARG;
    if (!std::isfinite(p->scale)) return NA_ERR_INVALID_ARG;
    const int nd = (int)p->ndim;
    UProb q{};
    for (int a = 0; a < 3; ++a) q.g.ext[a] = q.g.ker[a] = q.g.dil[a] = 1;
    int64_t tokens = 1, K = 1;
    for (int a = 0; a < nd; ++a) {
        const int64_t L = p->extent[a], k = p->kernel[a], d = p->dilation[a];
        if (L < 1 || k < 1 || d < 1) return NA_ERR_INVALID_ARG;
        if (L > INT32_MAX || d > L) return NA_ERR_INVALID_ARG;
        if (k > L / d) return NA_ERR_INVALID_ARG;
        tokens *= L;
        K *= k;
        if (tokens > INT32_MAX) return NA_ERR_INVALID_ARG;
        const int dst = a + (3 - nd);
        q.g.ext[dst] = (int)L;
        q.g.ker[dst] = (int)k;
        q.g.dil[dst] = (int)d;
    }
    if (p->batch > INT32_MAX || p->heads > INT32_MAX) return NA_ERR_INVALID_ARG;
    if (need_dim && p->head_dim != 16 && p->head_dim != 32 && p->head_dim != 64)
        return NA_ERR_UNSUPPORTED;
    if (p->dtype != NA_F32) return NA_ERR_UNSUPPORTED;  // the unfused ops are fp32
    q.g.tokens = (int)tokens;
    q.g.K = (int)K;
    q.g.kw = q.g.ker[2];
    q.g.khw = q.g.ker[1] * q.g.ker[2];
    q.heads = p->heads;
    q.bh = p->batch * p->heads;
    q.units = q.bh * tokens;
    q.D = (int)p->head_dim;
    if (out) *out = q;
    return NA_OK;
}

int grid_for(int64_t items, int per_block) {
    const int64_t b = (items + per_block - 1) / per_block;
    return (int)std::min<int64_t>(std::max<int64_t>(b, 1), 1 << 20);
}

na_status launched() { return hipGetLastError() == hipSuccess ? NA_OK : NA_ERR_HIP; }

// ----------------------------------------------------------------------------
// Plain kernels: one thread per output element (qk) or per 16-byte chunk of an
// output row (av, av_inverse), operands read straight from global memory.

using nu::Geo;

__device__ __forceinline__ void unit_coords(const Geo &g, int64_t u, int64_t *bh, int (&c)[3]) {
    *bh = u / g.tokens;
    int tok = (int)(u - *bh * g.tokens);
    c[2] = tok % g.ext[2];
    tok /= g.ext[2];
    c[1] = tok % g.ext[1];
    c[0] = tok / g.ext[1];
}

// Absolute coordinate of the first key of the window of coordinate x on axis a.
__device__ __forceinline__ int window_first(const Geo &g, int a, int x) {
    const int d = g.dil[a], r = x % d;
    return r + d * na::window_start(x / d, na::class_size(g.ext[a], d, r), g.ker[a]);
}

__device__ __forceinline__ int64_t token_of(const Geo &g, int t, int y, int x) {
    return ((int64_t)t * g.ext[1] + y) * g.ext[2] + x;
}

// Index in one head's bias table of the key at window offsets (jt, jh, jw) of
// the query at coordinates c: the offset key - query in class units plus k - 1
// per axis.
__device__ __forceinline__ int rpb_entry(const Geo &g, const int (&c)[3], int jt, int jh, int jw) {
    const int j3[3] = {jt, jh, jw};
    int idx = 0;
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
        const int d = g.dil[ax], i = c[ax] / d;
        const int s = na::window_start(i, na::class_size(g.ext[ax], d, c[ax] % d), g.ker[ax]);
        idx = idx * (2 * g.ker[ax] - 1) + (s + j3[ax] - i) + g.ker[ax] - 1;
    }
    return idx;
}

template <int D>
__global__ __launch_bounds__(256) void qk_plain(Geo g, const float *__restrict__ a,
                                                const float *__restrict__ b, float alpha,
                                                const float *__restrict__ rpb, int heads,
                                                const uint8_t *__restrict__ mask,
                                                float *__restrict__ attn, int64_t total) {
    for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += gridDim.x * 256ll) {
        const int64_t u = e / g.K;
        const int j = (int)(e - u * g.K);
        int64_t bh;
        int c[3];
        unit_coords(g, u, &bh, c);
        const int jt = j / g.khw, jh = (j / g.kw) % g.ker[1], jw = j % g.kw;
        const int kt = window_first(g, 0, c[0]) + g.dil[0] * jt;
        const int ky = window_first(g, 1, c[1]) + g.dil[1] * jh;
        const int kx = window_first(g, 2, c[2]) + g.dil[2] * jw;
        const int64_t ku = bh * g.tokens + token_of(g, kt, ky, kx);
        const float4 *pa = reinterpret_cast<const float4 *>(a + u * D);
        const float4 *pb = reinterpret_cast<const float4 *>(b + ku * D);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            const float4 x = pa[i], y = pb[i];
            s += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        }
        if (rpb) {
            const int R = (2 * g.ker[0] - 1) * (2 * g.ker[1] - 1) * (2 * g.ker[2] - 1);
            s = alpha * s + rpb[(int64_t)(bh % heads) * R + rpb_entry(g, c, jt, jh, jw)];
        } else {
            s = alpha * s;
        }
        // a masked-out entry: -inf, no weight after the softmax
        if (mask && !mask[(u - bh * g.tokens) * g.K + j]) s = -INFINITY;
        attn[e] = s;
    }
}

template <int D>
__global__ __launch_bounds__(256) void av_plain(Geo g, const float *__restrict__ attn,
                                                const float *__restrict__ b, float alpha,
                                                float *__restrict__ out, int64_t total) {
    constexpr int NC = D / 4;
    for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += gridDim.x * 256ll) {
        const int64_t u = e / NC;
        const int ch = (int)(e - u * NC);
        int64_t bh;
        int c[3];
        unit_coords(g, u, &bh, c);
        const int s0 = window_first(g, 0, c[0]), s1 = window_first(g, 1, c[1]),
                  s2 = window_first(g, 2, c[2]);
        const float *row = attn + u * g.K;
        const float4 *pb = reinterpret_cast<const float4 *>(b) + ch;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int j = 0;
        for (int it = 0; it < g.ker[0]; ++it)
            for (int ih = 0; ih < g.ker[1]; ++ih) {
                const int64_t rowtok =
                    bh * g.tokens + token_of(g, s0 + g.dil[0] * it, s1 + g.dil[1] * ih, s2);
                for (int iw = 0; iw < g.ker[2]; ++iw, ++j) {
                    const float w = row[j];
                    const float4 v = pb[(rowtok + (int64_t)g.dil[2] * iw) * NC];
                    acc.x += w * v.x;
                    acc.y += w * v.y;
                    acc.z += w * v.z;
                    acc.w += w * v.w;
                }
            }
        reinterpret_cast<float4 *>(out)[e] =
            make_float4(alpha * acc.x, alpha * acc.y, alpha * acc.z, alpha * acc.w);
    }
}

template <int D>
__global__ __launch_bounds__(256) void av_inverse_plain(Geo g, const float *__restrict__ attn,
                                                        const float *__restrict__ a, float alpha,
                                                        float *__restrict__ out, int64_t total) {
    constexpr int NC = D / 4;
    for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += gridDim.x * 256ll) {
        const int64_t u = e / NC;
        const int ch = (int)(e - u * NC);
        int64_t bh;
        int c[3];
        unit_coords(g, u, &bh, c);
        // per axis: residue, class size, key class index, inverse query range
        int r[3], n[3], kj[3], lo[3], hi[3];
#pragma unroll
        for (int ax = 0; ax < 3; ++ax) {
            r[ax] = c[ax] % g.dil[ax];
            n[ax] = na::class_size(g.ext[ax], g.dil[ax], r[ax]);
            kj[ax] = c[ax] / g.dil[ax];
            lo[ax] = na::inverse_first(kj[ax], n[ax], g.ker[ax]);
            hi[ax] = na::inverse_last(kj[ax], n[ax], g.ker[ax]);
        }
        const float4 *pa = reinterpret_cast<const float4 *>(a) + ch;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int qt = lo[0]; qt <= hi[0]; ++qt) {
            const int wt = kj[0] - na::window_start(qt, n[0], g.ker[0]);
            for (int qy = lo[1]; qy <= hi[1]; ++qy) {
                const int wh = kj[1] - na::window_start(qy, n[1], g.ker[1]);
                for (int qx = lo[2]; qx <= hi[2]; ++qx) {
                    const int ww = kj[2] - na::window_start(qx, n[2], g.ker[2]);
                    const int64_t xu =
                        bh * g.tokens + token_of(g, r[0] + g.dil[0] * qt, r[1] + g.dil[1] * qy,
                                                 r[2] + g.dil[2] * qx);
                    const float w = attn[xu * g.K + (wt * g.ker[1] + wh) * g.kw + ww];
                    const float4 v = pa[xu * NC];
                    acc.x += w * v.x;
                    acc.y += w * v.y;
                    acc.z += w * v.z;
                    acc.w += w * v.w;
                }
            }
        }
        reinterpret_cast<float4 *>(out)[e] =
            make_float4(alpha * acc.x, alpha * acc.y, alpha * acc.z, alpha * acc.w);
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// ----------------------------------------------------------------------------
// Gradient of the relative positional bias: drpb[head][o] = sum of dscores over
// every (batch, query, window entry) whose key sits at offset o from the
// query. Deterministic two-stage sum, no atomics: a workgroup takes one chunk
// of kRpbChunk queries of one (batch, head) plane, keeps as many of their rows
// in LDS as fit at a time, and each thread sums the entries of a few offsets
// (every query has at most one entry per offset) into a partial per chunk;
// a second kernel adds the partials of every chunk of every batch element in
// a fixed order.

constexpr int kRpbChunk = 256;        // queries per workgroup
constexpr int kRpbLds = 8192;         // floats of LDS for rows (32 KB)
constexpr int kRpbMaxK = 512;         // window entries (two per thread at most)
constexpr int kRpbPerThread = 8;      // offsets per thread: R <= 2048

__global__ __launch_bounds__(256) void rpb_partial_kernel(Geo g, const float *__restrict__ ds,
                                                          float *__restrict__ partial, int chunks) {
    __shared__ __align__(16) float rows[kRpbLds];
    __shared__ int rel[kRpbChunk][3];   // query's place in its window per axis (class units)
    __shared__ float colsum[kRpbMaxK];
    __shared__ unsigned long long refmask[kRpbChunk / 64];
    const int plane = blockIdx.x / chunks, chunk = blockIdx.x - plane * chunks;
    const int R1 = 2 * g.ker[1] - 1, R2 = 2 * g.ker[2] - 1;
    const int R = (2 * g.ker[0] - 1) * R1 * R2;
    const int nm = (R + 255) / 256, nj = (g.K + 255) / 256;
    const int G = g.K <= 128 ? 256 / g.K : 1;   // column groups summing in parallel
    const int lane = threadIdx.x & 63;
    // this thread's offsets: o = threadIdx.x + 256 m, as (dt, dh, dw) from k - 1
    int dt[kRpbPerThread], dh[kRpbPerThread], dw[kRpbPerThread];
    float acc[kRpbPerThread], cs[2] = {0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kRpbPerThread; ++m) {
        const int o = threadIdx.x + 256 * m;
        dt[m] = o / (R1 * R2) - (g.ker[0] - 1);
        dh[m] = (o / R2) % R1 - (g.ker[1] - 1);
        dw[m] = o % R2 - (g.ker[2] - 1);
        acc[m] = 0.f;
    }
    const int q0 = chunk * kRpbChunk;
    const int nq = min(kRpbChunk, g.tokens - q0);
    if (threadIdx.x < nq) {
        int tok = q0 + threadIdx.x;
        int c[3];
        c[2] = tok % g.ext[2];
        tok /= g.ext[2];
        c[1] = tok % g.ext[1];
        c[0] = tok / g.ext[1];
#pragma unroll
        for (int ax = 0; ax < 3; ++ax) {
            const int d = g.dil[ax], i = c[ax] / d;
            rel[threadIdx.x][ax] =
                i - na::window_start(i, na::class_size(g.ext[ax], d, c[ax] % d), g.ker[ax]);
        }
    }
    __syncthreads();
    // Most queries of a chunk sit at the same place in their windows (the
    // chunk's middle query's): for those the offset of entry j is fixed, so
    // their part is a column sum; the others are summed offset by offset.
    // refmask bit q: query q is such a query.
    const int ref0 = rel[nq / 2][0], ref1 = rel[nq / 2][1], ref2 = rel[nq / 2][2];
    {
        const int t = threadIdx.x;
        const bool isref = t < nq && rel[t][0] == ref0 && rel[t][1] == ref1 && rel[t][2] == ref2;
        const unsigned long long bal = __ballot(isref);
        if (lane == 0) refmask[t >> 6] = bal;
    }
    const int sub = (kRpbLds / g.K) & ~3;   // rows per LDS fill (a multiple of 4)
    const float *base = ds + ((int64_t)plane * g.tokens + q0) * g.K;
    const bool vec = ((((int64_t)plane * g.tokens + q0) * g.K) & 3) == 0;
    for (int s0 = 0; s0 < nq; s0 += sub) {
        const int ns = min(sub, nq - s0);
        __syncthreads();
        // direct loads, all in flight; lanes of a wave take consecutive pieces
        // (16 bytes when the rows start 16-byte aligned: s0 K is a multiple of 4)
        const int n = ns * g.K, n4 = vec ? n >> 2 : 0;
#if defined(__HIP_DEVICE_COMPILE__)
        for (int i = threadIdx.x; i < n4; i += 256)
            __builtin_amdgcn_global_load_lds(base + (int64_t)s0 * g.K + 4 * i,
                                             (lds_void *)(rows + 4 * (i - lane)), 16, 0, 0);
        for (int i = 4 * n4 + (int)threadIdx.x; i < n; i += 256)
            __builtin_amdgcn_global_load_lds(base + (int64_t)s0 * g.K + i,
                                             (lds_void *)(rows + (i - lane)), 4, 0, 0);
#else
        (void)base; (void)lane; (void)n4;
#endif
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int q = 0; q < ns;) {
            const int gq = s0 + q;
            const int run = min(64 - (gq & 63), ns - q);   // queries left in this mask word
            const unsigned long long live = run == 64 ? ~0ull : ((1ull << run) - 1);
            const unsigned long long word = (refmask[gq >> 6] >> (gq & 63)) & live;
            // column sums over the reference queries: thread (group gi, column
            // j) takes the queries u = gi, gi + G, ... of the run
            if (G > 1) {
                const int gi = threadIdx.x / g.K, j = threadIdx.x - gi * g.K;
                if (gi < G) {
                    const float *col = rows + q * g.K + j;
                    float sum = 0.f;
#pragma unroll 4
                    for (int u = gi; u < run; u += G) sum += ((word >> u) & 1ull) ? col[u * g.K] : 0.f;
                    cs[0] += sum;
                }
            } else {
                for (int m = 0; m < nj; ++m) {
                    const int j = threadIdx.x + 256 * m;
                    if (j >= g.K) continue;
                    const float *col = rows + q * g.K + j;
                    float sum = 0.f;
#pragma unroll 8
                    for (int u = 0; u < run; ++u) sum += ((word >> u) & 1ull) ? col[u * g.K] : 0.f;
                    cs[m] += sum;
                }
            }
            // the other queries, offset by offset
            for (unsigned long long other = ~word & live; other; other &= other - 1) {
                const int u = __ffsll((long long)other) - 1;
                const int rt = rel[gq + u][0], rh = rel[gq + u][1], rw = rel[gq + u][2];
                const float *row = rows + (q + u) * g.K;
                for (int m = 0; m < nm; ++m) {
                    const int jt = dt[m] + rt, jh = dh[m] + rh, jw = dw[m] + rw;
                    if (threadIdx.x + 256 * m < R && (unsigned)jt < (unsigned)g.ker[0] &&
                        (unsigned)jh < (unsigned)g.ker[1] && (unsigned)jw < (unsigned)g.ker[2])
                        acc[m] += row[(jt * g.ker[1] + jh) * g.kw + jw];
                }
            }
            q += run;
        }
    }
    if (G > 1) {
        // groups in order: colsum[j] = group 0 + group 1 + ...
        __syncthreads();
        const int gi = threadIdx.x / g.K, j = threadIdx.x - gi * g.K;
        if (gi < G) rows[gi * g.K + j] = cs[0];
        __syncthreads();
        if (threadIdx.x < g.K) {
            float sum = 0.f;
            for (int k2 = 0; k2 < G; ++k2) sum += rows[k2 * g.K + threadIdx.x];
            colsum[threadIdx.x] = sum;
        }
    } else {
        for (int m = 0; m < nj; ++m)
            if (threadIdx.x + 256 * m < g.K) colsum[threadIdx.x + 256 * m] = cs[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kRpbPerThread; ++m) {
        if (threadIdx.x + 256 * m >= R) continue;
        const int jt = dt[m] + ref0, jh = dh[m] + ref1, jw = dw[m] + ref2;
        float v = acc[m];
        if ((unsigned)jt < (unsigned)g.ker[0] && (unsigned)jh < (unsigned)g.ker[1] &&
            (unsigned)jw < (unsigned)g.ker[2])
            v += colsum[(jt * g.ker[1] + jh) * g.kw + jw];
        partial[(int64_t)blockIdx.x * R + threadIdx.x + 256 * m] = v;
    }
}

// drpb[h][o] = sum over batch elements b and chunks c of
// partial[(b * heads + h) * chunks + c][o]. A workgroup takes 16 offsets of
// one head; its 16 slices of 16 threads each sum every 16th (b, c) partial
// (eight loads in flight per thread), then the 16 slice sums are added in
// slice order: a fixed summation order, so the result is deterministic.
__global__ __launch_bounds__(256) void rpb_reduce_kernel(const float *__restrict__ partial,
                                                         float *__restrict__ drpb, int batch,
                                                         int heads, int chunks, int R) {
    __shared__ float slice_sum[16][17];
    const int oblocks = (R + 15) / 16;
    const int h = blockIdx.x / oblocks, ob = blockIdx.x - h * oblocks;
    const int oo = threadIdx.x & 15, sl = threadIdx.x >> 4;
    const int o = ob * 16 + oo;
    const int n = batch * chunks;   // partials per (head, offset)
    float sum = 0.f;
    if (o < R) {
        for (int i0 = sl; i0 < n; i0 += 16 * 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 16 * u;
                if (i < n) {
                    const int b = i / chunks, c = i - b * chunks;
                    v[u] = partial[((int64_t)(b * heads + h) * chunks + c) * R + o];
                } else {
                    v[u] = 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
    }
    slice_sum[sl][oo] = sum;
    __syncthreads();
    if (sl == 0 && o < R) {
        float t = 0.f;
        for (int k2 = 0; k2 < 16; ++k2) t += slice_sum[k2][oo];
        drpb[(int64_t)h * R + o] = t;
    }
}

// ----------------------------------------------------------------------------
// Window softmax and its backward over rows of K entries. A workgroup takes 64
// consecutive rows, one contiguous run of 64 K floats starting 16-byte aligned
// (64 K is a multiple of 4), moved between HBM and LDS with 16-byte accesses;
// four lanes share a row and reduce it with two shuffles. Rows of more than
// kRowMax entries take the plain path below (sixteen lanes per row, read in
// passes).

constexpr int kRowsPerBlock = 64;
constexpr int kRowMax = 160;   // 64 rows x 160 entries x 4 bytes = 40 KB of LDS per array

__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1, 4));
    return fmaxf(v, __shfl_xor(v, 2, 4));
}
__device__ __forceinline__ float quad_sum(float v) {
    v += __shfl_xor(v, 1, 4);
    return v + __shfl_xor(v, 2, 4);
}


// Copy the first n & ~3 floats (global offset 16-byte aligned) global -> LDS
// with direct 16-byte loads, all in flight at once; completion: waitcnt + barrier.
__device__ __forceinline__ void block_in(const float *g, float *l, int n) {
    const int lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < (n >> 2); i += 256) {
        // lanes of a wave hold consecutive i: LDS base l + 4 (i - lane) is wave-uniform
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_global_load_lds(g + 4 * i, (lds_void *)(l + 4 * (i - lane)), 16, 0, 0);
#else
        (void)g; (void)l; (void)lane;
#endif
    }
}
__device__ __forceinline__ void block_out(const float *l, float *g, int n) {
    const int n4 = n >> 2;
    const float4 *l4 = reinterpret_cast<const float4 *>(l);
    float4 *g4 = reinterpret_cast<float4 *>(g);
    int i = threadIdx.x;
    for (; i + 768 < n4; i += 1024) {
        const float4 a = l4[i], b = l4[i + 256], c = l4[i + 512], d = l4[i + 768];
        g4[i] = a;
        g4[i + 256] = b;
        g4[i + 512] = c;
        g4[i + 768] = d;
    }
    for (; i < n4; i += 256) g4[i] = l4[i];
}

// Rows [row0, row0 + nr) of one block; nr = 64 except for the last block,
// whose tail (nr * K not a multiple of 4) is moved with 4-byte accesses.
__device__ __forceinline__ void tail_in(const float *g, float *l, int n) {
    for (int i = (n & ~3) + (int)threadIdx.x; i < n; i += 256) l[i] = g[i];
}
__device__ __forceinline__ void tail_out(const float *l, float *g, int n) {
    for (int i = (n & ~3) + (int)threadIdx.x; i < n; i += 256) g[i] = l[i];
}

__global__ __launch_bounds__(256) void softmax_blocks(const float *x, float *y, int64_t rows,
                                                      int K) {
    __shared__ __align__(16) float xs[kRowsPerBlock * kRowMax];
    const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock;
    const int nr = (int)(rows - row0 < kRowsPerBlock ? rows - row0 : kRowsPerBlock);
    const int n = nr * K;
    const float *xg = x + row0 * K;
    float *yg = y + row0 * K;
    block_in(xg, xs, n);
    tail_in(xg, xs, n);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int r = threadIdx.x >> 2, l = threadIdx.x & 3;
    float *xr = xs + r * K;
    const bool ok = r < nr;
    float m = -INFINITY;
    for (int i = l; ok && i < K; i += 4) m = fmaxf(m, xr[i]);
    m = quad_max(m);
    if (m == -INFINITY) m = 0.f;   // every entry masked out: zero weights
    float sum = 0.f;
    for (int i = l; ok && i < K; i += 4) {
        const float e = __expf(xr[i] - m);
        xr[i] = e;
        sum += e;
    }
    sum = quad_sum(sum);
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    for (int i = l; ok && i < K; i += 4) xr[i] *= inv;
    __syncthreads();
    block_out(xs, yg, n);
    tail_out(xs, yg, n);
}

// dS = P (dP - sum_j P dP); ds may alias dp.
__global__ __launch_bounds__(256) void softmax_bwd_blocks(const float *p, const float *dp, float *ds,
                                                          int64_t rows, int K) {
    __shared__ __align__(16) float ps[kRowsPerBlock * kRowMax];
    __shared__ __align__(16) float gs[kRowsPerBlock * kRowMax];
    const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock;
    const int nr = (int)(rows - row0 < kRowsPerBlock ? rows - row0 : kRowsPerBlock);
    const int n = nr * K;
    block_in(p + row0 * K, ps, n);
    block_in(dp + row0 * K, gs, n);
    tail_in(p + row0 * K, ps, n);
    tail_in(dp + row0 * K, gs, n);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int r = threadIdx.x >> 2, l = threadIdx.x & 3;
    const bool ok = r < nr;
    const float *pr = ps + r * K;
    float *gr = gs + r * K;
    float sum = 0.f;
    for (int i = l; ok && i < K; i += 4) sum += pr[i] * gr[i];
    sum = quad_sum(sum);
    for (int i = l; ok && i < K; i += 4) gr[i] = pr[i] * (gr[i] - sum);
    __syncthreads();
    block_out(gs, ds + row0 * K, n);
    tail_out(gs, ds + row0 * K, n);
}

// Rows longer than kRowMax: sixteen lanes per row, sixteen rows per
// workgroup, each row read in passes.
__device__ __forceinline__ float row_max16(float v) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
    return v;
}

__global__ __launch_bounds__(256) void softmax_rows(const float *x, float *y, int64_t rows, int K) {
    const int64_t row = blockIdx.x * 16ll + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool ok = row < rows;   // every lane takes part in the shuffles
    const float *xr = x + (ok ? row : 0) * K;
    float *yr = y + (ok ? row : 0) * K;
    float m = -INFINITY;
    for (int idx = l; ok && idx < K; idx += 16) m = fmaxf(m, xr[idx]);
    m = row_max16(m);
    if (m == -INFINITY) m = 0.f;   // every entry masked out: zero weights
    float s = 0.f;
    for (int idx = l; ok && idx < K; idx += 16) s += __expf(xr[idx] - m);
    s = row_sum16(s);
    const float inv = s > 0.f ? 1.f / s : 0.f;
    for (int idx = l; ok && idx < K; idx += 16) yr[idx] = __expf(xr[idx] - m) * inv;
}

__global__ __launch_bounds__(256) void softmax_bwd_rows(const float *p, const float *dp, float *ds,
                                                        int64_t rows, int K) {
    const int64_t row = blockIdx.x * 16ll + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool ok = row < rows;
    const int64_t off = (ok ? row : 0) * K;
    float s = 0.f;
    for (int idx = l; ok && idx < K; idx += 16) s += p[off + idx] * dp[off + idx];
    s = row_sum16(s);
    for (int idx = l; ok && idx < K; idx += 16) ds[off + idx] = p[off + idx] * (dp[off + idx] - s);
}

// ----------------------------------------------------------------------------
// Launchers (host). Each returns after enqueueing on the stream.

#define NA_FOR_D(D, CALL)                      \
    switch (D) {                               \
    case 16: { constexpr int kD = 16; CALL; } break; \
    case 32: { constexpr int kD = 32; CALL; } break; \
    default: { constexpr int kD = 64; CALL; } break; \
    }

na_status run_qk(const UProb &q, const float *a, const float *b, float alpha, const float *rpb,
                 const uint8_t *mask, float *attn, hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if (nu::fast_qk(q.g, q.bh, q.D, a, b, alpha, rpb, mask, q.heads, attn, st)) return launched();
    const int64_t total = q.units * q.g.K;
    NA_FOR_D(q.D, hipLaunchKernelGGL(qk_plain<kD>, dim3(grid_for(total, 256)), dim3(256), 0, st,
                                     q.g, a, b, alpha, rpb, q.heads, mask, attn, total));
    return launched();
}

int rpb_size(const UProb &q) {
    return (2 * q.g.ker[0] - 1) * (2 * q.g.ker[1] - 1) * (2 * q.g.ker[2] - 1);
}

int64_t rpb_chunks(const UProb &q) { return (q.g.tokens + kRpbChunk - 1) / kRpbChunk; }

size_t rpb_workspace(const UProb &q) {
    return (size_t)(q.bh * rpb_chunks(q) * rpb_size(q)) * sizeof(float);
}

na_status run_rpb_grad(const UProb &q, const float *ds, float *drpb, void *ws, size_t ws_bytes,
                       hipStream_t st) {
    const int R = rpb_size(q);
    if (R > 256 * kRpbPerThread || q.g.K > kRpbMaxK) return NA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < rpb_workspace(q)) return NA_ERR_WORKSPACE;
    const int64_t blocks = q.bh * rpb_chunks(q);
    if (blocks > INT32_MAX) return NA_ERR_UNSUPPORTED;
    float *partial = static_cast<float *>(ws);
    hipLaunchKernelGGL(rpb_partial_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q.g, ds,
                       partial, (int)rpb_chunks(q));
    hipLaunchKernelGGL(rpb_reduce_kernel, dim3((unsigned)(q.heads * ((R + 15) / 16))), dim3(256), 0,
                       st, partial, drpb, (int)(q.bh / q.heads), (int)q.heads, (int)rpb_chunks(q), R);
    return launched();
}

// Scores and the window softmax: one kernel where the whole window of a query
// fits the lane's registers (single-plane grids), else scores then softmax.
na_status run_qk_softmax(const UProb &q, const float *a, const float *b, float alpha,
                         const float *rpb, const uint8_t *mask, float *probs, hipStream_t st);
na_status run_softmax(const UProb &q, const float *x, float *y, hipStream_t st);
na_status run_softmax_bwd(const UProb &q, const float *p, const float *dp, float *ds,
                          hipStream_t st);

na_status run_qk_softmax(const UProb &q, const float *a, const float *b, float alpha,
                         const float *rpb, const uint8_t *mask, float *probs, hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if (nu::fast_qk_softmax(q.g, q.bh, q.D, a, b, alpha, rpb, mask, (int)q.heads, probs, st))
        return launched();
    na_status s = run_qk(q, a, b, alpha, rpb, mask, probs, st);
    return s != NA_OK ? s : run_softmax(q, probs, probs, st);
}

// AGRAD and the softmax backward: one kernel on single-plane grids, else dP then dS.
na_status run_qk_softmax_bwd(const UProb &q, const float *dout, const float *v,
                             const float *probs, float *dscores, hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if (nu::fast_qk_softmax_bwd(q.g, q.bh, q.D, dout, v, probs, dscores, st)) return launched();
    na_status s = run_qk(q, dout, v, 1.f, nullptr, nullptr, dscores, st);
    return s != NA_OK ? s : run_softmax_bwd(q, probs, dscores, dscores, st);
}

na_status run_av(const UProb &q, const float *attn, const float *b, float alpha, float *out,
                 hipStream_t st) {
    if (nu::fast_av(q.g, q.bh, q.D, attn, b, alpha, out, st)) return launched();
    const int64_t total = q.units * (q.D / 4);
    NA_FOR_D(q.D, hipLaunchKernelGGL(av_plain<kD>, dim3(grid_for(total, 256)), dim3(256), 0, st,
                                     q.g, attn, b, alpha, out, total));
    return launched();
}

na_status run_av_inverse(const UProb &q, const float *attn, const float *a, float alpha,
                         float *out, hipStream_t st) {
    if (nu::fast_av_inverse(q.g, q.bh, q.D, attn, a, alpha, out, st)) return launched();
    const int64_t total = q.units * (q.D / 4);
    NA_FOR_D(q.D, hipLaunchKernelGGL(av_inverse_plain<kD>, dim3(grid_for(total, 256)), dim3(256),
                                     0, st, q.g, attn, a, alpha, out, total));
    return launched();
}

na_status run_softmax(const UProb &q, const float *x, float *y, hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if (q.g.K <= kRowMax) {
        const int64_t blocks = (q.units + kRowsPerBlock - 1) / kRowsPerBlock;
        if (blocks > INT32_MAX) return NA_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(softmax_blocks, dim3((unsigned)blocks), dim3(256), 0, st, x, y, q.units,
                           q.g.K);
    } else {
        const int64_t blocks = (q.units + 15) / 16;
        if (blocks > INT32_MAX) return NA_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(softmax_rows, dim3((unsigned)blocks), dim3(256), 0, st, x, y, q.units,
                           q.g.K);
    }
    return launched();
}

na_status run_softmax_bwd(const UProb &q, const float *p, const float *dp, float *ds,
                          hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if (q.g.K <= kRowMax) {
        const int64_t blocks = (q.units + kRowsPerBlock - 1) / kRowsPerBlock;
        if (blocks > INT32_MAX) return NA_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(softmax_bwd_blocks, dim3((unsigned)blocks), dim3(256), 0, st, p, dp, ds,
                           q.units, q.g.K);
    } else {
        const int64_t blocks = (q.units + 15) / 16;
        if (blocks > INT32_MAX) return NA_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(softmax_bwd_rows, dim3((unsigned)blocks), dim3(256), 0, st, p, dp, ds,
                           q.units, q.g.K);
    }
    return launched();
}

na_status check_ptrs(std::initializer_list<const void *> ps) {
    for (const void *p : ps)
        if (!p || !aligned16(p)) return NA_ERR_INVALID_ARG;
    return NA_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

na_status na_qk(const na_problem *p, const void *a, const void *b, double alpha, const float *rpb,
                const uint8_t *mask, float *attn, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q);
    if (s != NA_OK) return s;
    if (!std::isfinite(alpha)) return NA_ERR_INVALID_ARG;
    if ((s = check_ptrs({a, b, attn})) != NA_OK) return s;
    if (rpb && !aligned16(rpb)) return NA_ERR_INVALID_ARG;
    return run_qk(q, (const float *)a, (const float *)b, (float)alpha, rpb, mask, attn,
                  as_stream(hip_stream));
}

na_status na_qk_softmax(const na_problem *p, const void *a, const void *b, double alpha,
                        const float *rpb, const uint8_t *mask, float *probs, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q);
    if (s != NA_OK) return s;
    if (!std::isfinite(alpha)) return NA_ERR_INVALID_ARG;
    if ((s = check_ptrs({a, b, probs})) != NA_OK) return s;
    if (rpb && !aligned16(rpb)) return NA_ERR_INVALID_ARG;
    return run_qk_softmax(q, (const float *)a, (const float *)b, (float)alpha, rpb, mask, probs,
                          as_stream(hip_stream));
}

na_status na_qk_softmax_bwd(const na_problem *p, const void *dout, const void *v,
                            const float *probs, float *dscores, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({dout, v, probs, dscores})) != NA_OK) return s;
    return run_qk_softmax_bwd(q, (const float *)dout, (const float *)v, probs, dscores,
                              as_stream(hip_stream));
}

size_t na_rpb_grad_workspace_bytes(const na_problem *p) {
    UProb q;
    if (uvalidate(p, &q, false) != NA_OK) return 0;
    return rpb_workspace(q);
}

na_status na_rpb_grad(const na_problem *p, const float *dscores, float *drpb, void *workspace,
                      size_t workspace_bytes, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q, false);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({dscores, drpb})) != NA_OK) return s;
    if (q.units == 0) return NA_OK;
    return run_rpb_grad(q, dscores, drpb, workspace, workspace_bytes, as_stream(hip_stream));
}

na_status na_av(const na_problem *p, const float *attn, const void *b, double alpha, void *out,
                void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q);
    if (s != NA_OK) return s;
    if (!std::isfinite(alpha)) return NA_ERR_INVALID_ARG;
    if ((s = check_ptrs({attn, b, out})) != NA_OK) return s;
    return run_av(q, attn, (const float *)b, (float)alpha, (float *)out, as_stream(hip_stream));
}

na_status na_av_inverse(const na_problem *p, const float *attn, const void *a, double alpha,
                        void *out, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q);
    if (s != NA_OK) return s;
    if (!std::isfinite(alpha)) return NA_ERR_INVALID_ARG;
    if ((s = check_ptrs({attn, a, out})) != NA_OK) return s;
    return run_av_inverse(q, attn, (const float *)a, (float)alpha, (float *)out,
                          as_stream(hip_stream));
}

na_status na_softmax(const na_problem *p, const float *attn, float *probs, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q, false);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({attn, probs})) != NA_OK) return s;
    return run_softmax(q, attn, probs, as_stream(hip_stream));
}

na_status na_softmax_bwd(const na_problem *p, const float *probs, const float *dprobs,
                         float *dscores, void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q, false);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({probs, dprobs, dscores})) != NA_OK) return s;
    return run_softmax_bwd(q, probs, dprobs, dscores, as_stream(hip_stream));
}

na_status na_unfused_fwd(const na_problem *p, const void *q, const void *k, const void *v,
                         const float *rpb, const uint8_t *mask, float *probs, void *out,
                         void *hip_stream) {
    UProb u;
    na_status s = uvalidate(p, &u);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({q, k, v, probs, out})) != NA_OK) return s;
    if (rpb && !aligned16(rpb)) return NA_ERR_INVALID_ARG;
    const hipStream_t st = as_stream(hip_stream);
    if ((s = run_qk_softmax(u, (const float *)q, (const float *)k, (float)p->scale, rpb, mask,
                            probs, st)) != NA_OK)
        return s;
    return run_av(u, probs, (const float *)v, 1.f, (float *)out, st);
}

na_status na_unfused_bwd(const na_problem *p, const void *q, const void *k, const void *v,
                         const float *probs, const void *dout, float *dscores, void *dq, void *dk,
                         void *dv, float *drpb, void *workspace, size_t workspace_bytes,
                         void *hip_stream) {
    UProb u;
    na_status s = uvalidate(p, &u);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({q, k, v, probs, dout, dscores, dq, dk, dv})) != NA_OK) return s;
    if (drpb) {
        if (!aligned16(drpb)) return NA_ERR_INVALID_ARG;
        if (rpb_size(u) > 256 * kRpbPerThread || u.g.K > kRpbMaxK) return NA_ERR_UNSUPPORTED;
        if (!workspace || workspace_bytes < rpb_workspace(u)) return NA_ERR_WORKSPACE;
    }
    const hipStream_t st = as_stream(hip_stream);
    const float scale = (float)p->scale;
    // AGRAD and the softmax backward: dS = P (dP - rowsum(P dP)), dP = dout . v over
    // the window; VGRAD: dv = inverse sum of P dout; the bias gradient sums dS
    if ((s = run_qk_softmax_bwd(u, (const float *)dout, (const float *)v, probs, dscores, st)) !=
        NA_OK)
        return s;
    if ((s = run_av_inverse(u, probs, (const float *)dout, 1.f, (float *)dv, st)) != NA_OK)
        return s;
    if (drpb && (s = run_rpb_grad(u, dscores, drpb, workspace, workspace_bytes, st)) != NA_OK)
        return s;
    // QGRAD and KGRAD
    if ((s = run_av(u, dscores, (const float *)k, scale, (float *)dq, st)) != NA_OK) return s;
    return run_av_inverse(u, dscores, (const float *)q, scale, (float *)dk, st);
}

}  // extern "C"
