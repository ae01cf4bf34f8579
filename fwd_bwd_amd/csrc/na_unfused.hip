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

template <int D>
__global__ __launch_bounds__(256) void qk_plain(Geo g, const float *__restrict__ a,
                                                const float *__restrict__ b, float alpha,
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
        attn[e] = alpha * s;
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

// ----------------------------------------------------------------------------
// Window softmax and its backward over rows of K entries: sixteen lanes per
// row, sixteen rows per workgroup; a row lives in registers (NR entries per
// lane) when K <= 16 NR, otherwise it is read in passes (NR = 0).

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

template <int NR>
__global__ __launch_bounds__(256) void softmax_rows(const float *__restrict__ x, float *y,
                                                    int64_t rows, int K) {
    const int64_t row = blockIdx.x * 16ll + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool ok = row < rows;   // every lane takes part in the shuffles
    const float *xr = x + (ok ? row : 0) * K;
    float *yr = y + (ok ? row : 0) * K;
    if constexpr (NR > 0) {
        float v[NR];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int idx = l + 16 * i;
            v[i] = (ok && idx < K) ? xr[idx] : -INFINITY;
            m = fmaxf(m, v[i]);
        }
        m = row_max16(m);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            v[i] = (l + 16 * i < K) ? __expf(v[i] - m) : 0.f;
            s += v[i];
        }
        const float inv = 1.f / row_sum16(s);
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (ok && l + 16 * i < K) yr[l + 16 * i] = v[i] * inv;
    } else {
        float m = -INFINITY;
        for (int idx = l; ok && idx < K; idx += 16) m = fmaxf(m, xr[idx]);
        m = row_max16(m);
        float s = 0.f;
        for (int idx = l; ok && idx < K; idx += 16) s += __expf(xr[idx] - m);
        const float inv = 1.f / row_sum16(s);
        for (int idx = l; ok && idx < K; idx += 16) yr[idx] = __expf(xr[idx] - m) * inv;
    }
}

// dS = P (dP - sum_j P dP); ds may alias dp.
template <int NR>
__global__ __launch_bounds__(256) void softmax_bwd_rows(const float *__restrict__ p,
                                                        const float *dp, float *ds, int64_t rows,
                                                        int K) {
    const int64_t row = blockIdx.x * 16ll + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool ok = row < rows;
    const int64_t off = (ok ? row : 0) * K;
    if constexpr (NR > 0) {
        float pv[NR], gv[NR];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int idx = l + 16 * i;
            const bool in = ok && idx < K;
            pv[i] = in ? p[off + idx] : 0.f;
            gv[i] = in ? dp[off + idx] : 0.f;
            s += pv[i] * gv[i];
        }
        s = row_sum16(s);
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (ok && l + 16 * i < K) ds[off + l + 16 * i] = pv[i] * (gv[i] - s);
    } else {
        float s = 0.f;
        for (int idx = l; ok && idx < K; idx += 16) s += p[off + idx] * dp[off + idx];
        s = row_sum16(s);
        for (int idx = l; ok && idx < K; idx += 16) ds[off + idx] = p[off + idx] * (dp[off + idx] - s);
    }
}

// ----------------------------------------------------------------------------
// Launchers (host). Each returns after enqueueing on the stream.

#define NA_FOR_D(D, CALL)                      \
    switch (D) {                               \
    case 16: { constexpr int kD = 16; CALL; } break; \
    case 32: { constexpr int kD = 32; CALL; } break; \
    default: { constexpr int kD = 64; CALL; } break; \
    }

na_status run_qk(const UProb &q, const float *a, const float *b, float alpha, float *attn,
                 hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if (nu::fast_qk(q.g, q.bh, q.D, a, b, alpha, attn, st)) return launched();
    const int64_t total = q.units * q.g.K;
    NA_FOR_D(q.D, hipLaunchKernelGGL(qk_plain<kD>, dim3(grid_for(total, 256)), dim3(256), 0, st,
                                     q.g, a, b, alpha, attn, total));
    return launched();
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

// Launch a row kernel with the smallest register row that holds K entries.
#define NA_LAUNCH_ROWS(KERN, K, rows, st, ...)                                     \
    do {                                                                           \
        const dim3 grid_((unsigned)(((rows) + 15) / 16)), block_(256);             \
        const int need_ = ((K) + 15) / 16;                                         \
        if (need_ <= 2) KERN<2><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K);   \
        else if (need_ <= 4) KERN<4><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K);   \
        else if (need_ <= 6) KERN<6><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K);   \
        else if (need_ <= 8) KERN<8><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K);   \
        else if (need_ <= 12) KERN<12><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K); \
        else if (need_ <= 16) KERN<16><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K); \
        else if (need_ <= 24) KERN<24><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K); \
        else KERN<0><<<grid_, block_, 0, st>>>(__VA_ARGS__, rows, K);             \
    } while (0)

na_status run_softmax(const UProb &q, const float *x, float *y, hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if ((q.units + 15) / 16 > INT32_MAX) return NA_ERR_UNSUPPORTED;
    NA_LAUNCH_ROWS(softmax_rows, q.g.K, q.units, st, x, y);
    return launched();
}

na_status run_softmax_bwd(const UProb &q, const float *p, const float *dp, float *ds,
                          hipStream_t st) {
    if (q.units == 0) return NA_OK;
    if ((q.units + 15) / 16 > INT32_MAX) return NA_ERR_UNSUPPORTED;
    NA_LAUNCH_ROWS(softmax_bwd_rows, q.g.K, q.units, st, p, dp, ds);
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

na_status na_qk(const na_problem *p, const void *a, const void *b, double alpha, float *attn,
                void *hip_stream) {
    UProb q;
    na_status s = uvalidate(p, &q);
    if (s != NA_OK) return s;
    if (!std::isfinite(alpha)) return NA_ERR_INVALID_ARG;
    if ((s = check_ptrs({a, b, attn})) != NA_OK) return s;
    return run_qk(q, (const float *)a, (const float *)b, (float)alpha, attn, as_stream(hip_stream));
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
                         float *probs, void *out, void *hip_stream) {
    UProb u;
    na_status s = uvalidate(p, &u);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({q, k, v, probs, out})) != NA_OK) return s;
    const hipStream_t st = as_stream(hip_stream);
    if ((s = run_qk(u, (const float *)q, (const float *)k, (float)p->scale, probs, st)) != NA_OK)
        return s;
    if ((s = run_softmax(u, probs, probs, st)) != NA_OK) return s;
    return run_av(u, probs, (const float *)v, 1.f, (float *)out, st);
}

na_status na_unfused_bwd(const na_problem *p, const void *q, const void *k, const void *v,
                         const float *probs, const void *dout, float *dscores, void *dq, void *dk,
                         void *dv, void *hip_stream) {
    UProb u;
    na_status s = uvalidate(p, &u);
    if (s != NA_OK) return s;
    if ((s = check_ptrs({q, k, v, probs, dout, dscores, dq, dk, dv})) != NA_OK) return s;
    const hipStream_t st = as_stream(hip_stream);
    const float scale = (float)p->scale;
    // AGRAD: dP = dout . v over the window; VGRAD: dv = inverse sum of P dout
    if ((s = run_qk(u, (const float *)dout, (const float *)v, 1.f, dscores, st)) != NA_OK) return s;
    if ((s = run_av_inverse(u, probs, (const float *)dout, 1.f, (float *)dv, st)) != NA_OK)
        return s;
    // softmax backward in place: dS = P (dP - rowsum(P dP))
    if ((s = run_softmax_bwd(u, probs, dscores, dscores, st)) != NA_OK) return s;
    // QGRAD and KGRAD
    if ((s = run_av(u, dscores, (const float *)k, scale, (float *)dq, st)) != NA_OK) return s;
    return run_av_inverse(u, dscores, (const float *)q, scale, (float *)dk, st);
}

}  // extern "C"
