// na_api.hip -- the C ABI of libna (declared in include/na.h): problem
// validation on the host, workspace sizing, and kernel launches on the
// caller's stream. No allocation, no synchronization, no global state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "na.h"
#include "na_kernels.hpp"

namespace {

using na::bf16;

constexpr int kThreads = 256;

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

na_status validate(const na_problem *p, Prob *out) {
    if (!p) return NA_ERR_INVALID_ARG;
    if (p->ndim != 2 && p->ndim != 3) return NA_ERR_INVALID_ARG;
    if (p->dtype != NA_F32 && p->dtype != NA_BF16) return NA_ERR_INVALID_ARG;
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
    q.batch = p->batch;
    q.heads = p->heads;
    q.head_dim = p->head_dim;
    q.tokens = tokens;
    q.rows = p->batch * tokens * p->heads;
    q.dtype = (na_dtype)p->dtype;
    q.scale = (float)p->scale;
    if (out) *out = q;
    return NA_OK;
}

// Wave tiling of the class grids; false when the wave count overflows int32.
bool geometry(const Prob &q, na::Geometry *g) {
    int64_t n_waves = q.batch * q.heads;
    int nres = 1;
    for (int a = 0; a < 3; ++a) {
        g->ext[a] = q.ext[a];
        g->ker[a] = q.ker[a];
        g->dil[a] = q.dil[a];
        const int nmax = na::class_size(q.ext[a], q.dil[a], 0);
        g->tiles[a] = (nmax + na::kWaveTile[a] - 1) / na::kWaveTile[a];
        n_waves *= g->tiles[a];
        nres *= q.dil[a];
    }
    n_waves *= nres;
    if (n_waves > INT32_MAX - 64) return false;
    g->heads = (int)q.heads;
    g->batch = (int)q.batch;
    g->head_dim = (int)q.head_dim;
    g->nres = nres;
    g->n_waves = (int)n_waves;
    return true;
}

dim3 wave_grid(const na::Geometry &g) {
    return dim3((unsigned)((g.n_waves + na::kWavesPerBlock - 1) / na::kWavesPerBlock));
}

dim3 flat_grid(int64_t n) { return dim3((unsigned)((n + kThreads - 1) / kThreads)); }

na_status launched() { return hipGetLastError() == hipSuccess ? NA_OK : NA_ERR_HIP; }

template <typename T, int D>
na_status run_fwd(const na::FwdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((na::fwd_kernel<T, D>), wave_grid(a.g), dim3(kThreads), 0, s, a);
    return launched();
}

// Which kernels of the backward a call runs.
enum Phase { kPhaseDq = 1, kPhaseDkdv = 2, kPhaseBoth = 3 };

template <typename T, int D>
na_status run_bwd(const na::BwdArgs &a, const Prob &q, int32_t variant, int phases, hipStream_t s) {
    if (variant == NA_BWD_GATHER) {
        if (phases & kPhaseDq) {
            hipLaunchKernelGGL((na::dq_kernel<T, D>), wave_grid(a.g), dim3(kThreads), 0, s, a);
            if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
        }
        if (phases & kPhaseDkdv) {
            hipLaunchKernelGGL((na::dkdv_kernel<T, D, false>), wave_grid(a.g), dim3(kThreads), 0,
                               s, a);
            if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
        }
        return NA_OK;
    }
    const int64_t n4 = q.rows * D / 4;
    hipLaunchKernelGGL((na::delta_kernel<T, D>), flat_grid(q.rows), dim3(kThreads), 0, s,
                       static_cast<const T *>(a.out), static_cast<const T *>(a.dout), a.delta,
                       q.rows);
    if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
    hipLaunchKernelGGL(na::zero_kernel, flat_grid(n4), dim3(kThreads), 0, s, a.dq_acc, n4);
    if (hipGetLastError() != hipSuccess) return NA_ERR_HIP;
    hipLaunchKernelGGL((na::dkdv_kernel<T, D, true>), wave_grid(a.g), dim3(kThreads), 0, s, a);
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
        case NA_ERR_UNSUPPORTED: return "NA_ERR_UNSUPPORTED: no kernel for this head_dim or dtype";
        case NA_ERR_WORKSPACE: return "NA_ERR_WORKSPACE: workspace missing or too small";
        case NA_ERR_HIP: return "NA_ERR_HIP: HIP runtime error at launch";
    }
    return "unknown na_status";
}

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

na_status na_fwd(const na_problem *p, const void *q, const void *k, const void *v, void *out,
                 float *lse, void *hip_stream) {
    Prob pr;
    na_status st = validate(p, &pr);
    if (st != NA_OK) return st;
    if (!q || !k || !v || !out || !lse) return NA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
        return NA_ERR_INVALID_ARG;
    na::FwdArgs a{};
    if (!geometry(pr, &a.g)) return NA_ERR_INVALID_ARG;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.qscale = pr.scale * na::kLog2e;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const bool f32 = pr.dtype == NA_F32;
    switch (pr.head_dim) {
        case 16: return f32 ? run_fwd<float, 16>(a, s) : run_fwd<bf16, 16>(a, s);
        case 32: return f32 ? run_fwd<float, 32>(a, s) : run_fwd<bf16, 32>(a, s);
        case 64: return f32 ? run_fwd<float, 64>(a, s) : run_fwd<bf16, 64>(a, s);
    }
    return NA_ERR_UNSUPPORTED;
}

size_t na_bwd_workspace_bytes(const na_problem *p, int32_t variant) {
    Prob pr;
    if (validate(p, &pr) != NA_OK) return 0;
    const size_t delta = round256((size_t)pr.rows * sizeof(float));
    if (variant == NA_BWD_GATHER) return delta;
    if (variant == NA_BWD_KVPARALLEL)
        return delta + round256((size_t)pr.rows * pr.head_dim * sizeof(float));
    return 0;
}

namespace {

na_status bwd_common(const na_problem *p, const void *q, const void *k, const void *v,
                     const void *out, const void *dout, const float *lse, void *dq, void *dk,
                     void *dv, float *delta, float *dq_acc, int32_t variant, int phases,
                     void *hip_stream) {
    Prob pr;
    na_status st = validate(p, &pr);
    if (st != NA_OK) return st;
    na::BwdArgs a{};
    if (!geometry(pr, &a.g)) return NA_ERR_INVALID_ARG;
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
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const bool f32 = pr.dtype == NA_F32;
    switch (pr.head_dim) {
        case 16:
            return f32 ? run_bwd<float, 16>(a, pr, variant, phases, s)
                       : run_bwd<bf16, 16>(a, pr, variant, phases, s);
        case 32:
            return f32 ? run_bwd<float, 32>(a, pr, variant, phases, s)
                       : run_bwd<bf16, 32>(a, pr, variant, phases, s);
        case 64:
            return f32 ? run_bwd<float, 64>(a, pr, variant, phases, s)
                       : run_bwd<bf16, 64>(a, pr, variant, phases, s);
    }
    return NA_ERR_UNSUPPORTED;
}

bool ptrs_ok(std::initializer_list<const void *> ptrs) {
    for (const void *ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return false;
    return true;
}

}  // namespace

na_status na_bwd(const na_problem *p, const void *q, const void *k, const void *v,
                 const void *out, const void *dout, const float *lse, void *dq, void *dk,
                 void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                 void *hip_stream) {
    na_status st = validate(p, nullptr);
    if (st != NA_OK) return st;
    if (variant != NA_BWD_GATHER && variant != NA_BWD_KVPARALLEL) return NA_ERR_INVALID_ARG;
    if (!ptrs_ok({q, k, v, out, dout, lse, dq, dk, dv})) return NA_ERR_INVALID_ARG;
    const size_t need = na_bwd_workspace_bytes(p, variant);
    if (!workspace || workspace_bytes < need) return NA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return NA_ERR_WORKSPACE;
    Prob pr;
    validate(p, &pr);
    float *delta = static_cast<float *>(workspace);
    float *dq_acc = variant == NA_BWD_KVPARALLEL
                        ? reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                    round256((size_t)pr.rows * sizeof(float)))
                        : nullptr;
    return bwd_common(p, q, k, v, out, dout, lse, dq, dk, dv, delta, dq_acc, variant, kPhaseBoth,
                      hip_stream);
}

na_status na_bwd_dq(const na_problem *p, const void *q, const void *k, const void *v,
                    const void *out, const void *dout, const float *lse, void *dq, float *delta,
                    void *hip_stream) {
    na_status st = validate(p, nullptr);
    if (st != NA_OK) return st;
    if (!ptrs_ok({q, k, v, out, dout, lse, dq, delta})) return NA_ERR_INVALID_ARG;
    return bwd_common(p, q, k, v, out, dout, lse, dq, nullptr, nullptr, delta, nullptr,
                      NA_BWD_GATHER, kPhaseDq, hip_stream);
}

na_status na_bwd_dkdv(const na_problem *p, const void *q, const void *k, const void *v,
                      const void *dout, const float *lse, const float *delta, void *dk, void *dv,
                      void *hip_stream) {
    na_status st = validate(p, nullptr);
    if (st != NA_OK) return st;
    if (!ptrs_ok({q, k, v, dout, lse, delta, dk, dv})) return NA_ERR_INVALID_ARG;
    return bwd_common(p, q, k, v, nullptr, dout, lse, nullptr, dk, dv, const_cast<float *>(delta),
                      nullptr, NA_BWD_GATHER, kPhaseDkdv, hip_stream);
}

}  // extern "C"
