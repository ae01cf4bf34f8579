// na_kernels.hpp -- neighborhood attention forward and backward kernels for
// gfx950 (wave64, fp32 MFMA 4x4x1).
//
// Work decomposition. Every kernel runs independent waves; a wave owns a
// 1x8x8 tile of one residue class of one (batch, head), split into sixteen
// 1x2x2 patches, one per 4-lane MFMA block. Inside a block each lane owns one
// point of the patch (a query in the forward and dq kernels, a key in the dk/dv
// kernel), and the block walks the other side's points in 1x2x2 patches that
// cover the union of what its four points need. That union is at most one
// position longer per axis than a single window, so the contraction over a
// patch pair wastes little: a 9x9 window is covered by 5x5 patches of 4 keys
// (100 computed vs 81 needed scores), a 3x5x5 window by 3x3x3 patches (108 vs
// 75). Scores outside a point's window are masked by index arithmetic on the
// window starts, never by padding (the NATTEN maintainer names software
// predication of these bounds as the main overhead of 2D/3D fused kernels; here
// it costs a few integer compares per score).
//
// Softmax. Scores are kept in log2 units (q is pre-multiplied by
// scale * log2(e)) so exp2 is a single hardware instruction; each lane keeps
// the running maximum and sum of its own query, so no cross-lane reduction is
// needed anywhere in the softmax.
//
// Backward (query-parallel + key-parallel gather): the dq kernel recomputes
// P = exp2(S - lse) from the saved logsumexp, forms delta = <dout, out> for its
// own queries (NATTEN's ComputeDelta, fused here), dS = P (dP - delta) and
// dq. The dk/dv kernel walks each key's inverse neighborhood (a contiguous
// range per axis, closed form in na_index.hpp) and writes dk, dv exactly once,
// with no atomics.
#pragma once

#include "na_common.hpp"

namespace na {

struct FwdArgs {
    Geometry g;
    const void *q, *k, *v;
    void *out;
    float *lse;
    float qscale;  // scale * log2(e)
};

struct BwdArgs {
    Geometry g;
    const void *q, *k, *v, *out, *dout;
    const float *lse;
    float *delta;
    void *dq, *dk, *dv;
    float *dq_acc;  // KV-parallel variant only
    float qscale;   // scale * log2(e)
    float scale;
};

// Per-lane view of a patch-owning lane: the patch first point, the lane's
// own point, and whether the point is inside the class grid.
struct LanePoint {
    int f[3];   // first point of the lane's patch (clamped into the grid)
    int p[3];   // the lane's own point (clamped into the grid)
    bool active;
};

__device__ __forceinline__ LanePoint lane_point(const WaveCtx &w, int grp, int c) {
    LanePoint lp;
    int f[3] = {w.o[0], w.o[1] + 2 * (grp >> 2), w.o[2] + 2 * (grp & 3)};
    int p[3];
    patch_point(f, c, p);
    lp.active = p[0] < w.n[0] && p[1] < w.n[1] && p[2] < w.n[2];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        lp.f[a] = imin(f[a], w.n[a] - 1);
        lp.p[a] = imin(p[a], w.n[a] - 1);
    }
    return lp;
}

// Number of 1x2x2 patches per axis that cover the union of the windows of a
// patch of queries: the union is at most k + patch - 1 long.
__device__ __forceinline__ void key_patch_counts(const WaveCtx &w, int (&cnt)[3]) {
#pragma unroll
    for (int a = 0; a < 3; ++a) cnt[a] = (w.k[a] + kPatch[a] - 1 + kPatch[a] - 1) / kPatch[a];
}

// ============================================================================
// Forward: out, lse.
template <typename T, int D>
__global__ void __launch_bounds__(256) fwd_kernel(FwdArgs a) {
    constexpr int G = D / 4;
    const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= a.g.n_waves) return;
    WaveCtx w;
    if (!decode_wave(a.g, wave, w)) return;
    const int lane = threadIdx.x & 63, grp = lane >> 2, c = lane & 3;
    const LanePoint lp = lane_point(w, grp, c);

    const T *Q = static_cast<const T *>(a.q);
    const T *K = static_cast<const T *>(a.k);
    const T *V = static_cast<const T *>(a.v);

    // window of this lane's query, relative to the union start of its patch
    int us[3], off[3], cnt[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        us[x] = window_start(lp.f[x], w.n[x], w.k[x]);
        off[x] = window_start(lp.p[x], w.n[x], w.k[x]) - us[x];
    }
    key_patch_counts(w, cnt);

    float qr[D];
    load_row<T, D>(Q + elem_off(w, lp.p), qr);
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] *= a.qscale;

    float m = -1e30f, l = 0.f;
    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    for (int ct = 0; ct < cnt[0]; ++ct) {
        for (int ch = 0; ch < cnt[1]; ++ch) {
            for (int cw = 0; cw < cnt[2]; ++cw) {
                const int kb[3] = {us[0] + ct * kPatch[0], us[1] + ch * kPatch[1],
                                   us[2] + cw * kPatch[2]};
                // S_b[i][c] = <k_i, q_c>: this lane supplies key c of the patch
                int kc[3];
                patch_point(kb, c, kc);
#pragma unroll
                for (int x = 0; x < 3; ++x) kc[x] = imin(kc[x], w.n[x] - 1);
                float kr[D];
                load_row<T, D>(K + elem_off(w, kc), kr);
                f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < D; ++d) s = mfma4(kr[d], qr[d], s);

                // mask keys outside this query's window
                float sv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rel[3] = {ct * kPatch[0], ch * kPatch[1] + (i >> 1),
                                        cw * kPatch[2] + (i & 1)};
                    bool ok = true;
#pragma unroll
                    for (int x = 0; x < 3; ++x) ok = ok && rel[x] >= off[x] && rel[x] < off[x] + w.k[x];
                    sv[i] = ok ? s[i] : -INFINITY;
                }
                const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                const float mn = fmaxf(m, mx);
                const float alpha = exp2f(m - mn);
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = exp2f(sv[i] - mn);
                l = l * alpha + (p[0] + p[1]) + (p[2] + p[3]);
                m = mn;
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] *= alpha;

                // O_b[i][c] += v_kappa[i*G + g] * P[c][kappa]: this lane supplies
                // the d-chunk c of every key of the patch
#pragma unroll
                for (int kap = 0; kap < 4; ++kap) {
                    int vc[3];
                    patch_point(kb, kap, vc);
#pragma unroll
                    for (int x = 0; x < 3; ++x) vc[x] = imin(vc[x], w.n[x] - 1);
                    float vr[G];
                    load_row<T, G>(V + elem_off(w, vc) + c * G, vr);
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g] = mfma4(vr[g], p[kap], acc[g]);
                }
            }
        }
    }

    if (!lp.active) return;
    const float inv = 1.f / l;
    T *O = static_cast<T *>(a.out) + elem_off(w, lp.p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g] = acc[g][i] * inv;
#pragma unroll
        for (int g = 0; g < G; g += 4) Io<T>::store4(O + i * G + g, o + g);
    }
    a.lse[row_off(w, lp.p)] = (m + __log2f(l)) * kLn2;
}

// ============================================================================
// Backward, query side: delta and dq.
template <typename T, int D>
__global__ void __launch_bounds__(256) dq_kernel(BwdArgs a) {
    constexpr int G = D / 4;
    const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= a.g.n_waves) return;
    WaveCtx w;
    if (!decode_wave(a.g, wave, w)) return;
    const int lane = threadIdx.x & 63, grp = lane >> 2, c = lane & 3;
    const LanePoint lp = lane_point(w, grp, c);

    const T *Q = static_cast<const T *>(a.q);
    const T *K = static_cast<const T *>(a.k);
    const T *V = static_cast<const T *>(a.v);

    int us[3], off[3], cnt[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        us[x] = window_start(lp.f[x], w.n[x], w.k[x]);
        off[x] = window_start(lp.p[x], w.n[x], w.k[x]) - us[x];
    }
    key_patch_counts(w, cnt);

    const int64_t qo = elem_off(w, lp.p);
    float qr[D], dor[D];
    load_row<T, D>(Q + qo, qr);
    load_row<T, D>(static_cast<const T *>(a.dout) + qo, dor);
    float delta = 0.f;
    {
        float orow[D];
        load_row<T, D>(static_cast<const T *>(a.out) + qo, orow);
#pragma unroll
        for (int d = 0; d < D; ++d) delta += dor[d] * orow[d];
    }
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] *= a.qscale;
    const float lse2 = a.lse[row_off(w, lp.p)] * kLog2e;

    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    for (int ct = 0; ct < cnt[0]; ++ct) {
        for (int ch = 0; ch < cnt[1]; ++ch) {
            for (int cw = 0; cw < cnt[2]; ++cw) {
                const int kb[3] = {us[0] + ct * kPatch[0], us[1] + ch * kPatch[1],
                                   us[2] + cw * kPatch[2]};
                int kc[3];
                patch_point(kb, c, kc);
#pragma unroll
                for (int x = 0; x < 3; ++x) kc[x] = imin(kc[x], w.n[x] - 1);
                const int64_t ko = elem_off(w, kc);
                float kr[D], vr[D];
                load_row<T, D>(K + ko, kr);
                load_row<T, D>(V + ko, vr);
                f4 s = f4{0.f, 0.f, 0.f, 0.f}, dp = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < D; ++d) s = mfma4(kr[d], qr[d], s);
#pragma unroll
                for (int d = 0; d < D; ++d) dp = mfma4(vr[d], dor[d], dp);

                float ds[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rel[3] = {ct * kPatch[0], ch * kPatch[1] + (i >> 1),
                                        cw * kPatch[2] + (i & 1)};
                    bool ok = true;
#pragma unroll
                    for (int x = 0; x < 3; ++x) ok = ok && rel[x] >= off[x] && rel[x] < off[x] + w.k[x];
                    const float p = ok ? exp2f(s[i] - lse2) : 0.f;
                    ds[i] = p * (dp[i] - delta);
                }
                // dQ_b[i][c] += k_kappa[i*G + g] * dS[c][kappa]
#pragma unroll
                for (int kap = 0; kap < 4; ++kap) {
                    int vc[3];
                    patch_point(kb, kap, vc);
#pragma unroll
                    for (int x = 0; x < 3; ++x) vc[x] = imin(vc[x], w.n[x] - 1);
                    float kd[G];
                    load_row<T, G>(K + elem_off(w, vc) + c * G, kd);
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g] = mfma4(kd[g], ds[kap], acc[g]);
                }
            }
        }
    }

    if (!lp.active) return;
    a.delta[row_off(w, lp.p)] = delta;
    T *DQ = static_cast<T *>(a.dq) + qo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g] = acc[g][i] * a.scale;
#pragma unroll
        for (int g = 0; g < G; g += 4) Io<T>::store4(DQ + i * G + g, o + g);
    }
}

// ============================================================================
// Backward, key side: dk and dv by inverse-neighborhood gather. With
// KVPAR the same pass also produces each query's dq contributions from this
// key patch and adds them into the fp32 accumulator dq_acc.
template <typename T, int D, bool KVPAR>
__global__ void __launch_bounds__(256) dkdv_kernel(BwdArgs a) {
    constexpr int G = D / 4;
    const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= a.g.n_waves) return;
    WaveCtx w;
    if (!decode_wave(a.g, wave, w)) return;
    const int lane = threadIdx.x & 63, grp = lane >> 2, c = lane & 3;
    const LanePoint lp = lane_point(w, grp, c);  // here: this lane's key

    const T *Q = static_cast<const T *>(a.q);
    const T *K = static_cast<const T *>(a.k);
    const T *V = static_cast<const T *>(a.v);
    const T *DO = static_cast<const T *>(a.dout);

    // queries of the patch's inverse neighborhood, and of this lane's key
    int lo[3], ilo[3], ihi[3], cnt[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        int last = imin(lp.f[x] + kPatch[x] - 1, w.n[x] - 1);
        lo[x] = inverse_first(lp.f[x], w.n[x], w.k[x]);
        int hi = inverse_last(last, w.n[x], w.k[x]);
        ilo[x] = inverse_first(lp.p[x], w.n[x], w.k[x]);
        ihi[x] = inverse_last(lp.p[x], w.n[x], w.k[x]);
        cnt[x] = wave_max((hi - lo[x] + kPatch[x]) / kPatch[x]);
    }

    const int64_t ko = elem_off(w, lp.p);
    float kr[D], vr[D];
    load_row<T, D>(K + ko, kr);
    load_row<T, D>(V + ko, vr);
#pragma unroll
    for (int d = 0; d < D; ++d) kr[d] *= a.qscale;

    f4 dk[G], dv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        dk[g] = f4{0.f, 0.f, 0.f, 0.f};
        dv[g] = f4{0.f, 0.f, 0.f, 0.f};
    }

    for (int ct = 0; ct < cnt[0]; ++ct) {
        for (int ch = 0; ch < cnt[1]; ++ch) {
            for (int cw = 0; cw < cnt[2]; ++cw) {
                const int qb[3] = {lo[0] + ct * kPatch[0], lo[1] + ch * kPatch[1],
                                   lo[2] + cw * kPatch[2]};
                // S_b[i][c] = <q_i, k_c>: this lane supplies query c of the patch
                int qc[3];
                patch_point(qb, c, qc);
#pragma unroll
                for (int x = 0; x < 3; ++x) qc[x] = imin(qc[x], w.n[x] - 1);
                const int64_t qo = elem_off(w, qc);
                float qr[D], dor[D];
                load_row<T, D>(Q + qo, qr);
                load_row<T, D>(DO + qo, dor);
                f4 s = f4{0.f, 0.f, 0.f, 0.f}, dp = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < D; ++d) s = mfma4(qr[d], kr[d], s);
#pragma unroll
                for (int d = 0; d < D; ++d) dp = mfma4(dor[d], vr[d], dp);

                float p[4], ds[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int qi[3];
                    patch_point(qb, i, qi);
                    bool ok = true;
#pragma unroll
                    for (int x = 0; x < 3; ++x) ok = ok && qi[x] >= ilo[x] && qi[x] <= ihi[x];
                    int qcl[3];
#pragma unroll
                    for (int x = 0; x < 3; ++x) qcl[x] = imin(qi[x], w.n[x] - 1);
                    const int64_t ro = row_off(w, qcl);
                    const float l2 = a.lse[ro] * kLog2e;
                    const float dl = a.delta[ro];
                    p[i] = ok ? exp2f(s[i] - l2) : 0.f;
                    ds[i] = p[i] * (dp[i] - dl);
                }
                // dV_b[i][c] += dout_kappa[i*G + g] * P[kappa][c];
                // dK_b[i][c] += q_kappa[i*G + g] * dS[kappa][c]
#pragma unroll
                for (int kap = 0; kap < 4; ++kap) {
                    int qi[3];
                    patch_point(qb, kap, qi);
#pragma unroll
                    for (int x = 0; x < 3; ++x) qi[x] = imin(qi[x], w.n[x] - 1);
                    const int64_t o2 = elem_off(w, qi) + c * G;
                    float dod[G], qd[G];
                    load_row<T, G>(DO + o2, dod);
                    load_row<T, G>(Q + o2, qd);
#pragma unroll
                    for (int g = 0; g < G; ++g) dv[g] = mfma4(dod[g], p[kap], dv[g]);
#pragma unroll
                    for (int g = 0; g < G; ++g) dk[g] = mfma4(qd[g], ds[kap], dk[g]);
                }

                if constexpr (KVPAR) {
                    // A lane whose key lies past the grid edge was clamped onto a
                    // real key; it must not add that key's contribution twice.
                    float dsk[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) dsk[i] = lp.active ? ds[i] : 0.f;
                    // transpose dS inside the block: lane 4b+c gets
                    // tr[j] = dS[query c][key j] (held by lane 4b+j, register c)
                    float tr[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int src = (lane & ~3) | j;
                        float x0 = __shfl(dsk[0], src), x1 = __shfl(dsk[1], src);
                        float x2 = __shfl(dsk[2], src), x3 = __shfl(dsk[3], src);
                        tr[j] = c == 0 ? x0 : c == 1 ? x1 : c == 2 ? x2 : x3;
                    }
                    // dQ_b[i][c] = sum_j k_j[i*G + g] * dS[c][j]
                    f4 dq[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) dq[g] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        int kj[3];
                        patch_point(lp.f, j, kj);
#pragma unroll
                        for (int x = 0; x < 3; ++x) kj[x] = imin(kj[x], w.n[x] - 1);
                        float kd[G];
                        load_row<T, G>(K + elem_off(w, kj) + c * G, kd);
#pragma unroll
                        for (int g = 0; g < G; ++g) dq[g] = mfma4(kd[g], tr[j], dq[g]);
                    }
                    int qq[3];
                    patch_point(qb, c, qq);
                    if (qq[0] < w.n[0] && qq[1] < w.n[1] && qq[2] < w.n[2]) {
                        float *acc = a.dq_acc + elem_off(w, qq);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int g = 0; g < G; ++g) atomicAdd(acc + i * G + g, dq[g][i]);
                    }
                }
            }
        }
    }

    if (!lp.active) return;
    T *DK = static_cast<T *>(a.dk) + ko;
    T *DV = static_cast<T *>(a.dv) + ko;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float ok_[G], ov[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ok_[g] = dk[g][i] * a.scale;
            ov[g] = dv[g][i];
        }
#pragma unroll
        for (int g = 0; g < G; g += 4) {
            Io<T>::store4(DK + i * G + g, ok_ + g);
            Io<T>::store4(DV + i * G + g, ov + g);
        }
    }
}

// ============================================================================
// Elementwise helpers of the KV-parallel backward.

// delta[row] = <dout_row, out_row>, one thread per (token, head) row.
template <typename T, int D>
__global__ void __launch_bounds__(256) delta_kernel(const T *out, const T *dout, float *delta,
                                                    int64_t rows) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    float o[D], d_[D];
    load_row<T, D>(out + r * D, o);
    load_row<T, D>(dout + r * D, d_);
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s += o[d] * d_[d];
    delta[r] = s;
}

// Zero n floats (n a multiple of 4), four per thread.
__global__ void __launch_bounds__(256) zero_kernel(float *p, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4) reinterpret_cast<float4 *>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// dq = scale * dq_acc, cast to the tensor type, four elements per thread.
template <typename T>
__global__ void __launch_bounds__(256) dq_finalize_kernel(const float *acc, T *dq, float scale,
                                                          int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float v[4];
    Io<float>::load4(acc + 4 * i, v);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] *= scale;
    Io<T>::store4(dq + 4 * i, v);
}

}  // namespace na
