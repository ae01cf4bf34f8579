/*
 * na_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, brute-force CPU implementation of neighborhood attention (NA)
 * forward and backward, in fp64. It exists to check the GPU library against the
 * definition of the method; it is called only by the tests, by the smoke check
 * and by the CPU-baseline leg of the benchmark. It shares no code, header or
 * table with the GPU library and must never be used as a fallback for it.
 *
 * Source of the method: the NATTEN issue "Backward pass is very slow towards
 * much tokens and large kernels" (SHI-Labs/NATTEN #161).
 *   - Its benchmark script calls na2d / na3d on token-major tensors
 *     [B, (T,) H, W, heads, head_dim] with a per-axis kernel_size and a
 *     dilation argument, and drives the backward with loss = output.sum().
 *   - Its unfused variant spells the computation out: scores over the window
 *     (na*_qk), a softmax over the last (window) axis, then a weighted sum of
 *     the values over the same window (na*_av).
 *   - The maintainer's profiler tables name the backward pieces: the delta
 *     reduction (ComputeDelta), and gradients of the attention weights (AGRAD),
 *     of Q (QGRAD), of K (KGRAD) and of V (VGRAD).
 * The pages never write the window formula down. The reading used here (and
 * listed with the other readings in the design notes): along each axis the
 * window is centered on the query and shifted inward at the borders so it
 * always holds exactly k keys; with dilation d the axis splits into d residue
 * classes and the rule applies inside the query's own class.
 *
 * Everything is accumulated in double. Inputs are double arrays in token-major
 * layout [B, T, H, W, heads, D] (2D problems use T = 1, k_t = 1, d_t = 1).
 * Work can be restricted to a list of selected (b, token, head) units so the
 * full-size workloads can be sampled.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, heads, head_dim;
    int64_t extent[3];   /* T, H, W (T = 1 for 2D) */
    int64_t kernel[3];   /* k_t, k_h, k_w */
    int64_t dilation[3]; /* d_t, d_h, d_w */
    double scale;        /* score multiplier, head_dim^-0.5 by default */
} oracle_problem;

/*
 * First key coordinate of the window of query coordinate x along one axis.
 * The axis holds positions 0..L-1; with dilation d, x only sees positions of
 * its own residue class x mod d, which form a sub-axis of n positions. Inside
 * that sub-axis the window is centered on the query (floor(k/2) keys before
 * it) and pushed back inside the sub-axis when it would stick out, so it
 * always covers k positions. Returned as an absolute coordinate.
 */
int64_t oracle_window_start(int64_t L, int64_t k, int64_t d, int64_t x)
{
    int64_t r = x % d;                 /* residue class of x */
    int64_t i = x / d;                 /* index of x inside its class */
    int64_t n = (L - r + d - 1) / d;   /* positions in the class */
    int64_t s = i - k / 2;             /* centered start */
    if (s < 0) s = 0;                  /* shift inward at the low border */
    if (s + k > n) s = n - k;          /* shift inward at the high border */
    return r + d * s;
}

/* Number of tokens per batch element and offset helpers. */
static int64_t tokens(const oracle_problem *p)
{
    return p->extent[0] * p->extent[1] * p->extent[2];
}

static int64_t token_index(const oracle_problem *p, int64_t t, int64_t y, int64_t x)
{
    return (t * p->extent[1] + y) * p->extent[2] + x;
}

/* Pointer to the D-vector of (b, token, head). */
static const double *vec(const oracle_problem *p, const double *a, int64_t b, int64_t tok, int64_t h)
{
    return a + ((b * tokens(p) + tok) * p->heads + h) * p->head_dim;
}

static double dot(const double *a, const double *b, int64_t n)
{
    double s = 0.0;
    for (int64_t c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

/*
 * The neighborhood of a query token: the Cartesian product of the per-axis
 * windows, exactly k_t * k_h * k_w key tokens, listed in row-major order of
 * the window offsets. Writes the key token indices to keys[].
 */
static int64_t neighborhood(const oracle_problem *p, int64_t tok, int64_t *keys)
{
    int64_t W = p->extent[2], H = p->extent[1];
    int64_t t = tok / (H * W), y = (tok / W) % H, x = tok % W;
    int64_t st = oracle_window_start(p->extent[0], p->kernel[0], p->dilation[0], t);
    int64_t sy = oracle_window_start(p->extent[1], p->kernel[1], p->dilation[1], y);
    int64_t sx = oracle_window_start(p->extent[2], p->kernel[2], p->dilation[2], x);
    int64_t n = 0;
    for (int64_t a = 0; a < p->kernel[0]; ++a)
        for (int64_t b = 0; b < p->kernel[1]; ++b)
            for (int64_t c = 0; c < p->kernel[2]; ++c)
                keys[n++] = token_index(p, st + a * p->dilation[0], sy + b * p->dilation[1],
                                        sx + c * p->dilation[2]);
    return n;
}

static int64_t window_size(const oracle_problem *p)
{
    return p->kernel[0] * p->kernel[1] * p->kernel[2];
}

/*
 * Softmax attention of one query over its neighborhood, straight from the
 * definition: scores s_y = scale * <q, k_y>; lse = log sum_y exp(s_y) computed
 * as m + log sum exp(s_y - m) with m the largest score; weights
 * P_y = exp(s_y - lse); output sum_y P_y v_y.
 * keys[], w[] have room for the window; out may be NULL.
 */
static double attend(const oracle_problem *p, const double *q, const double *k, const double *v,
                     int64_t b, int64_t tok, int64_t h, int64_t *keys, double *w, double *out)
{
    int64_t D = p->head_dim;
    int64_t n = neighborhood(p, tok, keys);
    const double *qv = vec(p, q, b, tok, h);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        w[j] = p->scale * dot(qv, vec(p, k, b, keys[j], h), D);
        if (w[j] > m) m = w[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) sum += exp(w[j] - m);
    double lse = m + log(sum);
    for (int64_t j = 0; j < n; ++j) w[j] = exp(w[j] - lse);
    if (out) {
        for (int64_t c = 0; c < D; ++c) out[c] = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            const double *vv = vec(p, v, b, keys[j], h);
            for (int64_t c = 0; c < D; ++c) out[c] += w[j] * vv[c];
        }
    }
    return lse;
}

/* Decode a flat unit id (b, token, head) in token-major order. */
static void decode_unit(const oracle_problem *p, int64_t u, int64_t *b, int64_t *tok, int64_t *h)
{
    *h = u % p->heads;
    *tok = (u / p->heads) % tokens(p);
    *b = u / (p->heads * tokens(p));
}

/*
 * Forward: for each selected unit (or every unit when sel == NULL) writes the
 * output D-vector and the natural-log logsumexp of the window scores.
 * out is [n_sel, D] and lse is [n_sel] (full tensors when sel == NULL).
 */
void oracle_na_fwd(const oracle_problem *p, const double *q, const double *k, const double *v,
                   int64_t n_sel, const int64_t *sel, double *out, double *lse)
{
    int64_t K = window_size(p), D = p->head_dim;
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
        double *w = (double *)malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t b, tok, h;
            decode_unit(p, sel ? sel[s] : s, &b, &tok, &h);
            lse[s] = attend(p, q, k, v, b, tok, h, keys, w, out + s * D);
        }
        free(keys);
        free(w);
    }
}

/*
 * Attention weights of each selected query over its window, [n_sel, K], in
 * the neighborhood's row-major window order, plus the key token index of each
 * entry. Used to check the weights directly (they must sum to one).
 */
void oracle_na_weights(const oracle_problem *p, const double *q, const double *k,
                       int64_t n_sel, const int64_t *sel, double *weights, int64_t *key_tokens)
{
    int64_t K = window_size(p);
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < n_sel; ++s) {
        int64_t b, tok, h;
        decode_unit(p, sel ? sel[s] : s, &b, &tok, &h);
        attend(p, q, k, NULL, b, tok, h, key_tokens + s * K, weights + s * K, NULL);
    }
}

/*
 * Per-query quantities the backward needs, recomputed from scratch:
 * the weights P over the window, the output, and delta = <dout, out>
 * (the row sum of dout * out, NATTEN's ComputeDelta).
 */
static double query_backward_terms(const oracle_problem *p, const double *q, const double *k,
                                   const double *v, const double *dout, int64_t b, int64_t tok,
                                   int64_t h, int64_t *keys, double *w, double *o)
{
    attend(p, q, k, v, b, tok, h, keys, w, o);
    return dot(vec(p, dout, b, tok, h), o, p->head_dim);
}

/*
 * Backward of L = sum(out * dout). With P the window weights of query x,
 *   dP_xy = <dout_x, v_y>                  (gradient of the weights, AGRAD)
 *   dS_xy = P_xy (dP_xy - delta_x)         (softmax backward)
 *   dq_x  = scale * sum_{y in N(x)} dS_xy k_y                (QGRAD)
 *   dk_y  = scale * sum_{x : y in N(x)} dS_xy q_x            (KGRAD)
 *   dv_y  = sum_{x : y in N(x)} P_xy dout_x                  (VGRAD)
 * dq is computed per selected query. dk and dv are computed per selected key
 * by brute-force membership: every token x of the same residue class whose
 * distance to y is at most (k-1)*d on every axis is a candidate (a window
 * contains its own query, so no attendee is farther); the candidate's window is
 * rebuilt and y is looked up in it.
 * dq, dk, dv are [n_sel, D] (full tensors when sel == NULL). Any of them may
 * be NULL to skip it.
 */
void oracle_na_bwd(const oracle_problem *p, const double *q, const double *k, const double *v,
                   const double *dout, int64_t n_sel, const int64_t *sel, double *dq, double *dk,
                   double *dv)
{
    int64_t K = window_size(p), D = p->head_dim;
    int64_t T = p->extent[0], H = p->extent[1], W = p->extent[2];
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
        double *w = (double *)malloc(sizeof(double) * K);
        double *o = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 4)
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t b, tok, h;
            decode_unit(p, sel ? sel[s] : s, &b, &tok, &h);

            if (dq) {
                /* query side: x = tok */
                double delta = query_backward_terms(p, q, k, v, dout, b, tok, h, keys, w, o);
                const double *dox = vec(p, dout, b, tok, h);
                double *g = dq + s * D;
                for (int64_t c = 0; c < D; ++c) g[c] = 0.0;
                for (int64_t j = 0; j < K; ++j) {
                    double dP = dot(dox, vec(p, v, b, keys[j], h), D);
                    double dS = w[j] * (dP - delta);
                    const double *ky = vec(p, k, b, keys[j], h);
                    for (int64_t c = 0; c < D; ++c) g[c] += p->scale * dS * ky[c];
                }
            }

            if (dk || dv) {
                /* key side: y = tok; gather over every query that attends y */
                int64_t yt = tok / (H * W), yy = (tok / W) % H, yx = tok % W;
                double *gk = dk ? dk + s * D : NULL;
                double *gv = dv ? dv + s * D : NULL;
                for (int64_t c = 0; c < D; ++c) {
                    if (gk) gk[c] = 0.0;
                    if (gv) gv[c] = 0.0;
                }
                int64_t reach[3], ctr[3] = {yt, yy, yx}, lo[3], hi[3];
                for (int a = 0; a < 3; ++a) {
                    reach[a] = (p->kernel[a] - 1) * p->dilation[a];
                    lo[a] = ctr[a] - reach[a];
                    hi[a] = ctr[a] + reach[a];
                }
                for (int64_t xt = lo[0]; xt <= hi[0]; ++xt) {
                    if (xt < 0 || xt >= T || (xt - yt) % p->dilation[0]) continue;
                    for (int64_t xy = lo[1]; xy <= hi[1]; ++xy) {
                        if (xy < 0 || xy >= H || (xy - yy) % p->dilation[1]) continue;
                        for (int64_t xx = lo[2]; xx <= hi[2]; ++xx) {
                            if (xx < 0 || xx >= W || (xx - yx) % p->dilation[2]) continue;
                            int64_t xtok = token_index(p, xt, xy, xx);
                            neighborhood(p, xtok, keys);
                            int64_t j = 0;
                            while (j < K && keys[j] != tok) ++j;
                            if (j == K) continue; /* y is not in the window of x */
                            double delta =
                                query_backward_terms(p, q, k, v, dout, b, xtok, h, keys, w, o);
                            const double *dox = vec(p, dout, b, xtok, h);
                            double dP = dot(dox, vec(p, v, b, tok, h), D);
                            double dS = w[j] * (dP - delta);
                            const double *qx = vec(p, q, b, xtok, h);
                            for (int64_t c = 0; c < D; ++c) {
                                if (gk) gk[c] += p->scale * dS * qx[c];
                                if (gv) gv[c] += w[j] * dox[c];
                            }
                        }
                    }
                }
            }
        }
        free(keys);
        free(w);
        free(o);
    }
}

/*
 * The unfused formulation (the benchmark script's method = 'unfused'): the
 * window scores are materialized as an array attn[unit][K] by na*_qk, a
 * softmax runs over its last axis, and na*_av takes the weighted sum of the
 * values over the same windows. The maintainer's profiler tables list the
 * backward kernels of these two ops: AGRAD and VGRAD (backward of na*_av),
 * QGRAD and KGRAD (backward of na*_qk). Every one of them is one of the three
 * maps below with some pair of operands:
 *   qk:          attn[x][j] = alpha * <a_x, b_{N(x)_j}>           (QK, AGRAD)
 *   av:          out_x = alpha * sum_j attn[x][j] b_{N(x)_j}      (AV, QGRAD)
 *   av_inverse:  out_y = alpha * sum_{x: y in N(x)} attn[x][j] a_x,
 *                with j the position of y in the window of x      (KGRAD, VGRAD)
 * attn rows are indexed by unit (b, token, head) in token-major order, window
 * positions j in the neighborhood's row-major order (as neighborhood() lists
 * them).
 */

/* attn[s][j] for each selected unit s (all units when sel == NULL); attn is [n_sel, K]. */
void oracle_na_qk(const oracle_problem *p, const double *a, const double *b, double alpha,
                  int64_t n_sel, const int64_t *sel, double *attn)
{
    int64_t K = window_size(p), D = p->head_dim;
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t bb, tok, h;
            decode_unit(p, sel ? sel[s] : s, &bb, &tok, &h);
            neighborhood(p, tok, keys);
            const double *ax = vec(p, a, bb, tok, h);
            for (int64_t j = 0; j < K; ++j)
                attn[s * K + j] = alpha * dot(ax, vec(p, b, bb, keys[j], h), D);
        }
        free(keys);
    }
}

/* out[s] (D values) for each selected query unit; attn is the full [units, K] array. */
void oracle_na_av(const oracle_problem *p, const double *attn, const double *b, double alpha,
                  int64_t n_sel, const int64_t *sel, double *out)
{
    int64_t K = window_size(p), D = p->head_dim;
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t u = sel ? sel[s] : s, bb, tok, h;
            decode_unit(p, u, &bb, &tok, &h);
            neighborhood(p, tok, keys);
            double *o = out + s * D;
            for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                const double *bv = vec(p, b, bb, keys[j], h);
                for (int64_t c = 0; c < D; ++c) o[c] += attn[u * K + j] * bv[c];
            }
            for (int64_t c = 0; c < D; ++c) o[c] *= alpha;
        }
        free(keys);
    }
}

/*
 * out[s] (D values) for each selected key unit y: the sum over every query x
 * whose window holds y. Candidates are found by brute force exactly as in
 * oracle_na_bwd (same residue class, within (k-1)*d on every axis), the
 * candidate's window is rebuilt and y is looked up in it, which gives j.
 */
void oracle_na_av_inverse(const oracle_problem *p, const double *attn, const double *a,
                          double alpha, int64_t n_sel, const int64_t *sel, double *out)
{
    int64_t K = window_size(p), D = p->head_dim;
    int64_t T = p->extent[0], H = p->extent[1], W = p->extent[2];
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t bb, tok, h;
            decode_unit(p, sel ? sel[s] : s, &bb, &tok, &h);
            int64_t ctr[3] = {tok / (H * W), (tok / W) % H, tok % W}, lo[3], hi[3];
            for (int ax = 0; ax < 3; ++ax) {
                lo[ax] = ctr[ax] - (p->kernel[ax] - 1) * p->dilation[ax];
                hi[ax] = ctr[ax] + (p->kernel[ax] - 1) * p->dilation[ax];
            }
            double *o = out + s * D;
            for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
            for (int64_t xt = lo[0]; xt <= hi[0]; ++xt) {
                if (xt < 0 || xt >= T || (xt - ctr[0]) % p->dilation[0]) continue;
                for (int64_t xy = lo[1]; xy <= hi[1]; ++xy) {
                    if (xy < 0 || xy >= H || (xy - ctr[1]) % p->dilation[1]) continue;
                    for (int64_t xx = lo[2]; xx <= hi[2]; ++xx) {
                        if (xx < 0 || xx >= W || (xx - ctr[2]) % p->dilation[2]) continue;
                        int64_t xtok = token_index(p, xt, xy, xx);
                        neighborhood(p, xtok, keys);
                        int64_t j = 0;
                        while (j < K && keys[j] != tok) ++j;
                        if (j == K) continue; /* y is not in the window of x */
                        int64_t xu = (bb * tokens(p) + xtok) * p->heads + h;
                        const double *ax = vec(p, a, bb, xtok, h);
                        for (int64_t c = 0; c < D; ++c) o[c] += attn[xu * K + j] * ax[c];
                    }
                }
            }
            for (int64_t c = 0; c < D; ++c) o[c] *= alpha;
        }
        free(keys);
    }
}

/*
 * Relative positional bias (the maintainer's profile names the unfused score
 * kernel QKRPB: scores plus a bias that depends only on where the key sits
 * relative to the query). Reading taken: per head, one learned value per
 * relative offset key - query, counted per axis in steps of the dilation
 * (so in class units), over the full range a shifted window can reach,
 * -(k-1) .. k-1. Table layout [heads][2kt-1][2kh-1][2kw-1]; offset delta
 * on an axis sits at index delta + k - 1.
 */
static int64_t rpb_size(const oracle_problem *p)
{
    return (2 * p->kernel[0] - 1) * (2 * p->kernel[1] - 1) * (2 * p->kernel[2] - 1);
}

/* Index in one head's table of the offset from query token x to key token y. */
static int64_t rpb_index(const oracle_problem *p, int64_t x, int64_t y)
{
    int64_t W = p->extent[2], H = p->extent[1];
    int64_t xc[3] = {x / (H * W), (x / W) % H, x % W};
    int64_t yc[3] = {y / (H * W), (y / W) % H, y % W};
    int64_t idx = 0;
    for (int a = 0; a < 3; ++a) {
        int64_t delta = (yc[a] - xc[a]) / p->dilation[a]; /* same class: exact */
        idx = idx * (2 * p->kernel[a] - 1) + delta + p->kernel[a] - 1;
    }
    return idx;
}

/* attn[s][j] = alpha * <a_x, b_{N(x)_j}> + rpb[head][offset(x, N(x)_j)]. */
void oracle_na_qk_rpb(const oracle_problem *p, const double *a, const double *b, double alpha,
                      const double *rpb, int64_t n_sel, const int64_t *sel, double *attn)
{
    int64_t K = window_size(p), D = p->head_dim, R = rpb_size(p);
    if (!sel) n_sel = p->batch * tokens(p) * p->heads;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t bb, tok, h;
            decode_unit(p, sel ? sel[s] : s, &bb, &tok, &h);
            neighborhood(p, tok, keys);
            const double *ax = vec(p, a, bb, tok, h);
            for (int64_t j = 0; j < K; ++j)
                attn[s * K + j] = alpha * dot(ax, vec(p, b, bb, keys[j], h), D) +
                                  rpb[h * R + rpb_index(p, tok, keys[j])];
        }
        free(keys);
    }
}

/* Gradient of the bias: drpb[head][o] = sum over every batch element, query
 * and window entry whose offset is o of dattn (the full [units, K] array). */
void oracle_na_rpb_grad(const oracle_problem *p, const double *dattn, double *drpb)
{
    int64_t K = window_size(p), R = rpb_size(p), n = p->batch * tokens(p) * p->heads;
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * K);
    for (int64_t i = 0; i < p->heads * R; ++i) drpb[i] = 0.0;
    for (int64_t u = 0; u < n; ++u) {
        int64_t bb, tok, h;
        decode_unit(p, u, &bb, &tok, &h);
        neighborhood(p, tok, keys);
        for (int64_t j = 0; j < K; ++j) drpb[h * R + rpb_index(p, tok, keys[j])] += dattn[u * K + j];
    }
    free(keys);
}

/* Threads the OpenMP runtime will use for the loops above. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
