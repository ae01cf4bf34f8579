/*
 * na.h -- C ABI of libna: fused neighborhood attention (NA) forward and
 * backward over 2D and 3D token grids, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one discussed in NATTEN issue #161, "Backward pass is
 * very slow towards much tokens and large kernels" (SHI-Labs/NATTEN): its
 * benchmark script calls na2d / na3d(query, key, value, kernel_size) on
 * token-major tensors [B, (T,) H, W, heads, head_dim] and drives the backward
 * with loss = output.sum(); the unfused variant in the same script spells the
 * computation out as window scores (na*_qk), a softmax over the window, and a
 * weighted sum of values (na*_av); the maintainer's profiler tables split the
 * backward into ComputeDelta (delta = rowsum(dO * O)) and the gradients of Q,
 * K, V and of the attention weights.
 *
 * Definition implemented here. Along each axis of extent L with kernel k and
 * dilation d, a query at coordinate x sees only coordinates of its own
 * residue class x mod d. Inside that class (n positions, index i = x / d) its
 * window starts at clamp(i - floor(k/2), 0, n - k) and holds k positions, so
 * it is centered where it fits and shifted inward at the borders, and always
 * has exactly k keys. The neighborhood N(x) is the product of the per-axis
 * windows (prod(k) keys). With s_xy = scale * <q_x, k_y>:
 *   lse_x = log sum_{y in N(x)} exp(s_xy)          (natural log)
 *   out_x = sum_{y in N(x)} exp(s_xy - lse_x) v_y
 * and the backward of sum(out * dout) gives
 *   delta_x = <dout_x, out_x>,  dS_xy = P_xy (<dout_x, v_y> - delta_x),
 *   dq_x = scale sum_{y in N(x)} dS_xy k_y,
 *   dk_y = scale sum_{x: y in N(x)} dS_xy q_x,  dv_y = sum_{x: y in N(x)} P_xy dout_x.
 *
 * Layout. q, k, v, out, dout, dq, dk, dv are dense, contiguous, token-major
 * arrays [B, (T,) H, W, heads, head_dim] of the problem's dtype; lse is a
 * dense fp32 array [B, (T,) H, W, heads]. Device pointers must be 16-byte
 * aligned. Every buffer is allocated and owned by the caller; the library
 * never allocates, frees or synchronizes. Work is enqueued on the given HIP
 * stream (a hipStream_t; NULL means the default stream) and completes
 * asynchronously. Outputs are overwritten, never accumulated into.
 *
 * Errors. Argument errors are detected on the host before anything is
 * enqueued and return NA_ERR_INVALID_ARG (or NA_ERR_UNSUPPORTED for a valid
 * problem the library has no kernel for, NA_ERR_WORKSPACE for a workspace that
 * is too small). A failed kernel launch returns NA_ERR_HIP. Apart from the
 * static delta array of na_bwd_noalloc, the library keeps no state between
 * calls besides a once-per-kernel raise of the dynamic-LDS limit; calls on
 * different streams may run concurrently.
 *
 * Window limit. The kernels keep 32-bit validity masks over a patch walk
 * along each axis; the walk of a key near a grid border is longer than the
 * window (up to 2k points on short axes). Windows up to 16 per axis work for
 * every extent, 17 to 21 for all class extents (extent / dilation) except a
 * few between 33 and 42, and 22 or more only for class extents below 33;
 * na_check_problem and every entry point return NA_ERR_UNSUPPORTED for the
 * rest, before anything is enqueued.
 */
#ifndef NA_H
#define NA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NA_OK = 0,
    NA_ERR_INVALID_ARG = 1,  /* malformed problem, null or misaligned pointer */
    NA_ERR_UNSUPPORTED = 2,  /* well-formed, but no kernel for it (head_dim, window limit) */
    NA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than na_bwd_workspace_bytes */
    NA_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} na_status;

typedef enum {
    NA_F32 = 0,   /* fp32 tensors, fp32 arithmetic */
    NA_BF16 = 1,  /* bf16 tensors (round-to-nearest-even on output) */
    NA_F16 = 2    /* IEEE fp16 tensors (round-to-nearest-even on output; the issue's
                     maintainer profiles the fused op at fp16 beside fp32).
                     16-bit tensors with head_dim 32 or 64: products on the 16-bit
                     MFMA with fp32 accumulation; the attention weights and score
                     gradients are rounded to the tensor type before the weighted
                     sums; softmax statistics, lse and delta stay fp32. Other
                     16-bit problems, and every 16-bit problem with a window
                     mask: fp32 arithmetic after conversion. */
} na_dtype;

/* Backward strategies (the NATTEN issue's use_kv_parallelism_in_fused_na
 * switch selects between query-parallel and KV-parallel fused backwards; its
 * set_memory_usage_preference caps how far KV parallelism may go, here the
 * kv_splits argument of na_bwd). */
typedef enum {
    NA_BWD_GATHER = 0,     /* dq by query tiles, then dk/dv by key tiles over the
                              inverse neighborhood; no atomics, deterministic */
    NA_BWD_KVPARALLEL = 1  /* one pass over key tiles producing dk, dv and fp32
                              partial sums of dq in the workspace; dq is then
                              finalized. kv_splits = 0: one accumulator, float
                              atomics, not bitwise reproducible. kv_splits = S
                              >= 1: at most S accumulator copies; each key tile
                              sums its contributions exactly (64-bit fixed point,
                              32 fraction bits, partial sums below 2^31 in
                              magnitude) and adds them to one copy with plain
                              stores, tiles of one copy never overlapping within
                              a launch (tile classes run in rounds of S); the
                              copies are summed in order: bitwise reproducible */
} na_bwd_variant;

typedef struct {
    int64_t ndim;         /* 2 or 3 */
    int64_t dtype;        /* na_dtype */
    int64_t batch;        /* B >= 1 */
    int64_t heads;        /* >= 1 */
    int64_t head_dim;     /* 16, 32 or 64 */
    int64_t extent[3];    /* grid extents, outermost first: (T, H, W) for 3D, (H, W, -) for 2D */
    int64_t kernel[3];    /* window size per axis, same order; 1 <= k <= floor(extent / dilation)
                             (and the window limit above) */
    int64_t dilation[3];  /* >= 1 per axis, same order */
    double scale;         /* finite score multiplier; the usual choice is head_dim^-0.5 */
} na_problem;

/* Host-only validation of a problem description; enqueues nothing.
 * Returns NA_OK, NA_ERR_INVALID_ARG or NA_ERR_UNSUPPORTED. */
na_status na_check_problem(const na_problem *p);

/* Forward: out (problem dtype) and lse (fp32, natural log) from q, k, v. */
na_status na_fwd(const na_problem *p, const void *q, const void *k, const void *v, void *out,
                 float *lse, void *hip_stream);

/* Bytes of device workspace na_bwd needs for the given variant and kv_splits
 * (0 on an invalid problem, variant or a negative kv_splits). NA_BWD_GATHER:
 * the fp32 delta array [B,(T,)H,W,heads] (kv_splits ignored).
 * NA_BWD_KVPARALLEL: delta plus max(kv_splits, 1) fp32 dq accumulators
 * [B,(T,)H,W,heads,head_dim] back to back. Regions start 256-byte aligned. */
size_t na_bwd_workspace_bytes(const na_problem *p, int32_t variant, int32_t kv_splits);

/* Backward of sum(out * dout): dq, dk, dv (problem dtype) from q, k, v, the
 * forward's out and lse, and dout. workspace must be a device buffer of at
 * least na_bwd_workspace_bytes(p, variant, kv_splits) bytes, 256-byte
 * aligned; its contents on entry do not matter and are left undefined.
 * kv_splits (>= 0; see na_bwd_variant) only matters for NA_BWD_KVPARALLEL. */
na_status na_bwd(const na_problem *p, const void *q, const void *k, const void *v,
                 const void *out, const void *dout, const float *lse, void *dq, void *dk,
                 void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                 int32_t kv_splits, void *hip_stream);

/* The two halves of the NA_BWD_GATHER backward, for callers that want one of
 * the gradients alone or time the kernels separately. na_bwd with
 * NA_BWD_GATHER is exactly na_bwd_dq followed by na_bwd_dkdv on one stream.
 * na_bwd_dq writes dq and the fp32 row array delta[B,(T,)H,W,heads] =
 * <dout, out> (NATTEN's ComputeDelta); na_bwd_dkdv reads that delta and writes
 * dk and dv. Same layout, alignment and error rules as na_bwd. */
na_status na_bwd_dq(const na_problem *p, const void *q, const void *k, const void *v,
                    const void *out, const void *dout, const float *lse, void *dq, float *delta,
                    void *hip_stream);
na_status na_bwd_dkdv(const na_problem *p, const void *q, const void *k, const void *v,
                      const void *dout, const float *lse, const float *delta, void *dk, void *dv,
                      void *hip_stream);

/* Windows restricted along the outermost axis (T on 3D grids, H on 2D grids):
 * the NATTEN issue's requester asks for a time kernel that changes from frame
 * to frame, and the maintainer answers that only masking changes, with tiled
 * kernels gaining their speed by skipping fully masked key/value tiles.
 * frame_kernel is a device array of extent[0] int32 values, one per
 * coordinate x0 along that axis: a query at x0 keeps only the keys whose
 * coordinate along the axis lies in the window of frame_kernel[x0] positions
 * around x0 (the same centered-and-shifted rule, in x0's residue class),
 * inside its window of kernel[0] positions; values are clamped to
 * [0, kernel[0]], and 0 masks every key of the query (its out is zero and its
 * lse -inf, and it contributes nothing to the backward). Otherwise exactly
 * na_fwd and na_bwd (same buffers, rules and errors; frame_kernel must be
 * non-null and 4-byte aligned). On 3D grids whole key (or query) planes
 * outside a tile's frame windows are skipped, so runtime follows the
 * restricted window. */
na_status na_fwd_framed(const na_problem *p, const void *q, const void *k, const void *v,
                        void *out, float *lse, const int32_t *frame_kernel, void *hip_stream);
na_status na_bwd_framed(const na_problem *p, const void *q, const void *k, const void *v,
                        const void *out, const void *dout, const float *lse, void *dq, void *dk,
                        void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                        int32_t kv_splits, const int32_t *frame_kernel, void *hip_stream);

/* Windows with an arbitrary set of their keys masked: the requester's other
 * form in the same thread, a tensor of the attended tokens of each query
 * within its window (the maintainer: runtime follows the largest window, and
 * only the masking changes). mask is a device array of bytes
 * [(T,) H, W, prod(kernel)] in row-major order, one row per query token,
 * shared by every batch element and head; byte j of a query's row is zero
 * when the query drops the j-th key of its window (window offsets in
 * row-major (t, h, w) order), exactly the mask of na_qk. Masked scores are
 * -inf before the softmax; a query that keeps no key gets a zero output, lse
 * = -inf and contributes nothing to the backward. Otherwise exactly na_fwd
 * and na_bwd (same buffers, rules and errors; mask must be non-null). With a
 * 4-byte aligned mask, fp32 problems with head_dim 16 or 32 and bf16 / fp16
 * ones with head_dim 32 run on the register-resident kernels (16-bit tensors
 * converted to fp32 while staged; forward and dq read each query's mask row,
 * dk/dv one byte per query of each key's inverse walk) wherever a masked walk
 * is compiled; other problems, the dk/dv tiles without such a walk and the
 * KV-parallel backward run on the general tile kernels, which test every
 * pair against the mask. */
na_status na_fwd_masked(const na_problem *p, const void *q, const void *k, const void *v,
                        void *out, float *lse, const uint8_t *mask, void *hip_stream);
na_status na_bwd_masked(const na_problem *p, const void *q, const void *k, const void *v,
                        const void *out, const void *dout, const float *lse, void *dq, void *dk,
                        void *dv, void *workspace, size_t workspace_bytes, int32_t variant,
                        int32_t kv_splits, const uint8_t *mask, void *hip_stream);

/* The requester's index tensor turned into the mask above (same thread of
 * the NATTEN issue: the attended tokens of each query given as indices, for
 * na3d_qk; the maintainer: a tiled kernel keeps the largest window and only
 * masks inside it). indices is a device array of int64 [(T,) H, W, m], 8-byte
 * aligned: per query token, m flat token indices (t * H + h) * W + w of one
 * batch element's grid, shared by every batch element and head; -1 marks an
 * unused slot. Writes mask [(T,) H, W, prod(kernel)] (any alignment): byte j
 * of a query's row is 1 when a slot lists the j-th key of its window, else 0
 * (a key listed twice is kept once; m = 0 drops every key), and bad
 * [(T,) H, W] int32 (4-byte aligned): the number of the query's slots holding
 * neither -1 nor a token of its window. The masked kernels only visit the
 * window, so such a row does not describe the caller's attention: the caller
 * checks bad (the Python binding raises). Only the problem's ndim, extent,
 * kernel and dilation are read (the same rules as na_check_problem, without
 * the window limit); NA_ERR_INVALID_ARG for a malformed grid, m < 0, null
 * mask or bad, null indices with m > 0, or misaligned pointers. */
na_status na_window_mask_from_indices(const na_problem *p, const int64_t *indices, int32_t m,
                                      uint8_t *mask, int32_t *bad, void *hip_stream);

/* Static, human-readable name of a status code. */
const char *na_status_string(na_status s);

/* Static string: the sha256 (hex) of the sources this library was built
 * from (every file of the kernel and ABI sources and this header, in name
 * order, as fwd_bwd_amd/build.py hashes them), or "unknown". */
const char *na_source_sha256(void);

/* ------------------------------------------------------------------------
 * Backward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Exactly na_bwd with NA_BWD_GATHER (the same kernels, bitwise the same
 * dq, dk, dv), except that the delta rows live in a static device array of
 * the library instead of a caller workspace: NA_NOALLOC_MAX_ROWS fp32 values
 * (32 MiB), held on every GPU the library runs on until the process ends.
 * Problems with more than NA_NOALLOC_MAX_ROWS (token, head) rows, i.e.
 * batch * prod(extent) * heads, return NA_ERR_WORKSPACE before anything is
 * enqueued. Nothing is allocated, freed or synchronized; inputs and outputs
 * are the caller's, as for na_bwd. All calls on one GPU share that GPU's
 * array (it keeps the last call's contents, which the next call overwrites
 * before reading): calls that overlap in time on one GPU, e.g. on two
 * streams, race and must be ordered by the caller. */
#define NA_NOALLOC_MAX_ROWS 8388608
na_status na_bwd_noalloc(const na_problem *p, const void *q, const void *k, const void *v,
                         const void *out, const void *dout, const float *lse, void *dq, void *dk,
                         void *dv, void *hip_stream);

/* Host helpers exposing the window rule on one axis (absolute coordinates).
 * na_window_start returns the first key coordinate of the window of query
 * coordinate x (keys are start + d*j, j < k), or -1 on invalid arguments.
 * na_inverse_window writes the first and last query coordinate (same residue
 * class, step d) whose window contains key coordinate y; every class member
 * between them attends y. Returns NA_ERR_INVALID_ARG on invalid arguments. */
int64_t na_window_start(int64_t extent, int64_t kernel, int64_t dilation, int64_t x);
na_status na_inverse_window(int64_t extent, int64_t kernel, int64_t dilation, int64_t y,
                            int64_t *first, int64_t *last);

/* ------------------------------------------------------------------------
 * Unfused ops (NATTEN issue #161: the benchmark script's method = 'unfused'
 * materializes the window scores with na2d_qk / na3d_qk, applies a softmax
 * over the window axis, and forms the output with na2d_av / na3d_av; the
 * maintainer's profiler tables list their backward kernels AGRAD, QGRAD,
 * KGRAD and VGRAD).
 *
 * Layout. As in that script these ops take head-major tensors: a, b, q, k, v,
 * out, dout, dq, dk, dv are dense [B, heads, (T,) H, W, head_dim] arrays and
 * the attention arrays (attn, probs, dprobs, dscores) are dense fp32
 * [B, heads, (T,) H, W, K], K = prod(kernel), entry j of a row being the key
 * at window offset j in row-major (t, h, w) order; the window and the
 * dilation rule are those of the fused ops above. Only NA_F32 problems are
 * supported (others return NA_ERR_UNSUPPORTED); problem->scale is used only
 * by na_unfused_fwd / na_unfused_bwd, and na_softmax / na_softmax_bwd accept
 * any head_dim >= 1 (they never read a head_dim-long vector). Pointers must be non-null and 16-byte
 * aligned; buffers are caller-owned, outputs are overwritten, work is
 * enqueued on hip_stream and nothing is allocated or synchronized. Errors as
 * for the fused ops.
 */

/* attn[x][j] = alpha * <a_x, b_{N(x)_j}> [+ rpb[head][offset]]: the window
 * scores (na*_qk with a = q, b = k, alpha = scale) and the gradient of the
 * weights of na*_av (AGRAD: a = dout, b = v, alpha = 1, rpb = mask = NULL).
 * attn must not overlap a or b.
 * mask (may be NULL): masked windows, as the issue's requester masks the
 * result of na3d_qk to give each frame its own window: a byte array
 * [(T,) H, W, K] per token, shared by every batch element and head; entries
 * whose byte is 0 get the score -inf, so na_softmax gives them zero weight (a
 * query with every entry masked gets all-zero weights and a zero output).
 * rpb (may be NULL): relative positional bias, the QKRPB of the maintainer's
 * unfused profile. A dense fp32 table [heads][2kt-1][2kh-1][2kw-1] (2D:
 * [heads][2kh-1][2kw-1]); the entry added to the score of query x and key y
 * sits at (y - x) / dilation + (k - 1) along each axis, i.e. it depends only
 * on the offset of the key from the query in class units, over the full
 * range -(k-1) .. k-1 a border-shifted window can reach. */
na_status na_qk(const na_problem *p, const void *a, const void *b, double alpha, const float *rpb,
                const uint8_t *mask, float *attn, void *hip_stream);

/* na_qk (with a = q, b = k, alpha = scale, optional rpb and mask) followed by
 * na_softmax, writing only the probabilities: on single-plane grids one
 * kernel takes each query's whole window softmax in registers, elsewhere the
 * two ops run in turn. Same layouts and rules as na_qk. */
na_status na_qk_softmax(const na_problem *p, const void *a, const void *b, double alpha,
                        const float *rpb, const uint8_t *mask, float *probs, void *hip_stream);

/* AGRAD followed by the softmax backward: dscores = probs * (dP - rowsum(probs * dP))
 * with dP[x][j] = <dout_x, v_{N(x)_j}>; one kernel on single-plane grids, else
 * na_qk then na_softmax_bwd. dscores must not overlap probs. */
na_status na_qk_softmax_bwd(const na_problem *p, const void *dout, const void *v,
                            const float *probs, float *dscores, void *hip_stream);

/* Bytes of device workspace na_rpb_grad needs (0 on an invalid problem). */
size_t na_rpb_grad_workspace_bytes(const na_problem *p);

/* Gradient of the bias table: drpb[head][o] = the sum of dscores over every
 * batch element, query and window entry whose key sits at offset o from the
 * query (layout of rpb in na_qk). Deterministic (fixed summation order, no
 * atomics); uses a caller-owned workspace of na_rpb_grad_workspace_bytes.
 * Windows of more than 512 entries or tables of more than 2048 offsets
 * return NA_ERR_UNSUPPORTED. */
na_status na_rpb_grad(const na_problem *p, const float *dscores, float *drpb, void *workspace,
                      size_t workspace_bytes, void *hip_stream);

/* out_x = alpha * sum_j attn[x][j] * b_{N(x)_j}: na*_av (b = v, alpha = 1) and
 * the query gradient of na*_qk (QGRAD: attn = dscores, b = k, alpha = scale). */
na_status na_av(const na_problem *p, const float *attn, const void *b, double alpha, void *out,
                void *hip_stream);

/* out_y = alpha * sum over the queries x whose window holds y of attn[x][j] * a_x,
 * j being the offset of y in the window of x: the key gradient of na*_qk
 * (KGRAD: attn = dscores, a = q, alpha = scale) and the value gradient of
 * na*_av (VGRAD: attn = probs, a = dout, alpha = 1). Each output row is
 * written once by its owner; no atomics. */
na_status na_av_inverse(const na_problem *p, const float *attn, const void *a, double alpha,
                        void *out, void *hip_stream);

/* probs = softmax of attn over the window axis (rows of K); in place allowed. */
na_status na_softmax(const na_problem *p, const float *attn, float *probs, void *hip_stream);

/* Softmax backward over rows of K: dscores = probs * (dprobs - rowsum(probs * dprobs));
 * dscores may alias dprobs. */
na_status na_softmax_bwd(const na_problem *p, const float *probs, const float *dprobs,
                         float *dscores, void *hip_stream);

/* The unfused forward: probs = softmax(scale * na_qk(q, k) [+ rpb], masked)
 * (na_qk_softmax), out = na_av(probs, v). rpb and mask may be NULL (as in na_qk). probs
 * ([B, heads, (T,) H, W, K] fp32) is an output, kept for the backward, which
 * needs no mask: masked entries have zero weight in probs. */
na_status na_unfused_fwd(const na_problem *p, const void *q, const void *k, const void *v,
                         const float *rpb, const uint8_t *mask, float *probs, void *out,
                         void *hip_stream);

/* The unfused backward of sum(out * dout), from the forward's probs:
 * dscores = softmax backward of dprobs = na_qk(dout, v) (AGRAD; together
 * na_qk_softmax_bwd), dv = na_av_inverse(probs, dout) (VGRAD), dq = scale * na_av(dscores, k) (QGRAD),
 * dk = scale * na_av_inverse(dscores, q) (KGRAD), and, when drpb is not
 * NULL, the bias gradient drpb = na_rpb_grad(dscores) (workspace of
 * na_rpb_grad_workspace_bytes; ignored when drpb is NULL). dscores is a
 * caller-owned fp32 [B, heads, (T,) H, W, K] scratch array, left holding
 * dscores. */
na_status na_unfused_bwd(const na_problem *p, const void *q, const void *k, const void *v,
                         const float *probs, const void *dout, float *dscores, void *dq,
                         void *dk, void *dv, float *drpb, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* NA_H */
