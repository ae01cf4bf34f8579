// na_fast.hpp -- neighborhood attention kernels with register-resident scores,
// for fp32 tensors and small windows (gfx950, wave64, MFMA 4x4x1 f32).
//
// Work decomposition. A workgroup of four waves owns a 1 x 16 x 16 tile of one
// residue class of one (batch, head); each wave owns an 8 x 8 quarter of it,
// one point per lane, in sixteen 1 x 2 x 2 patches (one per 4-lane MFMA
// block). Every wave walks the whole window (forward, dq) or inverse window
// (dk/dv) of its own points, so no partial results are merged between waves.
// The walk along H and W has a compile-time length (CH x CW patches of the
// other side per block), which lets each lane keep the scores of its point for
// the whole walk in registers: the kernels run in phases that each need one
// staged tensor only, and the LDS holds one box plane of one tensor at a time.
//
//   forward, per key plane:  K -> S and its maximum;  V -> P = exp2(S - m), O += P V
//   dq, per key plane:       V -> dP;  K -> S, dS = P (dP - delta);  K -> dQ += dS K
//   dk/dv, per query plane:  Q -> P;  dO -> dV += P dO;  dO -> dS;  Q -> dK += dS Q
//
// (NATTEN issue #161, "Backward pass is very slow towards much tokens and large
// kernels": the backward recomputes the attention weights from the saved
// logsumexp, uses delta = rowsum(dO * O), and forms dK and dV by gathering
// over each key's inverse neighborhood.)
//
// LDS layouts. A staged point takes D * 4 bytes (NC 16-byte chunks), points of
// a box row contiguous, rows at a padded pitch. The 16 lanes of a quarter wave
// hold four patches stacked along H (an 8 x 2 block of points), and read
//  * key-major (A): chunk s of each lane's own point; conflict-free when the
//    row pitch is an odd number of 16-byte slots;
//  * d-major (B): the four lanes of a block read chunks c, c + 4, ... of the
//    same point, all blocks the same entry of their patch; conflict-free when
//    the row pitch is 2 (mod 4) slots.
// Within a point every chunk offset is a compile-time immediate, and a walk
// item only adds a wave-uniform row offset, so LDS addressing costs about one
// VALU add per item row.
//
// Softmax (forward). The exact maximum of a plane's scores is known before any
// exponential is taken, so the sums are rescaled at most once per key plane (2D
// grids: never).
#pragma once

#include "na_common.hpp"

#include <type_traits>

namespace na {
namespace fast {

constexpr int kTH = 16, kTW = 16;  // tile extent along H and W (T: 1)

struct Geom {
    int ext[3], ker[3], dil[3];
    int heads, batch, head_dim;
    int tiles[3];      // tiles per axis over the largest residue class
    int nres, n_tiles;
    int ra, rb;        // LDS row pitch in bytes of the key-major (A) and d-major (B) layouts
    int rows_off;      // dk/dv: byte offset of the per-point (lse, delta) rows in LDS
    int rows_pitch;    // dk/dv: points per row of those rows
    Border border;     // when on: the border tiles only
    // divisors of the tile decode
    FastDiv f_heads, f_t, f_plane, f_bandrows, f_band, f_lastband, f_nres, f_c, f_cb;
    FastDiv f_dil[3], f_dil21;
};

// T: the tensors' element type (float, or bf16 / f16, which the staging
// converts to fp32 on the way into LDS); lse and delta are fp32.
template <typename T>
struct FwdArgsT {
    Geom g;
    const T *q, *k, *v;
    T *out;
    float *lse;
    float qscale;  // scale * log2(e)
    const int *frame;  // windows restricted along frame_axis (null: none)
    int frame_axis;
    // window mask (MASK kernels): mask_k bytes per query token, mask_bytes in all
    const uint8_t *mask;
    int64_t mask_bytes;
    int mask_k;
};
using FwdArgs = FwdArgsT<float>;

template <typename T>
struct BwdArgsT {
    Geom g;
    const T *q, *k, *v, *out, *dout;
    const float *lse;
    float *delta;
    T *dq, *dk, *dv;
    float qscale, scale;
    int walk_lo;  // dk/dv: this launch takes the tiles whose inverse walk exceeds walk_lo
    // dk/dv border classes (when edge >= 0, instead of walk_lo): the launch
    // takes the tiles whose inverse walk along H exceeds walk_c exactly when
    // bit 0 of edge is set, and along W exactly when bit 1 is set
    int edge, walk_c;
    const int *frame;  // windows restricted along frame_axis (null: none)
    int frame_axis;
    // window mask (MASK kernels, dq): mask_k bytes per query token, mask_bytes in all
    const uint8_t *mask;
    int64_t mask_bytes;
    int mask_k;
};
using BwdArgs = BwdArgsT<float>;

// Tile id -> tile. The head varies fastest: consecutive tiles (and so the
// workgroups one XCD runs at a time) cover all heads of one position, whose
// rows of one token are adjacent in memory (measured faster than one head at
// a time over twice as many positions). Then T (the tiles of one (H, W)
// column share two of every three key planes of a 3-plane window), then (H,
// W) in bands kFastBand tiles wide along W, residue class, batch.
constexpr int kFastBand = 8;

// Plane of step j of a walk over planes [first, first + len): the one
// congruent to j modulo len. The tiles of neighbouring planes, which run at
// the same time, then stage the same plane in the same step wherever their
// walks overlap, so that its second and third reads come from L2 (3D grid
// 16 x 256 x 256, window 3 x 5 x 5: forward HBM reads -16%, dk/dv -5%, step
// 10.76 -> 10.54 ms). Sums over the planes are taken in this order.
__device__ __forceinline__ int plane_of_step(int first, int len, int j) {
    int r = (j - first) % len;
    if (r < 0) r += len;
    return first + r;
}

__device__ __forceinline__ bool decode(const Geom &g, int tile, TileCtx &w) {
    int rem = tile, q;
    q = fdiv(rem, g.f_heads);
    const int head = rem - q * g.heads;
    rem = q;
    q = fdiv(rem, g.f_t);
    const int tt = rem - q * g.tiles[0];
    rem = q;
    int th, tw, res = 0;
    if (g.border.on) {
        q = fdiv(rem, g.f_plane);  // f_plane: border tiles per plane here
        int i = rem - q * g.border.per_plane;
        rem = q;
        const int rb = g.border.rows_lo + g.border.rows_hi;
        const int cls = g.border.cls;
        if (cls != 0) {
            // one class: f_c divides by its number of columns
            const int ncol = (cls & 2) ? g.border.cols_lo + g.border.cols_hi
                                       : g.tiles[2] - g.border.cols_lo - g.border.cols_hi;
            const int rr = fdiv(i, g.f_c), cc = i - rr * ncol;
            th = !(cls & 1) ? g.border.rows_lo + rr
                 : rr < g.border.rows_lo ? rr : g.tiles[1] - g.border.rows_hi + (rr - g.border.rows_lo);
            tw = !(cls & 2) ? g.border.cols_lo + cc
                 : cc < g.border.cols_lo ? cc : g.tiles[2] - g.border.cols_hi + (cc - g.border.cols_lo);
        } else if (i < rb * g.tiles[2]) {
            const int rr = fdiv(i, g.f_c);
            tw = i - rr * g.tiles[2];
            th = rr < g.border.rows_lo ? rr : g.tiles[1] - g.border.rows_hi + (rr - g.border.rows_lo);
        } else {
            i -= rb * g.tiles[2];
            const int cb = g.border.cols_lo + g.border.cols_hi;
            const int qq = fdiv(i, g.f_cb), cc = i - qq * cb;
            th = g.border.rows_lo + qq;
            tw = cc < g.border.cols_lo ? cc : g.tiles[2] - g.border.cols_hi + (cc - g.border.cols_lo);
        }
    } else {
        q = fdiv(rem, g.f_plane);
        int in = rem - q * (g.tiles[1] * g.tiles[2]);
        rem = q;
        const int band = fdiv(in, g.f_bandrows);
        const int bw = imin(kFastBand, g.tiles[2] - band * kFastBand);
        in -= band * kFastBand * g.tiles[1];
        th = fdiv(in, bw == kFastBand ? g.f_band : g.f_lastband);
        tw = band * kFastBand + (in - th * bw);
        q = fdiv(rem, g.f_nres);
        res = rem - q * g.nres;
        rem = q;
    }
    const int b = rem;
    // residue class of each axis, its size and the tile origin
    int r[3];
    q = fdiv(res, g.f_dil[2]);
    r[2] = res - q * g.dil[2];
    const int q1 = fdiv(q, g.f_dil[1]);
    r[1] = q - q1 * g.dil[1];
    r[0] = fdiv(res, g.f_dil21);
    const int o[3] = {tt, th * kTH, tw * kTW};
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        w.n[a] = fdiv(g.ext[a] - r[a] + g.dil[a] - 1, g.f_dil[a]);
        w.k[a] = g.ker[a];
        w.o[a] = o[a];
        w.r[a] = r[a];
        w.d[a] = g.dil[a];
        inside = inside && (o[a] < w.n[a]);
    }
    const int64_t HW = (int64_t)g.ext[1] * g.ext[2];
    const int64_t ntok = HW * g.ext[0];
    const int64_t hd = (int64_t)g.heads * g.head_dim;
    const int64_t origin_tok = r[0] * HW + (int64_t)r[1] * g.ext[2] + r[2];
    w.base = ((int64_t)b * ntok + origin_tok) * hd + (int64_t)head * g.head_dim;
    w.st[0] = g.dil[0] * HW * hd;
    w.st[1] = (int64_t)g.dil[1] * g.ext[2] * hd;
    w.st[2] = (int64_t)g.dil[2] * hd;
    w.lbase = ((int64_t)b * ntok + origin_tok) * g.heads + head;
    w.lst[0] = g.dil[0] * HW * g.heads;
    w.lst[1] = (int64_t)g.dil[1] * g.ext[2] * g.heads;
    w.lst[2] = (int64_t)g.dil[2] * g.heads;
    return inside;
}

// The lane's point and its patch (first point) in the tile, clamped into the
// grid. Wave v owns the 8 x 8 quarter at (8 (v >> 1), 8 (v & 1)); lane l is
// entry l % 4 of patch l / 4, patches stacked four along H per quarter wave.
struct Lane {
    int f[3], p[3];
    bool active;
};

__device__ __forceinline__ Lane lane_geom(const TileCtx &w, int wave, int lane) {
    const int c = lane & 3, grp = lane >> 2;
    Lane L;
    L.f[0] = L.p[0] = w.o[0];
    L.f[1] = w.o[1] + 8 * (wave >> 1) + 2 * (grp & 3);
    L.f[2] = w.o[2] + 8 * (wave & 1) + 2 * (grp >> 2);
    L.p[1] = L.f[1] + (c >> 1);
    L.p[2] = L.f[2] + (c & 1);
    L.active = L.p[1] < w.n[1] && L.p[2] < w.n[2];
#pragma unroll
    for (int a = 1; a < 3; ++a) {
        L.f[a] = imin(L.f[a], w.n[a] - 1);
        L.p[a] = imin(L.p[a], w.n[a] - 1);
    }
    return L;
}

// Copy one plane (class T coordinate tk) of the box [U1, U1 + E1) x [U2, U2 + E2)
// of src into lds, box row r at byte r * rowb, points PS bytes apart (D * 4,
// or one 16-byte slot more), with direct global-to-LDS loads (16 bytes per
// lane, 64 consecutive slots per wave instruction; lanes on padding slots are
// idle). Points past the grid repeat the last grid point; they are only ever
// read masked. Completion: stage_wait().
template <typename T, int D, int PS>
__device__ __forceinline__ void stage_plane(const T *src, const TileCtx &w, int tk, int U1,
                                            int E1, int U2, int E2, int rowb, char *lds) {
    constexpr int NC = D / 4, SP = PS / 16;  // chunks of data, slots per point
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int parts = (E2 * SP + 63) >> 6;
    if constexpr (!std::is_same<T, float>::value) {
        // 16-bit elements: the same fp32 layout, four elements (8 bytes) per
        // 16-byte slot, loaded into registers and converted on the way
        const T *plane = src + w.base + tk * w.st[0];
        for (int part = 0; part < parts; ++part) {
            const int j = part * 64 + lane;
            const int col = j / SP, chunk = j - col * SP;
            if (col >= E2 || chunk >= NC) continue;
            const T *colp = plane + imin(U2 + col, w.n[2] - 1) * w.st[2] + chunk * 4;
            char *dst = lds + part * 1024 + lane * 16;
#pragma unroll 4
            for (int r = wave; r < E1; r += kWaves) {
                float d[4];
                Io<T>::load4(colp + imin(U1 + r, w.n[1] - 1) * w.st[1], d);
                *reinterpret_cast<f4 *>(dst + r * rowb) = f4{d[0], d[1], d[2], d[3]};
            }
        }
        return;
    }
    const char *plane = reinterpret_cast<const char *>(src) + (w.base + tk * w.st[0]) * 4;
    for (int part = 0; part < parts; ++part) {
        const int j = part * 64 + lane;
        const int col = j / SP, chunk = j - col * SP;
        if (col >= E2 || chunk >= NC) continue;
        const int c2 = imin(U2 + col, w.n[2] - 1);
        const int colb = (int)(c2 * w.st[2]) * 4 + (chunk << 4);
        for (int r = wave; r < E1; r += kWaves) {
            const int c1 = imin(U1 + r, w.n[1] - 1);
            const char *rowp = plane + c1 * w.st[1] * 4;
#if defined(__HIP_DEVICE_COMPILE__)
            __builtin_amdgcn_global_load_lds(rowp + colb, (lds_void *)(lds + r * rowb + part * 1024),
                                             16, 0, 0);
#else
            (void)rowp;
            (void)colb;
#endif
        }
    }
}

// (logsumexp * log2(e), delta) of every point of one box plane, as float2 at
// rows + (r * pitch + col).
__device__ __forceinline__ void stage_rows_plane(const float *lse, const float *delta,
                                                 const TileCtx &w, int tk, int U1, int E1, int U2,
                                                 int E2, int pitch, float2 *rows) {
    for (int i = threadIdx.x; i < E1 * E2; i += kThreads) {
        const int r = i / E2, col = i - r * E2;
        const int c[3] = {tk, imin(U1 + r, w.n[1] - 1), imin(U2 + col, w.n[2] - 1)};
        const int64_t ro = row_off(w, c);
        rows[r * pitch + col] = make_float2(lse[ro] * kLog2e, delta[ro]);
    }
}

// A 16-byte chunk at LDS byte address base + off.
__device__ __forceinline__ f4 lds_chunk(const char *base, int off) {
    return *reinterpret_cast<const f4 *>(base + off);
}

// Software pipeline over the N items of a fully unrolled walk: the LDS reads
// of item i + 1 (into register buffer (i + 1) & 1) are issued before the MFMAs
// of item i, and scheduling barriers keep the compiler from pulling them back
// next to their uses (it otherwise trades this overlap for registers).
template <int N, typename Load, typename Compute>
__device__ __forceinline__ void pipelined(Load &&load, Compute &&compute) {
    load(0, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i + 1 < N) load(i + 1, (i + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(i, i & 1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Keeps the four values of an item in registers at this point: otherwise the
// compiler may sink their last arithmetic into the next phase and hold its
// inputs (twice the registers) across the staging in between.
__device__ __forceinline__ void pin4(float (&x)[4]) {
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

// A zero the compiler cannot see through: added to the address of a row that
// is reloaded inside the plane loop, it keeps the load there instead of
// hoisting it (and its registers) across the loop.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// Half-item pipelining: step j of a walk covers item j / 2, half j % 2 (half
// of a point's chunks key-major, or one row of the patch d-major), so the
// register buffer of the next step holds half an item.
template <int NH>
__device__ __forceinline__ void load_chunks(const char *pt, f4 (&x)[NH]) {
#pragma unroll
    for (int s = 0; s < NH; ++s) x[s] = lds_chunk(pt, s * 16);
}

// z0, z1 += the chunks x (elements from chunk c0 on) times b, as two chains.
template <int NH, int N>
__device__ __forceinline__ void dot_half(const f4 (&x)[NH], const float (&b)[N], int c0, f4 &z0,
                                         f4 &z1) {
#pragma unroll
    for (int s = 0; s < NH; ++s) {
        const int d = 4 * (c0 + s);
        z0 = mfma4(x[s][0], b[d + 0], z0);
        z1 = mfma4(x[s][1], b[d + 1], z1);
        z0 = mfma4(x[s][2], b[d + 2], z0);
        z1 = mfma4(x[s][3], b[d + 3], z1);
    }
}

// One row (entries 2h, 2h + 1, points PS bytes apart) of a patch read d-major.
template <int D, int PS>
__device__ __forceinline__ void load_row_dmajor(const char *row, int col, f4 (&x)[2][D / 16]) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < D / 16; ++j) x[e][j] = lds_chunk(row + col + e * PS, j * 64);
}

// acc[g] += entry[dim(i, g)] * w[e] over the two entries of a patch row.
template <int D>
__device__ __forceinline__ void axpy_row(const f4 (&x)[2][D / 16], float w0, float w1,
                                         f4 (&acc)[D / 4]) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[4 * j + t] = mfma4(x[0][j][t], w0, acc[4 * j + t]);
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[4 * j + t] = mfma4(x[1][j][t], w1, acc[4 * j + t]);
}

// Store a per-lane accumulator (dims as in axpy_patch) times mul to the
// lane's own row.
template <typename T, int D>
__device__ __forceinline__ void store_row(T *dst, const f4 (&acc)[D / 4], float mul) {
    constexpr int NQ = D / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const float o[4] = {acc[4 * j][i] * mul, acc[4 * j + 1][i] * mul,
                                acc[4 * j + 2][i] * mul, acc[4 * j + 3][i] * mul};
            Io<T>::store4(dst + 4 * (i + 4 * j), o);
        }
}

// ----------------------------------------------------------------------------
// Window masks (MASK kernels: na_fwd_masked, and dq of na_bwd_masked). The
// mask holds mask_k bytes per query token ([(T,) H, W, K] in row-major order,
// shared by batch elements and heads); byte it * kh * kw + jh * kw + jw of a
// query's row is zero when the query drops that key of its window (plane it,
// row jh, column jw of the window).

// Bit b (b < 4) set when byte b of u is nonzero.
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t u) {
    uint32_t t = u | (u >> 4);
    t |= t >> 2;
    t |= t >> 1;
    t &= 0x01010101u;
    return (t | (t >> 7) | (t >> 14) | (t >> 21)) & 0xfu;
}

// Dword of the mask at byte a (a multiple of 4; the mask is 4-byte aligned):
// read whole when it lies inside the mask, else byte by byte up to its end.
__device__ __forceinline__ uint32_t mask_dword(const uint8_t *mask, int64_t nbytes, int64_t a) {
    if (a + 4 <= nbytes) return *reinterpret_cast<const uint32_t *>(mask + a);
    uint32_t v = 0u;
    for (int b = 0; b < 4; ++b)
        if (a + b < nbytes) v |= (uint32_t)mask[a + b] << (8 * b);
    return v;
}

// The mask bits of one query's window plane laid over its walk: bit
// (r & 1) * 16 + q of word r / 2 for walk row r, column q, which is window
// row r - lo1, column q - lo2 (lo1, lo2 in {0, 1}); zero outside the window.
// rowbase: byte of the plane's first entry in the query's mask row.
template <int CH, int CW>
__device__ __forceinline__ void walk_mask_bits(const uint8_t *mask, int64_t nbytes,
                                               int64_t rowbase, int kh, int kw, int lo1, int lo2,
                                               uint32_t (&wb)[CH]) {
    static_assert(2 * CW <= 16, "a walk row must fit 16 bits");
#pragma unroll
    for (int i = 0; i < CH; ++i) wb[i] = 0u;
    const uint32_t keep = (1u << kw) - 1u;  // kw <= 2 CW - 1 <= 15
#pragma unroll
    for (int r = 0; r < 2 * CH; ++r) {
        const int jh = r - lo1;
        if ((unsigned)jh >= (unsigned)kh) continue;
        const int64_t st = rowbase + (int64_t)jh * kw;  // the window row's first byte
        const int64_t d0 = st & ~(int64_t)3;
        const uint32_t sh = (uint32_t)(st - d0) * 8u;
        const uint32_t x0 = mask_dword(mask, nbytes, d0), x1 = mask_dword(mask, nbytes, d0 + 4);
        const uint32_t x2 = kw > 4 ? mask_dword(mask, nbytes, d0 + 8) : 0u;
        // bytes 0..3 and 4..7 of the window row, and byte 8
        const uint64_t lo = (((uint64_t)x1 << 32) | x0) >> sh;
        const uint64_t hi = (((uint64_t)x2 << 32) | x1) >> sh;
        const uint32_t bits = nonzero_bytes4((uint32_t)lo) | (nonzero_bytes4((uint32_t)hi) << 4) |
                              (((uint32_t)(hi >> 32) & 0xffu) ? 0x100u : 0u);
        wb[r >> 1] |= ((bits & keep) << lo2) << ((r & 1) * 16);
    }
}

// Byte of the first entry of the query's mask row: the query's grid token
// (class coordinates p of residue class r, dilation d) times mask_k.
__device__ __forceinline__ int64_t mask_row_base(const TileCtx &w, const int (&ext)[3],
                                                 const int (&p)[3], int mask_k) {
    const int64_t t = w.r[0] + (int64_t)w.d[0] * p[0];
    const int64_t h = w.r[1] + (int64_t)w.d[1] * p[1];
    const int64_t x = w.r[2] + (int64_t)w.d[2] * p[2];
    return ((t * ext[1] + h) * ext[2] + x) * mask_k;
}

__device__ __forceinline__ bool walk_bit(const uint32_t *wb, int r, int q) {
    return (wb[r >> 1] >> ((r & 1) * 16 + q)) & 1u;
}

// Whether walk row r (0 .. 2C - 1, relative to the block's walk start) lies
// in the window of a point whose window starts lo (0 or 1) rows after the walk
// start: rows 1 .. 2C - 3 always do (k >= 2C - 2 for a walk of C patches).
template <int C>
__device__ __forceinline__ bool walk_row_valid(int r, int lo, int k) {
    if (r >= 1 && r <= 2 * C - 3) return true;
    return (unsigned)(r - lo) < (unsigned)k;
}

template <int CH, int CW>
struct Edge {
    // validity of this lane's entries in walk rows / columns that can be
    // outside its window
    bool h[2 * CH], w[2 * CW];
};

// ============================================================================
// Forward.
// MASK: the window mask of a.mask as well (its bits per key plane in uint32_t
// words over the walk, see walk_mask_bits).
template <typename T, int D, int CH, int CW, bool T3, bool MASK = false>
__device__ __forceinline__ void fwd_tile(const FwdArgsT<T> &a, int tile, char *smem) {
    constexpr int PS = D * 4, NC = D / 4, G = D / 4, NI = CH * CW;
    TileCtx w;
    if (!decode(a.g, tile, w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3;
    const Lane L = lane_geom(w, wave, lane);

    int us[3], lo[3], U[3], E[3];
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        us[x] = window_start(L.f[x], w.n[x], w.k[x]);
        lo[x] = window_start(L.p[x], w.n[x], w.k[x]) - us[x];
        key_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], &U[x], &E[x]);
    }
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    Edge<CH, CW> ed;
#pragma unroll
    for (int r = 0; r < 2 * CH; ++r) ed.h[r] = walk_row_valid<CH>(r, lo[1], w.k[1]);
#pragma unroll
    for (int r = 0; r < 2 * CW; ++r) ed.w[r] = walk_row_valid<CW>(r, lo[2], w.k[2]);
    // frames along H (2D grids): walk rows outside the query row's frame window
    // are masked; along T (3D grids) whole key planes are skipped below
    if (a.frame && a.frame_axis == 1) {
        const unsigned fb = frame_bits(us[1], L.p[1], w.n[1], frame_size(a.frame, w, 1, L.p[1]));
#pragma unroll
        for (int r = 0; r < 2 * CH; ++r) ed.h[r] = ed.h[r] && ((fb >> r) & 1u);
    }
    const int fk_t = (a.frame && a.frame_axis == 0) ? frame_size(a.frame, w, 0, w.o[0]) : 0;

    const int ra = a.g.ra, rb = a.g.rb;
    // key-major: this lane supplies entry c of its block's patch
    const char *baseA = smem + (us[1] - U[1] + (c >> 1)) * ra + (us[2] - U[2] + (c & 1)) * PS;
    // d-major: this lane supplies chunks c, c + 4, ... of the block's entries
    const char *baseB = smem + (us[1] - U[1]) * rb + (us[2] - U[2]) * PS + c * 16;

    const int64_t qo = elem_off(w, L.p);
    float m = -1e30f, l = 0.f;
    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    const int nplanes = T3 ? w.k[0] : 1;
    for (int j = 0; j < nplanes; ++j) {
        const int tk = plane_of_step(t0, nplanes, j);
        if (a.frame && a.frame_axis == 0 && !in_frame(tk, w.o[0], w.n[0], fk_t)) continue;
        if (j > 0) __syncthreads();
        stage_plane<T, D, PS>(a.k, w, tk, U[1], E[1], U[2], E[2], ra, smem);
        float qr[D];
        load_row<T, D>(a.q + qo + opaque_zero(), qr);
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] *= a.qscale;
        uint32_t wb[MASK ? CH : 1];
        if constexpr (MASK)
            walk_mask_bits<CH, CW>(a.mask, a.mask_bytes,
                                   mask_row_base(w, a.g.ext, L.p, a.mask_k) +
                                       (int64_t)(tk - t0) * w.k[1] * w.k[2],
                                   w.k[1], w.k[2], lo[1], lo[2], wb);
        stage_wait();

        // S_b[i][c] = <k_i, q_c>, masked; plane maximum
        float s[NI][4];
        float mj = -1e30f;
        {
            f4 kb[2][NC / 2], z0, z1;
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (j & 1) * (NC / 2) * 16, kb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1, c1 = i / CW, c2 = i % CW;
                    if ((j & 1) == 0) z0 = z1 = f4{0.f, 0.f, 0.f, 0.f};
                    dot_half<NC / 2>(kb[b], qr, (j & 1) * (NC / 2), z0, z1);
                    if ((j & 1) == 0) return;
                    const f4 z = z0 + z1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bool ok = ed.h[2 * c1 + (e >> 1)] && ed.w[2 * c2 + (e & 1)];
                        if constexpr (MASK) ok = ok && walk_bit(wb, 2 * c1 + (e >> 1), 2 * c2 + (e & 1));
                        s[i][e] = ok ? z[e] : -INFINITY;
                    }
                    mj = fmaxf(mj, fmaxf(fmaxf(s[i][0], s[i][1]), fmaxf(s[i][2], s[i][3])));
                    pin4(s[i]);
                    asm volatile("" : "+v"(mj));
                });
        }
        if constexpr (T3) {
            const float mn = fmaxf(m, mj);
            const float alpha = fast_exp2(m - mn);
            l *= alpha;
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] *= alpha;
            m = mn;
        } else {
            m = mj;
        }
        __syncthreads();
        stage_plane<T, D, PS>(a.v, w, tk, U[1], E[1], U[2], E[2], rb, smem);
        stage_wait();

        // O_b[i][c] += v_e[dim(i, g)] * P[c][e]
        {
            f4 vb[2][2][D / 16];
            float p[4];
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_row_dmajor<D, PS>(baseB + (2 * (i / CW) + (j & 1)) * rb, 2 * (i % CW) * PS,
                                       vb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1, h = j & 1;
                    if (h == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(s[i][e] - m);
                        l += (p[0] + p[1]) + (p[2] + p[3]);
                    }
                    axpy_row<D>(vb[b], p[2 * h], p[2 * h + 1], acc);
                });
        }
    }

    if (L.active) {
        // a query whose window is masked away entirely: zero output, lse -inf
        store_row<T, D>(a.out + qo, acc, l > 0.f ? 1.f / l : 0.f);
        a.lse[row_off(w, L.p)] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// ============================================================================
// Backward, query side: delta and dq.
// PAD: points one 16-byte slot apart in LDS (row pitch 2 mod 4 slots), which
// makes key-major and d-major reads both conflict-free, so K is staged once
// for both of its uses. Without it K is staged once as well when the plan
// gives both layouts one pitch (the d-major reads then take bank conflicts),
// else once per layout.
template <typename T, int D, int CH, int CW, bool T3, bool PAD, bool MASK = false>
__device__ __forceinline__ void dq_tile(const BwdArgsT<T> &a, int tile, char *smem) {
    constexpr int PS = D * 4 + (PAD ? 16 : 0), NC = D / 4, G = D / 4, NI = CH * CW;
    TileCtx w;
    if (!decode(a.g, tile, w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3;
    const Lane L = lane_geom(w, wave, lane);

    int us[3], lo[3], U[3], E[3];
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        us[x] = window_start(L.f[x], w.n[x], w.k[x]);
        lo[x] = window_start(L.p[x], w.n[x], w.k[x]) - us[x];
        key_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], &U[x], &E[x]);
    }
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    Edge<CH, CW> ed;
#pragma unroll
    for (int r = 0; r < 2 * CH; ++r) ed.h[r] = walk_row_valid<CH>(r, lo[1], w.k[1]);
#pragma unroll
    for (int r = 0; r < 2 * CW; ++r) ed.w[r] = walk_row_valid<CW>(r, lo[2], w.k[2]);
    // frames along H (2D grids): walk rows outside the query row's frame window
    // are masked; along T (3D grids) whole key planes are skipped below
    if (a.frame && a.frame_axis == 1) {
        const unsigned fb = frame_bits(us[1], L.p[1], w.n[1], frame_size(a.frame, w, 1, L.p[1]));
#pragma unroll
        for (int r = 0; r < 2 * CH; ++r) ed.h[r] = ed.h[r] && ((fb >> r) & 1u);
    }
    const int fk_t = (a.frame && a.frame_axis == 0) ? frame_size(a.frame, w, 0, w.o[0]) : 0;

    const int ra = a.g.ra, rb = a.g.rb;
    const char *baseA = smem + (us[1] - U[1] + (c >> 1)) * ra + (us[2] - U[2] + (c & 1)) * PS;
    const char *baseB = smem + (us[1] - U[1]) * rb + (us[2] - U[2]) * PS + c * 16;

    const int64_t qo = elem_off(w, L.p);
    const int64_t ro = row_off(w, L.p);
    float delta = 0.f;
    {
        float dor[D], orow[D];
        load_row<T, D>(a.dout + qo, dor);
        load_row<T, D>(a.out + qo, orow);
#pragma unroll
        for (int d = 0; d < D; ++d) delta += dor[d] * orow[d];
    }
    if (L.active) a.delta[ro] = delta;
    const float lse2 = a.lse[ro] * kLog2e;

    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    const int nplanes = T3 ? w.k[0] : 1;
    for (int j = 0; j < nplanes; ++j) {
        const int tk = plane_of_step(t0, nplanes, j);
        if (a.frame && a.frame_axis == 0 && !in_frame(tk, w.o[0], w.n[0], fk_t)) continue;
        if (j > 0) __syncthreads();
        stage_plane<T, D, PS>(a.v, w, tk, U[1], E[1], U[2], E[2], ra, smem);
        float dor[D];
        load_row<T, D>(a.dout + qo + opaque_zero(), dor);
        stage_wait();

        // dP_b[i][c] = <v_i, dout_c>
        float s[NI][4];
        {
            f4 kb[2][NC / 2], z0, z1;
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (j & 1) * (NC / 2) * 16, kb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1;
                    if ((j & 1) == 0) z0 = z1 = f4{0.f, 0.f, 0.f, 0.f};
                    dot_half<NC / 2>(kb[b], dor, (j & 1) * (NC / 2), z0, z1);
                    if ((j & 1) == 0) return;
                    const f4 z = z0 + z1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[i][e] = z[e];
                    pin4(s[i]);
                });
        }
        __syncthreads();
        stage_plane<T, D, PS>(a.k, w, tk, U[1], E[1], U[2], E[2], ra, smem);
        float qr[D];
        load_row<T, D>(a.q + qo + opaque_zero(), qr);
#pragma unroll
        for (int d = 0; d < D; ++d) qr[d] *= a.qscale;
        uint32_t wb[MASK ? CH : 1];
        if constexpr (MASK)
            walk_mask_bits<CH, CW>(a.mask, a.mask_bytes,
                                   mask_row_base(w, a.g.ext, L.p, a.mask_k) +
                                       (int64_t)(tk - t0) * w.k[1] * w.k[2],
                                   w.k[1], w.k[2], lo[1], lo[2], wb);
        stage_wait();

        // P = exp2(S - lse), dS = P (dP - delta)
        {
            f4 kb[2][NC / 2], z0, z1;
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (j & 1) * (NC / 2) * 16, kb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1, c1 = i / CW, c2 = i % CW;
                    if ((j & 1) == 0) z0 = z1 = f4{0.f, 0.f, 0.f, 0.f};
                    dot_half<NC / 2>(kb[b], qr, (j & 1) * (NC / 2), z0, z1);
                    if ((j & 1) == 0) return;
                    const f4 z = z0 + z1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bool ok = ed.h[2 * c1 + (e >> 1)] && ed.w[2 * c2 + (e & 1)];
                        if constexpr (MASK) ok = ok && walk_bit(wb, 2 * c1 + (e >> 1), 2 * c2 + (e & 1));
                        const float p = ok ? fast_exp2(z[e] - lse2) : 0.f;
                        s[i][e] = p * (s[i][e] - delta);
                    }
                    pin4(s[i]);
                });
        }
        // the d-major layout: a restaging unless both layouts share the pitch
        if constexpr (!PAD) {
            if (rb != ra) {
                __syncthreads();
                stage_plane<T, D, PS>(a.k, w, tk, U[1], E[1], U[2], E[2], rb, smem);
                stage_wait();
            }
        }

        // dQ_b[i][c] += k_e[dim(i, g)] * dS[c][e]
        {
            f4 vb[2][2][D / 16];
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_row_dmajor<D, PS>(baseB + (2 * (i / CW) + (j & 1)) * rb, 2 * (i % CW) * PS,
                                       vb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1, h = j & 1;
                    axpy_row<D>(vb[b], s[i][2 * h], s[i][2 * h + 1], acc);
                });
        }
    }

    if (L.active) store_row<T, D>(a.dq + qo, acc, a.scale);
}

// The mask bits of the queries of a key's inverse walk (dk/dv with a window
// mask): bit (r & 1) * 16 + q of word r / 2 for walk row r, column q, the
// query at (lo1 + r, lo2 + q) of plane tq (class coordinates): that query's
// mask byte for this key's place in its window. Only the queries of the key's
// inverse window (vm) are read; the others get zero bits (their bytes are
// read from the mask's first byte, so that the loads need no branches).
template <typename T, int CH, int CW>
__device__ __forceinline__ void inverse_walk_mask_bits(const BwdArgsT<T> &a, const TileCtx &w,
                                                       const int (&key)[3], int tq,
                                                       const int (&lo)[3], const unsigned (&vm)[3],
                                                       uint32_t (&mb)[CH]) {
    const int64_t H = a.g.ext[1], W = a.g.ext[2], K = a.mask_k;
    const int kh = w.k[1], kw = w.k[2];
    const int64_t tabs = w.r[0] + (int64_t)w.d[0] * tq;
    const int jt = key[0] - window_start(tq, w.n[0], w.k[0]);
    const int64_t base = ((tabs * H + w.r[1] + (int64_t)w.d[1] * lo[1]) * W + w.r[2] +
                          (int64_t)w.d[2] * lo[2]) * K + (int64_t)jt * kh * kw;
    int64_t rowo[2 * CH];
    int colo[2 * CW];
#pragma unroll
    for (int r = 0; r < 2 * CH; ++r) {
        const int qh = imin(lo[1] + r, w.n[1] - 1);
        rowo[r] = base + r * w.d[1] * W * K + (int64_t)(key[1] - window_start(qh, w.n[1], kh)) * kw;
    }
#pragma unroll
    for (int q = 0; q < 2 * CW; ++q) {
        const int qw = imin(lo[2] + q, w.n[2] - 1);
        colo[q] = q * w.d[2] * (int)K + key[2] - window_start(qw, w.n[2], kw);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) mb[i] = 0u;
#pragma unroll
    for (int r = 0; r < 2 * CH; ++r)
#pragma unroll
        for (int q = 0; q < 2 * CW; ++q) {
            const bool in = ((vm[1] >> r) & (vm[2] >> q) & 1u) != 0;
            const uint8_t b = a.mask[in ? rowo[r] + colo[q] : 0];
            if (in && b) mb[r >> 1] |= 1u << ((r & 1) * 16 + q);
        }
}

// ============================================================================
// Backward, key side: dk and dv by inverse-neighborhood gather, without
// atomics. Every block walks CH x CW query patches; entries outside a key's
// inverse window are masked, and the staged box covers the whole walk of
// every block (points past the grid repeat real data), so masked reads are
// always finite. Near a grid border the window shift makes inverse
// neighborhoods longer: a launch takes the tiles whose longest inverse walk
// lies in (walk_lo, C]; longer ones are left to another launch.
__device__ __forceinline__ int tile_walk(const TileCtx &w) {
    return imax(tile_inverse_walk(w.o[1], kTH, 2, w.n[1], w.k[1]),
                tile_inverse_walk(w.o[2], kTW, 2, w.n[2], w.k[2]));
}

// PAD: as for dq_tile; dout is then staged once for dV and dS. MASK: the
// window mask of a.mask as well (inverse_walk_mask_bits).
template <typename T, int D, int CH, int CW, bool T3, bool PAD, bool MASK = false>
__device__ __forceinline__ void dkdv_tile(const BwdArgsT<T> &a, int tile, char *smem) {
    constexpr int PS = D * 4 + (PAD ? 16 : 0), NC = D / 4, G = D / 4, NI = CH * CW;
    TileCtx w;
    if (!decode(a.g, tile, w)) return;
    if (a.edge >= 0) {
        const int wh = tile_inverse_walk(w.o[1], kTH, 2, w.n[1], w.k[1]);
        const int ww = tile_inverse_walk(w.o[2], kTW, 2, w.n[2], w.k[2]);
        if ((wh > a.walk_c) != ((a.edge & 1) != 0) || (ww > a.walk_c) != ((a.edge & 2) != 0) ||
            wh > CH || ww > CW)
            return;
    } else {
        const int tw = tile_walk(w);
        if (tw <= a.walk_lo || tw > (CH > CW ? CH : CW)) return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3;
    const Lane L = lane_geom(w, wave, lane);  // keys

    int lo[3], U[3], E[3];
    unsigned vm[3];
#pragma unroll
    for (int x = 1; x < 3; ++x) {
        query_box(w.o[x], x == 1 ? kTH : kTW, 2, w.n[x], w.k[x], x == 1 ? CH : CW, &U[x], &E[x]);
        lo[x] = inverse_first(L.f[x], w.n[x], w.k[x]);
        const int ilo = inverse_first(L.p[x], w.n[x], w.k[x]);
        vm[x] = bit_range(ilo - lo[x], inverse_last(L.p[x], w.n[x], w.k[x]) - ilo + 1);
    }
    const int tq0 = inverse_first(w.o[0], w.n[0], w.k[0]);
    const int tq1 = inverse_last(w.o[0], w.n[0], w.k[0]);
    // frames along H (2D grids): query rows whose frame window misses the key
    // row are masked; along T (3D grids) whole query planes are skipped below
    if (a.frame && a.frame_axis == 1)
        vm[1] &= frame_bits_inverse(a.frame, w, 1, lo[1], L.p[1], w.n[1], 2 * CH);

    const int ra = a.g.ra, rb = a.g.rb;
    const char *baseA = smem + (lo[1] - U[1] + (c >> 1)) * ra + (lo[2] - U[2] + (c & 1)) * PS;
    const char *baseB = smem + (lo[1] - U[1]) * rb + (lo[2] - U[2]) * PS + c * 16;
    const int rp = a.g.rows_pitch;
    const float2 *baseR = reinterpret_cast<const float2 *>(smem + a.g.rows_off) +
                          (lo[1] - U[1] + (c >> 1)) * rp + (lo[2] - U[2] + (c & 1));

    const int64_t ko = elem_off(w, L.p);

    f4 dk[G], dv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        dk[g] = f4{0.f, 0.f, 0.f, 0.f};
        dv[g] = f4{0.f, 0.f, 0.f, 0.f};
    }

    const int nplanes = T3 ? tq1 - tq0 + 1 : 1;
    for (int j = 0; j < nplanes; ++j) {
        const int tq = plane_of_step(tq0, nplanes, j);
        if (a.frame && a.frame_axis == 0 &&
            !in_frame(w.o[0], tq, w.n[0], frame_size(a.frame, w, 0, tq)))
            continue;
        if (j > 0) __syncthreads();
        stage_plane<T, D, PS>(a.q, w, tq, U[1], E[1], U[2], E[2], ra, smem);
        stage_rows_plane(a.lse, a.delta, w, tq, U[1], E[1], U[2], E[2], rp,
                         reinterpret_cast<float2 *>(smem + a.g.rows_off));
        uint32_t mb[MASK ? CH : 1];
        if constexpr (MASK) inverse_walk_mask_bits<T, CH, CW>(a, w, L.p, tq, lo, vm, mb);
        float kr[D];
        load_row<T, D>(a.k + ko + opaque_zero(), kr);
#pragma unroll
        for (int d = 0; d < D; ++d) kr[d] *= a.qscale;
        stage_wait();

        // S_b[i][c] = <q_i, k_c> - lse_i (the lse term is one more MFMA step:
        // lane 4b+i supplies -lse of its entry, every lane 1); P, masked
        float s[NI][4];
        {
            f4 kb[2][NC / 2], z0, z1;
            float lr[2];
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (j & 1) * (NC / 2) * 16, kb[b]);
                    if ((j & 1) == 0) lr[b] = baseR[2 * (i / CW) * rp + 2 * (i % CW)].x;
                },
                [&](int j, int b) {
                    const int i = j >> 1, c1 = i / CW, c2 = i % CW;
                    if ((j & 1) == 0) {
                        z0 = mfma4(-lr[b], 1.f, f4{0.f, 0.f, 0.f, 0.f});
                        z1 = f4{0.f, 0.f, 0.f, 0.f};
                    }
                    dot_half<NC / 2>(kb[b], kr, (j & 1) * (NC / 2), z0, z1);
                    if ((j & 1) == 0) return;
                    const f4 z = z0 + z1;
                    const unsigned hb = vm[1] >> (2 * c1), wb = vm[2] >> (2 * c2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bool ok = ((hb >> (e >> 1)) & (wb >> (e & 1)) & 1u) != 0;
                        if constexpr (MASK) ok = ok && walk_bit(mb, 2 * c1 + (e >> 1), 2 * c2 + (e & 1));
                        s[i][e] = ok ? fast_exp2(z[e]) : 0.f;
                    }
                    pin4(s[i]);
                });
        }
        __syncthreads();
        stage_plane<T, D, PS>(a.dout, w, tq, U[1], E[1], U[2], E[2], rb, smem);
        stage_wait();

        // dV_b[i][c] += dout_e[dim(i, g)] * P[c][e]
        {
            f4 vb[2][2][D / 16];
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_row_dmajor<D, PS>(baseB + (2 * (i / CW) + (j & 1)) * rb, 2 * (i % CW) * PS,
                                       vb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1, h = j & 1;
                    axpy_row<D>(vb[b], s[i][2 * h], s[i][2 * h + 1], dv);
                });
        }
        // one plane: dv is final here; storing it now frees its registers
        if constexpr (!T3)
            if (L.active) store_row<T, D>(a.dv + ko, dv, 1.f);
        float vr[D];
        // the key-major layout: a restaging unless both layouts share the pitch
        const bool restage = !PAD && rb != ra;
        if (restage) {
            __syncthreads();
            stage_plane<T, D, PS>(a.dout, w, tq, U[1], E[1], U[2], E[2], ra, smem);
        }
        load_row<T, D>(a.v + ko + opaque_zero(), vr);
        if (restage) stage_wait();

        // dP_b[i][c] = <dout_i, v_c> - delta_i;  dS = P dP
        {
            f4 kb[2][NC / 2], z0, z1;
            float dr[2];
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_chunks<NC / 2>(baseA + 2 * (i / CW) * ra + 2 * (i % CW) * PS +
                                            (j & 1) * (NC / 2) * 16, kb[b]);
                    if ((j & 1) == 0) dr[b] = baseR[2 * (i / CW) * rp + 2 * (i % CW)].y;
                },
                [&](int j, int b) {
                    const int i = j >> 1;
                    if ((j & 1) == 0) {
                        z0 = mfma4(-dr[b], 1.f, f4{0.f, 0.f, 0.f, 0.f});
                        z1 = f4{0.f, 0.f, 0.f, 0.f};
                    }
                    dot_half<NC / 2>(kb[b], vr, (j & 1) * (NC / 2), z0, z1);
                    if ((j & 1) == 0) return;
                    const f4 z = z0 + z1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[i][e] *= z[e];
                    pin4(s[i]);
                });
        }
        __syncthreads();
        stage_plane<T, D, PS>(a.q, w, tq, U[1], E[1], U[2], E[2], rb, smem);
        stage_wait();

        // dK_b[i][c] += q_e[dim(i, g)] * dS[c][e]
        {
            f4 vb[2][2][D / 16];
            pipelined<2 * NI>(
                [&](int j, int b) {
                    const int i = j >> 1;
                    load_row_dmajor<D, PS>(baseB + (2 * (i / CW) + (j & 1)) * rb, 2 * (i % CW) * PS,
                                       vb[b]);
                },
                [&](int j, int b) {
                    const int i = j >> 1, h = j & 1;
                    axpy_row<D>(vb[b], s[i][2 * h], s[i][2 * h + 1], dk);
                });
        }
    }

    if (L.active) {
        store_row<T, D>(a.dk + ko, dk, a.scale);
        if constexpr (T3) store_row<T, D>(a.dv + ko, dv, 1.f);
    }
}

// ============================================================================
// Kernels: one workgroup per tile.
template <typename T, int D, int CH, int CW, bool T3, bool MASK = false>
__global__ void __launch_bounds__(kThreads, 2) fwd_kernel(FwdArgsT<T> a) {
    extern __shared__ __align__(16) char smem[];
    fwd_tile<T, D, CH, CW, T3, MASK>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

template <typename T, int D, int CH, int CW, bool T3, bool PAD, bool MASK = false>
__global__ void __launch_bounds__(kThreads, 2) dq_kernel(BwdArgsT<T> a) {
    extern __shared__ __align__(16) char smem[];
    dq_tile<T, D, CH, CW, T3, PAD, MASK>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

template <typename T, int D, int CH, int CW, bool T3, bool PAD, bool MASK = false>
__global__ void __launch_bounds__(kThreads, 2) dkdv_kernel(BwdArgsT<T> a) {
    extern __shared__ __align__(16) char smem[];
    dkdv_tile<T, D, CH, CW, T3, PAD, MASK>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

// The same for the few border tiles with a longer walk: one workgroup per CU,
// so that the longer walk never spills registers.
template <typename T, int D, int CH, int CW, bool T3, bool PAD, bool MASK = false>
__global__ void __launch_bounds__(kThreads, 1) dkdv_border_kernel(BwdArgsT<T> a) {
    extern __shared__ __align__(16) char smem[];
    dkdv_tile<T, D, CH, CW, T3, PAD, MASK>(a, xcd_tile_id(blockIdx.x, a.g.n_tiles), smem);
}

}  // namespace fast
}  // namespace na
