// na_common.hpp -- types, element I/O, tile geometry and LDS staging shared by
// the neighborhood-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "na_index.hpp"

namespace na {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16;  // storage of a bfloat16 value
typedef _Float16 f16;   // IEEE binary16
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------------------
// Element I/O. Tensors are fp32 or bf16; arithmetic is always fp32.

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even (values are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename T>
struct Io;

template <>
struct Io<float> {
    static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
    __device__ __forceinline__ static void load4(const float *p, float *d) {
        float4 v = *reinterpret_cast<const float4 *>(p);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __device__ __forceinline__ static void store4(float *p, const float *s) {
        *reinterpret_cast<float4 *>(p) = make_float4(s[0], s[1], s[2], s[3]);
    }
    // a 16-byte LDS chunk to fp32
    __device__ __forceinline__ static void chunk(const char *lds, float *d) {
        float4 v = *reinterpret_cast<const float4 *>(lds);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    // 4 elements (half chunk never needed for fp32)
    __device__ __forceinline__ static void quad(const char *lds, float *d) { chunk(lds, d); }
};

template <>
struct Io<bf16> {
    static constexpr int kPerChunk = 8;
    __device__ __forceinline__ static void load4(const bf16 *p, float *d) {
        uint2 v = *reinterpret_cast<const uint2 *>(p);
        d[0] = bf16_to_f32(v.x & 0xffffu); d[1] = bf16_to_f32(v.x >> 16);
        d[2] = bf16_to_f32(v.y & 0xffffu); d[3] = bf16_to_f32(v.y >> 16);
    }
    __device__ __forceinline__ static void store4(bf16 *p, const float *s) {
        uint2 v;
        v.x = f32_to_bf16(s[0]) | (f32_to_bf16(s[1]) << 16);
        v.y = f32_to_bf16(s[2]) | (f32_to_bf16(s[3]) << 16);
        *reinterpret_cast<uint2 *>(p) = v;
    }
    __device__ __forceinline__ static void chunk(const char *lds, float *d) {
        uint4 v = *reinterpret_cast<const uint4 *>(lds);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[2 * i] = bf16_to_f32(w[i] & 0xffffu);
            d[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
    __device__ __forceinline__ static void quad(const char *lds, float *d) {
        uint2 v = *reinterpret_cast<const uint2 *>(lds);
        d[0] = bf16_to_f32(v.x & 0xffffu); d[1] = bf16_to_f32(v.x >> 16);
        d[2] = bf16_to_f32(v.y & 0xffffu); d[3] = bf16_to_f32(v.y >> 16);
    }
};

template <>
struct Io<f16> {
    static constexpr int kPerChunk = 8;
    __device__ __forceinline__ static float cvt(uint32_t h) {
        return (float)__builtin_bit_cast(f16, (uint16_t)h);
    }
    // round to nearest, ties to even (the default rounding mode of the conversion)
    __device__ __forceinline__ static uint32_t bits(float f) {
        return __builtin_bit_cast(uint16_t, (f16)f);
    }
    __device__ __forceinline__ static void load4(const f16 *p, float *d) {
        uint2 v = *reinterpret_cast<const uint2 *>(p);
        d[0] = cvt(v.x & 0xffffu); d[1] = cvt(v.x >> 16);
        d[2] = cvt(v.y & 0xffffu); d[3] = cvt(v.y >> 16);
    }
    __device__ __forceinline__ static void store4(f16 *p, const float *s) {
        uint2 v;
        v.x = bits(s[0]) | (bits(s[1]) << 16);
        v.y = bits(s[2]) | (bits(s[3]) << 16);
        *reinterpret_cast<uint2 *>(p) = v;
    }
    __device__ __forceinline__ static void chunk(const char *lds, float *d) {
        uint4 v = *reinterpret_cast<const uint4 *>(lds);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[2 * i] = cvt(w[i] & 0xffffu);
            d[2 * i + 1] = cvt(w[i] >> 16);
        }
    }
    __device__ __forceinline__ static void quad(const char *lds, float *d) {
        uint2 v = *reinterpret_cast<const uint2 *>(lds);
        d[0] = cvt(v.x & 0xffffu); d[1] = cvt(v.x >> 16);
        d[2] = cvt(v.y & 0xffffu); d[3] = cvt(v.y >> 16);
    }
};

// Load N (a multiple of 4) consecutive elements into fp32 registers.
template <typename T, int N>
__device__ __forceinline__ void load_row(const T *p, float (&d)[N]) {
#pragma unroll
    for (int c = 0; c < N; c += 4) Io<T>::load4(p + c, d + c);
}

// ----------------------------------------------------------------------------
// MFMA: v_mfma_f32_4x4x1_16b_f32. Sixteen independent 4x4 outer products per
// wave; lane l belongs to block b = l / 4 with index c = l % 4:
//   A_b[c] = a (lane 4b+c),  B_b[c] = b (lane 4b+c),
//   D_b[i][c] = C_b[i][c] + A_b[i] * B_b[c], row i in result register i of
//   lane 4b+c.
// With A a key-indexed operand and B a query-indexed one, lane 4b+c ends up
// holding the products of its own query c with the 4 keys of its block, one
// per register.
__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// Bits [lo, lo + len) set (len >= 0, lo + len <= 32).
__device__ __forceinline__ unsigned bit_range(int lo, int len) {
    const unsigned ones = len >= 32 ? 0xffffffffu : ((1u << len) - 1u);
    return ones << lo;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------
// Division by a launch constant: m = ceil(2^32 / d) makes floor(n * m / 2^32)
// either floor(n / d) or one more (for 0 <= n < 2^31), which one comparison
// corrects; a few scalar instructions instead of a full integer division.
struct FastDiv {
    uint32_t d, m;  // m = 0: d = 1
};

NA_HD FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.m = d <= 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + d - 1) / d);
    return f;
}

__device__ __forceinline__ int fdiv(int n, const FastDiv &f) {
    if (f.m == 0) return n;
    const uint32_t q = __umulhi((uint32_t)n, f.m);
    return (int)(q - (q * f.d > (uint32_t)n));
}

// ----------------------------------------------------------------------------
// Tiles. Axis 0 is T (1 for 2D problems), axis 1 is H, axis 2 is W, all in
// class coordinates of one residue class (dilation). A workgroup of kWaves
// waves owns a tile of 1 x 8 x 8 points (64: one per lane), split into sixteen
// 1 x 2 x 2 patches, one per 4-lane MFMA block; all waves of the workgroup
// hold the same 64 points and split the other side's patches between them.

constexpr int kPatch[3] = {1, 2, 2};
constexpr int kTile[3] = {1, 8, 8};
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// The 16 x 16 (H, W) tiles near the borders of a dilation-1 grid: tile rows
// [0, rows_lo) and [R - rows_hi, R), tile columns [0, cols_lo) and
// [C - cols_hi, C), of R x C tiles per plane. Near a border the window shift
// makes inverse neighborhoods longer, and only these tiles need the kernels for
// longer inverse walks; a launch over them enumerates them directly instead of
// starting (and ending) a workgroup for every tile.
struct Border {
    int on;                          // the launch covers the border tiles only
    int rows_lo, rows_hi, cols_lo, cols_hi;
    int per_plane;                   // border tiles per (batch, head, T) plane
    // 0: every tile of the frame; otherwise one class of it: rows from the
    // bands (bit 0 set) or between them, columns likewise (bit 1)
    int cls;
};

// Border tile i (0 .. per_plane - 1) of a plane of R x C tiles: (row, col).
__device__ __forceinline__ void border_tile(const Border &bd, int R, int C, int i, int &r, int &c) {
    const int rb = bd.rows_lo + bd.rows_hi, cb = bd.cols_lo + bd.cols_hi;
    if (i < rb * C) {
        const int rr = i / C;
        c = i - rr * C;
        r = rr < bd.rows_lo ? rr : R - bd.rows_hi + (rr - bd.rows_lo);
    } else {
        i -= rb * C;
        const int q = i / cb, cc = i - q * cb;
        r = bd.rows_lo + q;
        c = cc < bd.cols_lo ? cc : C - bd.cols_hi + (cc - bd.cols_lo);
    }
}

struct Geometry {
    int ext[3], ker[3], dil[3];
    int heads, batch, head_dim;
    int tiles[3];     // tiles per axis, over the largest residue class
    int nres;         // dil[0] * dil[1] * dil[2]
    int n_tiles;      // batch * heads * nres * tiles[0] * tiles[1] * tiles[2] (or the border tiles)
    int chunk_axis;   // axis along which a staged box is split when it exceeds the budget
    int lds_budget;   // bytes of LDS a staged chunk may use
    Border border;    // when on: the 8 x 8 tiles of the border 16 x 16 tiles only
    int dq_lds_off;   // KV-parallel dk/dv: byte offset of the LDS dq accumulator (0: none)
};

// Where a workgroup works: batch element, head, residue class, tile origin,
// and the address arithmetic of that class.
struct TileCtx {
    int n[3], k[3];     // class sizes and window sizes per axis
    int o[3];           // tile origin in class coordinates
    int r[3], d[3];     // residue class and dilation per axis (absolute = r + d * class)
    int64_t base;       // element offset of (b, class origin token, head, 0)
    int64_t st[3];      // element offset of one class step per axis
    int64_t lbase;      // lse / delta offset of (b, class origin token, head)
    int64_t lst[3];     // lse / delta offset of one class step per axis
};

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2. Renumber them so that every XCD walks one contiguous run of tiles:
// neighbouring tiles share most of their halo, which then hits in that XCD's
// L2. The map is a bijection of [0, n).
__device__ __forceinline__ int xcd_tile_id(int bid, int n) {
    const int xcd = bid & 7, j = bid >> 3;
    const int q = n >> 3, r = n & 7;
    return xcd < r ? xcd * (q + 1) + j : r * (q + 1) + (xcd - r) * q + j;
}

// Decodes a tile id. Within one (batch, head, residue, T-tile) plane the
// tiles are walked in bands kBand tiles wide along W, row by row inside a
// band, so a tile's upper neighbour was staged at most kBand tiles earlier
// (its halo is then still in L2); then T, residue, head, batch.
// Returns false when the tile lies past the end of its residue class.
constexpr int kBand = 32;

// Fills w for batch element b, head, residue class res and tile origin o
// (class coordinates); false when the origin lies past the end of its class.
__device__ __forceinline__ bool fill_ctx(const int (&ext)[3], const int (&ker)[3],
                                         const int (&dil)[3], int heads, int head_dim, int b,
                                         int head, int res, const int (&o)[3], TileCtx &w) {
    int r[3];
    r[2] = res % dil[2];
    r[1] = (res / dil[2]) % dil[1];
    r[0] = res / (dil[2] * dil[1]);
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        w.n[a] = class_size(ext[a], dil[a], r[a]);
        w.k[a] = ker[a];
        w.o[a] = o[a];
        w.r[a] = r[a];
        w.d[a] = dil[a];
        inside = inside && (o[a] < w.n[a]);
    }
    const int64_t HW = (int64_t)ext[1] * ext[2];
    const int64_t ntok = HW * ext[0];
    const int64_t hd = (int64_t)heads * head_dim;
    const int64_t origin_tok = r[0] * HW + (int64_t)r[1] * ext[2] + r[2];
    w.base = ((int64_t)b * ntok + origin_tok) * hd + (int64_t)head * head_dim;
    w.st[0] = dil[0] * HW * hd;
    w.st[1] = (int64_t)dil[1] * ext[2] * hd;
    w.st[2] = (int64_t)dil[2] * hd;
    w.lbase = ((int64_t)b * ntok + origin_tok) * heads + head;
    w.lst[0] = dil[0] * HW * heads;
    w.lst[1] = (int64_t)dil[1] * ext[2] * heads;
    w.lst[2] = (int64_t)dil[2] * heads;
    return inside;
}

__device__ __forceinline__ bool decode_tile(const Geometry &g, int tile, TileCtx &w) {
    if (g.border.on) {
        // four 8 x 8 tiles per border 16 x 16 tile, then head, T, batch
        const int sub = tile & 3;
        int rem = tile >> 2;
        const int head = rem % g.heads;
        rem /= g.heads;
        const int tt = rem % g.tiles[0];
        rem /= g.tiles[0];
        const int R = (g.tiles[1] + 1) >> 1, C = (g.tiles[2] + 1) >> 1;
        int r, c;
        border_tile(g.border, R, C, rem % g.border.per_plane, r, c);
        const int b = rem / g.border.per_plane;
        const int o[3] = {tt * kTile[0], 16 * r + 8 * (sub >> 1), 16 * c + 8 * (sub & 1)};
        return fill_ctx(g.ext, g.ker, g.dil, g.heads, g.head_dim, b, head, 0, o, w);
    }
    const int plane = g.tiles[1] * g.tiles[2];
    int rem = tile / plane;
    int in = tile - rem * plane;
    const int band = in / (kBand * g.tiles[1]);
    const int bw = imin(kBand, g.tiles[2] - band * kBand);   // width of this band
    in -= band * kBand * g.tiles[1];
    const int th = in / bw;
    const int tw = band * kBand + (in - th * bw);
    const int tt = rem % g.tiles[0];
    rem /= g.tiles[0];
    const int res = rem % g.nres;
    rem /= g.nres;
    const int head = rem % g.heads;
    const int b = rem / g.heads;
    const int o[3] = {tt * kTile[0], th * kTile[1], tw * kTile[2]};
    return fill_ctx(g.ext, g.ker, g.dil, g.heads, g.head_dim, b, head, res, o, w);
}

__device__ __forceinline__ int64_t elem_off(const TileCtx &w, const int (&c)[3]) {
    return w.base + c[0] * w.st[0] + c[1] * w.st[1] + c[2] * w.st[2];
}
__device__ __forceinline__ int64_t row_off(const TileCtx &w, const int (&c)[3]) {
    return w.lbase + c[0] * w.lst[0] + c[1] * w.lst[1] + c[2] * w.lst[2];
}

// Coordinates of entry c (0..3) of the 1x2x2 patch whose first point is f.
__device__ __forceinline__ void patch_point(const int (&f)[3], int c, int (&p)[3]) {
    p[0] = f[0];
    p[1] = f[1] + (c >> 1);
    p[2] = f[2] + (c & 1);
}

// The point a lane owns in its workgroup's tile, and its patch.
struct LanePoint {
    int f[3];     // first point of the lane's patch (clamped into the grid)
    int l[3];     // last point of the lane's patch (clamped into the grid)
    int p[3];     // the lane's own point (clamped into the grid)
    bool active;  // the unclamped point lies inside the grid
};

__device__ __forceinline__ LanePoint lane_point(const TileCtx &w, int lane) {
    const int grp = lane >> 2, c = lane & 3;
    int f[3] = {w.o[0], w.o[1] + 2 * (grp >> 2), w.o[2] + 2 * (grp & 3)};
    int p[3];
    patch_point(f, c, p);
    LanePoint lp;
    lp.active = p[0] < w.n[0] && p[1] < w.n[1] && p[2] < w.n[2];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        lp.f[a] = imin(f[a], w.n[a] - 1);
        lp.l[a] = imin(f[a] + kPatch[a] - 1, w.n[a] - 1);
        lp.p[a] = imin(p[a], w.n[a] - 1);
    }
    return lp;
}

// Tile extent clamped to the grid: first and last point per axis.
__device__ __forceinline__ void tile_span(const TileCtx &w, int (&f)[3], int (&l)[3]) {
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        f[a] = w.o[a];
        l[a] = imin(w.o[a] + kTile[a] - 1, w.n[a] - 1);
    }
}

// ----------------------------------------------------------------------------
// LDS staging of a box of points. A point (one (token, head) vector of D
// elements) takes D * sizeof(T) bytes = NC 16-byte chunks, points in row-major
// box order. Chunk s of a point sits at slot s ^ swz(point).
//
// Bank model (measured on gfx950): 16-byte reads of the 16 lanes of a quarter
// wave conflict when two of them hit the same 16-byte slot modulo 256 bytes.
// The swizzle keeps both read patterns of the kernels conflict-free for
// fp32 (NC = 8) and D = 64 (NC = 16):
//  * key-major: each lane reads chunk s of its own point; a quarter wave holds
//    four 1x2x2 patches side by side, i.e. a 2x8 block of points;
//  * d-major: the four lanes of a block read the four quarters of one point
//    of their patch, and the blocks of a quarter wave visit that point's
//    patch in orders differing in the w bit (see lds_quarter).
struct Box {
    int o[3];   // origin (class coordinates)
    int e[3];   // extents
};

template <int NC>
__device__ __forceinline__ int swz(int lh, int lw) {
    if constexpr (NC == 16) return ((lw >> 1) & 3) | ((lw & 1) << 2) | ((lh & 1) << 3);
    if constexpr (NC == 8) {
        const int x = lw >> 1;
        return ((x & 3) ^ ((x >> 1) & 1)) | ((lh & 1) << 2);
    }
    if constexpr (NC == 4) return ((lw >> 2) & 1) | ((lh & 1) << 1);
    return (lw >> 1) & (NC - 1);
}

template <int NC>
__device__ __forceinline__ constexpr int log2_of() {
    return NC == 16 ? 4 : NC == 8 ? 3 : NC == 4 ? 2 : NC == 2 ? 1 : 0;
}

// All threads of the workgroup copy the box of tensor src into lds with
// direct global-to-LDS loads, one box row at a time (16 bytes per lane, 64
// consecutive slots per wave instruction). Box points past the end of the
// grid (the box may overhang it by up to one patch) repeat the last grid
// point; they are never used unmasked. Completion: stage_wait().
//
// The per-lane part of an address (column, chunk, swizzle) only depends on
// the lane's slot in a row, so it is computed once per slot group ("part");
// the row only contributes a uniform base pointer and the parity of its H
// coordinate, which flips one swizzle bit.
template <typename T, int D>
__device__ __forceinline__ void stage_box(const T *src, const TileCtx &w, const Box &b,
                                          char *lds) {
    constexpr int PB = D * (int)sizeof(T), NC = PB / 16, LNC = log2_of<NC>();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int rowchunks = b.e[2] * NC;
    const int ipr = (rowchunks + 63) >> 6;
    const int rows = b.e[0] * b.e[1];
    const int hbit = swz<NC>(1, 0) << 4;   // byte offset flip of odd H rows
    const char *gsrc = reinterpret_cast<const char *>(src);
    for (int part = 0; part < ipr; ++part) {
        const int j = part * 64 + lane;
        const int lw = j >> LNC, slot = j & (NC - 1);
        if (lw >= b.e[2]) continue;
        const int c2 = imin(b.o[2] + lw, w.n[2] - 1);
        // byte offset of the lane's chunk within its row (even H rows)
        const int col = (int)(c2 * w.st[2]) * (int)sizeof(T) + ((slot ^ swz<NC>(0, lw)) << 4);
        for (int r = wave; r < rows; r += kWaves) {
            const int lt = r / b.e[1], lh = r - lt * b.e[1];
            const int c0 = imin(b.o[0] + lt, w.n[0] - 1), c1 = imin(b.o[1] + lh, w.n[1] - 1);
            const char *rowp = gsrc + (w.base + c0 * w.st[0] + c1 * w.st[1]) * (int64_t)sizeof(T);
            const int voff = col ^ ((lh & 1) ? hbit : 0);
#if defined(__HIP_DEVICE_COMPILE__)
            // the host pass of single-source HIP has no gfx950 builtins
            __builtin_amdgcn_global_load_lds(rowp + voff,
                                             (lds_void *)(lds + (r * rowchunks + part * 64) * 16),
                                             16, 0, 0);
#else
            (void)rowp;
            (void)voff;
#endif
        }
    }
}

// Per-point (logsumexp * log2(e), delta) pairs of a box, plain loads.
__device__ __forceinline__ void stage_rows(const float *lse, const float *delta, const TileCtx &w,
                                           const Box &b, float2 *lds) {
    const int np = b.e[0] * b.e[1] * b.e[2];
    const int e12 = b.e[1] * b.e[2];
    for (int i = threadIdx.x; i < np; i += kThreads) {
        const int lt = i / e12, rem = i - lt * e12;
        const int lh = rem / b.e[2], lw = rem - lh * b.e[2];
        const int c[3] = {imin(b.o[0] + lt, w.n[0] - 1), imin(b.o[1] + lh, w.n[1] - 1),
                          imin(b.o[2] + lw, w.n[2] - 1)};
        const int64_t ro = row_off(w, c);
        lds[i] = make_float2(lse[ro] * kLog2e, delta[ro]);
    }
}

__device__ __forceinline__ void stage_wait() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Byte offset of point (lh, lw) relative coordinates already folded into pt.
// Full point (D elements) from LDS, chunk by chunk.
template <typename T, int D>
__device__ __forceinline__ void lds_point(const char *lds, int pt, int sw, float (&d)[D]) {
    constexpr int PB = D * (int)sizeof(T), NC = PB / 16, EPC = 16 / (int)sizeof(T);
    const char *p = lds + pt * PB;
#pragma unroll
    for (int s = 0; s < NC; ++s) Io<T>::chunk(p + ((s ^ sw) << 4), d + s * EPC);
}

// Elements [c*G, c*G + G) (G = D / 4) of a point from LDS.
template <typename T, int D>
__device__ __forceinline__ void lds_quarter(const char *lds, int pt, int sw, int c,
                                            float (&d)[D / 4]) {
    constexpr int PB = D * (int)sizeof(T), EPC = 16 / (int)sizeof(T);
    constexpr int G = D / 4;
    const char *p = lds + pt * PB;
    if constexpr (G >= EPC) {
#pragma unroll
        for (int s = 0; s < G / EPC; ++s) {
            const int chunk = c * (G / EPC) + s;
            Io<T>::chunk(p + ((chunk ^ sw) << 4), d + s * EPC);
        }
    } else {
        // G = 4 < EPC = 8 (bf16, D = 16): half a chunk
        const int chunk = (c * G) / EPC, half = (c * G) % EPC;
        Io<T>::quad(p + ((chunk ^ sw) << 4) + half * (int)sizeof(T), d);
    }
}

// ----------------------------------------------------------------------------
// Windows restricted along one axis ("frames": T on 3D grids, H on 2D grids).
// frame[x], x an absolute coordinate along the frame axis, is the size of a
// window around x (the same centered-and-shifted rule, inside x's residue
// class) that the keys of the queries at x must also lie in along that axis;
// 0 masks every key. This is the NATTEN issue requester's per-frame time
// kernel, applied by index arithmetic: whole planes outside a tile's frame
// window are skipped, rows are masked.

__device__ __forceinline__ int pick3(const int (&v)[3], int a) {
    return a == 0 ? v[0] : (a == 1 ? v[1] : v[2]);
}

// Window size of class coordinate i along axis a (clamped to [0, k]).
__device__ __forceinline__ int frame_size(const int *frame, const TileCtx &w, int a, int i) {
    const int v = frame[pick3(w.r, a) + pick3(w.d, a) * i];
    return imin(imax(v, 0), pick3(w.k, a));
}

// Whether class coordinate key lies in the frame window of size fk around
// class coordinate query (n positions on the axis).
__device__ __forceinline__ bool in_frame(int key, int query, int n, int fk) {
    return fk > 0 && (unsigned)(key - window_start(query, n, fk)) < (unsigned)fk;
}

// Bits r (0..31) of the positions start + r lying in the frame window of
// query (a query's window walk).
__device__ __forceinline__ unsigned frame_bits(int start, int query, int n, int fk) {
    if (fk <= 0) return 0u;
    const int s = window_start(query, n, fk) - start;
    const int lo = imax(s, 0), hi = imin(s + fk, 32);
    return hi > lo ? bit_range(lo, hi - lo) : 0u;
}

// Bits r (0..len-1, len <= 32) of the queries at start + r whose frame window
// holds key (a key's inverse walk).
__device__ __forceinline__ unsigned frame_bits_inverse(const int *frame, const TileCtx &w, int a,
                                                       int start, int key, int n, int len) {
    unsigned m = 0u;
    for (int r = 0; r < len; ++r) {
        const int x = start + r;
        if (x >= 0 && x < n && in_frame(key, x, n, frame_size(frame, w, a, x))) m |= 1u << r;
    }
    return m;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) v = imax(v, __shfl_xor(v, m));
    return v;
}

}  // namespace na
