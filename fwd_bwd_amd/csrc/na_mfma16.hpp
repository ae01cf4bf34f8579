// na_mfma16.hpp -- neighborhood attention forward and backward for 16-bit
// tensors (bf16, fp16) on the gfx950 16-bit MFMA v_mfma_f32_16x16x32_{bf16,f16}
// (fp32 accumulation).
//
// The operation is that of NATTEN issue #161, "Backward pass is very slow
// towards much tokens and large kernels": per query a softmax over the scores
// scale * <q, k> of its window of keys, weighted sum of values; the backward
// recomputes the weights from the saved logsumexp, uses delta = rowsum(dO * O)
// (the maintainer's ComputeDelta) and forms dK, dV over each key's inverse
// neighborhood. The maintainer notes that fused attention is compute bound only
// at 16-bit precision; this is the path for those tensors.
//
// Work decomposition. A wave owns a patch of 16 points (1 x 4 x 4 along T, H,
// W in class coordinates of one residue class): queries in the forward and dq
// kernels, keys in the dk/dv kernel. A workgroup of eight waves owns a tile of
// patches (one plane of 1 x 8 x 16 on 2D grids; on 3D grids possibly several
// planes, see Geom), so its waves need rows of the same planes of the other
// side's box: the box is staged one 4-row slab of one plane at a time, and
// every wave walks the 4 x 4 blocks of its own patch's window union (or
// inverse union) inside the slab, skipping slabs outside it and planes outside
// its own plane's window.
// One MFMA contracts 16 points of one side with a 4 x 4 block of the other
// over 32 channels; pairs of blocks (32 points) form the 32-deep reductions of
// the weighted sums.
//
// Staging. Slabs are copied with direct global-to-LDS loads into one layout,
// key-major: each point's channels in 16-byte chunks, their order rotated by
// the slab row (and XOR-swizzled at 64 channels) so that both kinds of reads
// below are free of bank conflicts. With two slab buffers
// the next slab's loads are issued before the current slab is walked, so they
// run under the walk, and one barrier per slab orders the two.
//
// Operand layouts (lane l, lane group g = l / 16, n = l % 16):
//  * A (16 x 32) and B (32 x 16) operands: lane l holds row / column n and
//    reduction entries 8g .. 8g + 7; result C (16 x 16): lane l holds rows
//    4g .. 4g + 3 of column n.
//  * A block is 4 slab rows by 4 columns; its point m sits at row m % 4,
//    column m / 4. Scores are formed transposed, S^T = K Q^T: A = a key block
//    (point n's chunk of channels, one 16-byte LDS read), B = the wave's
//    queries (registers). Lane l then holds the scores of query n against
//    column g of the block, rows 0..3 -- exactly the B operand of a weighted
//    sum over a pair of blocks whose reduction entries 8g .. 8g + 3 are column
//    g of the first block and 8g + 4 .. 8g + 7 column g of the second:
//    O^T += V^T P^T. Its A operand (channel 16d + n of the four rows of
//    column g) comes from the same key-major slab through the LDS transpose
//    read ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a + s
//    receives element s of the 8 bytes addressed by lanes a, a + 4, a + 8 and
//    a + 12 (in that order), so lane a + 4j addresses row j at channels
//    16d + 4a .. 16d + 4a + 3.
//  * Row sums of the weights come out of the MFMA as well: one more product
//    against an all-ones A operand gives every lane the sum for its query.
//
// Windows are clamped by index arithmetic only: a score is kept when the key
// lies in the query's window (equivalently the query in the key's inverse
// window), which also rejects every point a slab holds past the grid (those
// repeat the last grid point, so they are finite). A wave with an odd number
// of blocks takes its last block alone: the second half of that reduction
// gets zero weights and repeats the first block's operand (no scores or
// exponentials for it), so every LDS byte a walk reads was staged for that
// step.
#pragma once

#include "na_common.hpp"

#include <type_traits>

namespace na {
namespace m16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Mf;

template <>
struct Mf<bf16> {
    __device__ __forceinline__ static f4 mma(uint4 a, uint4 b, f4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two fp32 values to two bf16 (round to nearest even), low half first
    __device__ __forceinline__ static uint32_t pack(float lo, float hi) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ __forceinline__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ __forceinline__ static float hi(uint32_t w) {
        return __uint_as_float(w & 0xffff0000u);
    }
    static constexpr uint32_t kOne2 = 0x3f803f80u;  // (1.0, 1.0)
};

template <>
struct Mf<f16> {
    __device__ __forceinline__ static f4 mma(uint4 a, uint4 b, f4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack(float lo, float hi) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ __forceinline__ static float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    __device__ __forceinline__ static float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    static constexpr uint32_t kOne2 = 0x3c003c00u;
};

// A workgroup of kWG waves owns a tp x (4 << prsh) x (4 << pcsh) tile of 4 x 4
// patches, tp << (prsh + pcsh) = kWG: wave v takes plane v >> (prsh + pcsh),
// patch row (v >> pcsh) mod (1 << prsh), patch column v mod (1 << pcsh). One
// plane of two rows of four patches (1 x 8 x 16) suits 2D grids; on 3D grids
// several planes per tile let every staged key plane serve each of the
// tile's query planes whose window holds it, instead of being staged once per
// query plane.
constexpr int kWG = 8, kTG = 64 * kWG;

struct Geom {
    int ext[3], ker[3], dil[3];
    int heads, batch;
    int tiles[3];  // tiles per axis over the largest residue class
    int nres, n_tiles;
    int box_w;     // points per slab row (a multiple of 4)
    int wmax;      // the kernel's compiled bound on box_w (24, 32 or 48)
    int tp, prsh, pcsh;  // tile shape: planes, log2 patch rows, log2 patch columns
    FastDiv f_heads, f_tw, f_th, f_t, f_nres;
    FastDiv f_dil[3], f_dil21;
};

template <typename T>
struct Args {
    Geom g;
    const T *q, *k, *v, *out, *dout;
    const float *lse;
    float *lse_out;  // forward: logsumexp output
    float *delta;    // dq: written; dk/dv: read
    T *o, *dq, *dk, *dv;
    float qscale;  // scale * log2(e)
    float scale;
    const int *frame;  // windows restricted along frame_axis (null: none)
    int frame_axis;
};

// Tile id -> batch, head, residue class and tile origin (class coordinates).
// The head varies fastest (the heads of one token are adjacent in memory),
// then T (the tiles of neighbouring planes share all but one of their key
// planes, which then come from L2), then W, H tiles, residue class, batch.
__device__ __forceinline__ bool decode(const Geom &g, int tile, TileCtx &w) {
    int rem = tile, q;
    q = fdiv(rem, g.f_heads);
    const int head = rem - q * g.heads;
    rem = q;
    q = fdiv(rem, g.f_t);
    const int tt = rem - q * g.tiles[0];
    rem = q;
    q = fdiv(rem, g.f_tw);
    const int tw = rem - q * g.tiles[2];
    rem = q;
    q = fdiv(rem, g.f_th);
    const int th = rem - q * g.tiles[1];
    rem = q;
    q = fdiv(rem, g.f_nres);
    const int res = rem - q * g.nres;
    const int b = q;
    int r[3];
    q = fdiv(res, g.f_dil[2]);
    r[2] = res - q * g.dil[2];
    const int q1 = fdiv(q, g.f_dil[1]);
    r[1] = q - q1 * g.dil[1];
    r[0] = fdiv(res, g.f_dil21);
    const int o[3] = {tt * g.tp, th * (4 << g.prsh), tw * (4 << g.pcsh)};
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
    // (token, head) row offsets; element offsets are these times head_dim
    const int64_t HW = (int64_t)g.ext[1] * g.ext[2];
    const int64_t ntok = HW * g.ext[0];
    const int64_t origin_tok = r[0] * HW + (int64_t)r[1] * g.ext[2] + r[2];
    w.lbase = ((int64_t)b * ntok + origin_tok) * g.heads + head;
    w.lst[0] = g.dil[0] * HW * g.heads;
    w.lst[1] = (int64_t)g.dil[1] * g.ext[2] * g.heads;
    w.lst[2] = (int64_t)g.dil[2] * g.heads;
    // every field is uniform over the workgroup: readfirstlane keeps them, and
    // the address arithmetic derived from them, in scalar registers
    auto u32 = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    auto u64 = [](int64_t v) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        w.n[a] = u32(w.n[a]);
        w.o[a] = u32(w.o[a]);
        w.r[a] = u32(w.r[a]);
        w.lst[a] = u64(w.lst[a]);
    }
    w.lbase = u64(w.lbase);
    return inside;
}

// Element offset of class point c: (row offset) * D.
template <int D>
__device__ __forceinline__ int64_t eoff(const TileCtx &w, int c0, int c1, int c2) {
    return (w.lbase + c0 * w.lst[0] + c1 * w.lst[1] + c2 * w.lst[2]) * D;
}
__device__ __forceinline__ int64_t roff(const TileCtx &w, int c0, int c1, int c2) {
    return w.lbase + c0 * w.lst[0] + c1 * w.lst[1] + c2 * w.lst[2];
}

// Key-major layout: chunk c of the point in column col and slab row r sits in
// slot ((c ^ x(col)) + r) mod NC of the point, x(col) = bit 1 of col at 8
// chunks per point (64 channels), 0 at 4; rows are a pitch apart that is 128
// (mod 256) bytes at 4 chunks per point and 16 (mod 256) at 8. Then the
// 16-byte score-operand reads of a 16-lane group (4 rows x 4 columns) and the
// 8-byte transpose reads of a 32-lane half (4 rows x 2 columns x 32 bytes)
// each touch every one of the 64 four-byte banks once (checked over all
// pitches and XOR / rotation swizzles of this form with a bank model).
template <int NC>
__device__ __forceinline__ int kslot(int c, int col, int r) {
    return ((c ^ (NC == 8 ? (col >> 1) & 1 : 0)) + r) & (NC - 1);
}
// The chunk stored in slot s (the inverse of kslot).
template <int NC>
__device__ __forceinline__ int kchunk(int s, int col, int r) {
    return ((s - r) & (NC - 1)) ^ (NC == 8 ? (col >> 1) & 1 : 0);
}

// Key-major slab: rows [r0, r0 + 4) of plane tk (class coordinates), columns
// [U2, U2 + box_w), of a tensor; row r at lds + r * Pitch, chunk s of column c
// at 16 * (c * NC + kslot(s, c, r)). Direct global-to-LDS loads, 64 consecutive
// chunks per wave instruction; the workgroup's waves take the (row, 64-chunk
// part) pieces of a slab in turn, wave v the pieces v, v + kWG, ... The lane's
// byte offset within a global row depends only on its piece, so it is
// computed once per tile; a step adds the row's (uniform) address. Points past
// the grid repeat the last grid point. Completion: stage_wait().
template <int D, int W, int Pitch>
struct Stager {
    static constexpr int NC = D * 2 / 16, PARTS = (W * NC + 63) / 64;
    static constexpr int ITEMS = (4 * PARTS + kWG - 1) / kWG;
    int goff[ITEMS];  // byte offset of the lane's chunk within its global row
    bool on[ITEMS];   // the lane has a chunk in this piece
    int n;            // pieces of this wave (uniform)
    int wave;
    __device__ __forceinline__ Stager(const TileCtx &w, int U2, int box_w, int wave_, int lane) {
        wave = wave_;
        const int nch = box_w * NC, parts = (nch + 63) >> 6;
        n = 0;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int it = wave + kWG * i;
            if (it < 4 * parts) n = i + 1;
            const int s = (it >> 2) * 64 + lane;
            const int col = s / NC, slot = s - col * NC;
            const int c2 = imin(U2 + col, w.n[2] - 1);
            goff[i] = (int)(c2 * w.lst[2]) * D * 2 + (kchunk<NC>(slot, col, it & 3) << 4);
            on[i] = s < nch;
        }
        n = __builtin_amdgcn_readfirstlane(n);
    }
    template <typename T>
    __device__ __forceinline__ void stage(const T *src, const TileCtx &w, int tk, int r0,
                                          char *lds) const {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            if (i >= n) break;
            const int it = wave + kWG * i, row = it & 3, part = it >> 2;
            const int c1 = imin(r0 + row, w.n[1] - 1);
            const char *rowp =
                reinterpret_cast<const char *>(src) + eoff<D>(w, tk, c1, 0) * (int64_t)sizeof(T);
            if (on[i]) {
#if defined(__HIP_DEVICE_COMPILE__)
                __builtin_amdgcn_global_load_lds(rowp + goff[i],
                                                 (lds_void *)(lds + row * Pitch + part * 1024), 16,
                                                 0, 0);
#else
                (void)rowp;
                (void)part;
#endif
            }
        }
    }
};

// (logsumexp, delta) of the slab point thread i stages (i < 4 box_w; column
// major: the four rows of column c at 4c .. 4c + 3). rows_load only issues the
// loads, so that they can run under a walk; rows_store writes
// (-logsumexp * log2(e), -delta) to LDS.
__device__ __forceinline__ float2 rows_load(const float *lse, const float *delta,
                                            const TileCtx &w, int tk, int r0, int U2, int box_w) {
    const int i = threadIdx.x;
    if (i >= 4 * box_w) return make_float2(0.f, 0.f);
    const int col = i >> 2, r = i & 3;
    const int64_t ro = roff(w, tk, imin(r0 + r, w.n[1] - 1), imin(U2 + col, w.n[2] - 1));
    return make_float2(lse[ro], delta[ro]);
}
__device__ __forceinline__ void rows_store(float2 v, int box_w, float2 *rows) {
    if ((int)threadIdx.x < 4 * box_w) rows[threadIdx.x] = make_float2(-v.x * kLog2e, -v.y);
}

// Maximum and sum over the four lanes n, n + 16, n + 32, n + 48 (the lane
// groups holding one query's scores): each lane swap returns the lane's own
// value and that of its partner (lane ^ 32, then lane ^ 16), VALU only.
__device__ __forceinline__ float xmax4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Origin of wave v's patch in class coordinates (uniform over the wave).
struct Patch {
    int t, h, w;
};
__device__ __forceinline__ Patch patch_origin(const Geom &g, const TileCtx &w, int wave) {
    Patch p;
    p.t = w.o[0] + (wave >> (g.prsh + g.pcsh));
    p.h = w.o[1] + 4 * ((wave >> g.pcsh) & ((1 << g.prsh) - 1));
    p.w = w.o[2] + 4 * (wave & ((1 << g.pcsh) - 1));
    return p;
}

// The lane's point of the wave's patch: patch origin + (0, n / 4, n % 4).
struct Pt {
    int t, h, w;    // clamped into the grid
    bool active;    // unclamped point inside the grid
};
__device__ __forceinline__ Pt patch_point(const Geom &g, const TileCtx &w, int wave, int n) {
    const Patch o = patch_origin(g, w, wave);
    const int h = o.h + (n >> 2), c = o.w + (n & 3);
    Pt p;
    p.active = o.t < w.n[0] && h < w.n[1] && c < w.n[2];
    p.t = __builtin_amdgcn_readfirstlane(imin(o.t, w.n[0] - 1));
    p.h = imin(h, w.n[1] - 1);
    p.w = imin(c, w.n[2] - 1);
    return p;
}

// A wave's walk: block columns [aw, aw + 4 nbw) of the slab rows (relative to
// the box start U2, aw a multiple of 4), slab rows [wr0, wr1) of its patch's
// window (or inverse-window) union; the workgroup's slabs start at row Uh.
struct Walk {
    int Uh, U2, nslab, aw, nbw, wr0, wr1;
    bool on;  // the wave's patch has a point inside the grid
};
// Planes [first, last] of the tile (clamped into the grid).
__device__ __forceinline__ int tile_last_plane(const Geom &g, const TileCtx &w) {
    return imin(w.o[0] + g.tp - 1, w.n[0] - 1);
}
template <bool Inverse>
__device__ __forceinline__ int wfirst(int x, int n, int k) {
    return Inverse ? inverse_first(x, n, k) : window_start(x, n, k);
}
template <bool Inverse>
__device__ __forceinline__ int wend(int x, int n, int k) {
    return Inverse ? inverse_last(x, n, k) + 1 : window_start(x, n, k) + k;
}
template <bool Inverse>
__device__ __forceinline__ Walk make_walk(const Geom &g, const TileCtx &w, int wave) {
    const int nh = w.n[1], nw = w.n[2], kh = w.k[1], kw = w.k[2];
    const Patch po = patch_origin(g, w, wave);
    Walk k;
    k.Uh = wfirst<Inverse>(w.o[1], nh, kh);
    const int hend = wend<Inverse>(imin(w.o[1] + (4 << g.prsh) - 1, nh - 1), nh, kh);
    k.nslab = (hend - k.Uh + 3) >> 2;
    k.U2 = wfirst<Inverse>(w.o[2], nw, kw);
    k.on = po.t < w.n[0] && po.w < nw && po.h < nh;
    const int pw0 = imin(po.w, nw - 1), pw1 = imin(pw0 + 3, nw - 1);
    k.aw = __builtin_amdgcn_readfirstlane((wfirst<Inverse>(pw0, nw, kw) - k.U2) & ~3);
    k.nbw = __builtin_amdgcn_readfirstlane((wend<Inverse>(pw1, nw, kw) - k.U2 - k.aw + 3) >> 2);
    const int ph0 = imin(po.h, nh - 1), ph1 = imin(ph0 + 3, nh - 1);
    k.wr0 = __builtin_amdgcn_readfirstlane(wfirst<Inverse>(ph0, nh, kh));
    k.wr1 = __builtin_amdgcn_readfirstlane(wend<Inverse>(ph1, nh, kh));
    return k;
}

// Per-lane LDS byte offsets within a slab (block columns added per block).
//  * km: A operand of a score product: lane n supplies point n (row n % 4,
//    column n / 4), chunk lg + 4 h;
//  * tr: transpose read of channels 16 d + 4 (n % 4) .. + 3 of row n / 4 of
//    the lane group's column (see the header).
template <int D>
struct LaneAddr {
    static constexpr int NC = D * 2 / 16, NH = D / 32, ND = D / 16;
    int km[NH];
    int tr[ND];
    __device__ __forceinline__ LaneAddr(int pitch, int lg, int n) {
        const int col = n >> 2, row = n & 3;
#pragma unroll
        for (int h = 0; h < NH; ++h)
            km[h] = row * pitch + ((col * NC + kslot<NC>(lg + 4 * h, col, row)) << 4);
        // block columns start at multiples of 4, so column lg of a block has
        // the swizzle of lg
        const int a = n & 3, j = n >> 2;
#pragma unroll
        for (int d = 0; d < ND; ++d)
            tr[d] = j * pitch + ((lg * NC + kslot<NC>(2 * d + (a >> 1), lg, j)) << 4) +
                    ((a & 1) << 3);
    }
};

__device__ __forceinline__ uint4 km_at(const char *lds, int addr) {
    return *reinterpret_cast<const uint4 *>(lds + addr);
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

__device__ __forceinline__ uint2 lds_tr(const char *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(const_cast<char *>(p)));
    return __builtin_bit_cast(uint2, v);
#else
    (void)p;
    return make_uint2(0u, 0u);
#endif
}

// A operand of a weighted sum over the blocks at blk and blk + second:
// channel 16 d + n of the lane group's column, rows 0..3 of each block. TWO
// false (a wave's odd last block, whose second half has zero weights) repeats
// the first block instead of reading a second.
template <bool TWO = true>
__device__ __forceinline__ uint4 tr_pair(const char *blk, int second, int tr) {
    const uint2 x = lds_tr(blk + tr);
    if constexpr (!TWO) return make_uint4(x.x, x.y, x.x, x.y);
    const uint2 y = lds_tr(blk + second + tr);
    return make_uint4(x.x, x.y, y.x, y.y);
}

// Weights are rescaled only when a score exceeds the running maximum by more
// than this (log2 units): weights then stay below 2^8, harmless in fp32 sums
// and in the 16-bit operands, and the rescale is rare.
constexpr float kLazyRescale = 8.f;

// Slab steps of a walk over planes [p0, p1] (those with plane_ok) times slabs
// [0, nslab), alternating between two buffers (even steps in b0, odd ones in
// b1): step s + 1 is staged into the other buffer while step s is walked, and
// one barrier per step separates the two. The buffers are distinct LDS
// arrays, each named at compile time in its half of the loop, so the compiler
// sees that the walk's LDS reads and the staging's direct loads into the other
// buffer do not alias and lets the loads run under the walk.
// stage(p, sl, buf, i) issues the loads of a step into buffer i, walk(p, sl,
// buf, i) consumes one, done(i) runs after a walk that has a next step (in
// buffer i).
template <typename OK, typename Stage, typename WalkFn, typename Done>
__device__ __forceinline__ void slab_steps(int p0, int p1, int nslab, char *b0, char *b1,
                                           OK plane_ok, Stage stage, WalkFn walk, Done done) {
    // every index here is uniform over the workgroup; readfirstlane keeps the
    // compiler from carrying them as per-lane values
    p0 = __builtin_amdgcn_readfirstlane(p0);
    p1 = __builtin_amdgcn_readfirstlane(p1);
    nslab = __builtin_amdgcn_readfirstlane(nslab);
    auto skip = [&](int q) {
        while (q <= p1 && !plane_ok(q)) ++q;
        return __builtin_amdgcn_readfirstlane(q);
    };
    int p = skip(p0);
    if (p > p1) return;
    stage(p, 0, b0, 0);
    int sl = 0;
    auto next = [&](int &pn, int &sn) {
        pn = p;
        sn = sl + 1;
        if (sn == nslab) {
            sn = 0;
            pn = skip(p + 1);
        }
        return pn <= p1;
    };
    for (;;) {
        int pn, sn;
        bool more = next(pn, sn);
        stage_wait();
        if (more) stage(pn, sn, b1, 1);
        walk(p, sl, b0, 0);
        if (!more) return;
        done(1);
        p = pn;
        sl = sn;
        more = next(pn, sn);
        stage_wait();
        if (more) stage(pn, sn, b0, 0);
        walk(p, sl, b1, 1);
        if (!more) return;
        done(0);
        p = pn;
        sl = sn;
    }
}

// Static LDS of a kernel with slab rows of up to W points: per buffer the
// slabs of two tensors.
template <int D, int W>
struct Slabs {
    static constexpr int NC = D * 2 / 16;
    // 128 (4 chunks per point) or 16 (8 chunks) bytes past a multiple of 256
    static constexpr int kRes = NC == 4 ? 128 : 16;
    static constexpr int kPitch = (W * NC * 16 - kRes + 255) / 256 * 256 + kRes;
    static constexpr int kSlab = 4 * kPitch;
    static constexpr int kBuf = 2 * kSlab;
};

// ============================================================================
// Forward: out, lse.
// Waves per SIMD (the launch bound's second value): the head_dim-32 forward
// fits 64 VGPRs, four workgroups per CU; wider slabs are bound by their LDS.
template <typename T, int D, int W>
__global__ void __launch_bounds__(kTG, D == 32 && W <= 32 ? 8 : 2) fwd_kernel(Args<T> a) {
    using S = Slabs<D, W>;
    __shared__ __align__(16) char buf0[S::kBuf];
    __shared__ __align__(16) char buf1[S::kBuf];
    constexpr int NC = D * 2 / 16, ND = D / 16, NH = D / 32, BLK = 4 * NC * 16;
    const Geom &g = a.g;
    TileCtx w;
    if (!decode(g, xcd_tile_id(blockIdx.x, g.n_tiles), w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lg = lane >> 4, n = lane & 15;
    const int nh = w.n[1], nw = w.n[2];
    constexpr int slab = S::kSlab;  // per buffer: the K slab, then the V slab

    // key planes [t0, t1] of the tile's query planes; [wt0, wt0 + k) of this wave's
    const int tl = tile_last_plane(g, w);
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    const int t1 = window_start(tl, w.n[0], w.k[0]) + w.k[0] - 1;
    const Walk wk = make_walk<false>(g, w, wave);
    const Pt P = patch_point(g, w, wave, n);
    const int wt0 = __builtin_amdgcn_readfirstlane(window_start(P.t, w.n[0], w.k[0]));
    const int wh = window_start(P.h, nh, w.k[1]);
    // column of this lane group in a block relative to the lane's window start
    const int wrel = lg - (window_start(P.w, nw, w.k[2]) - wk.U2);
    // scores are kept unscaled; a negative scale flips the query's sign instead.
    // A zero scale becomes the tiniest normal one (every weight still exp2(0)
    // in fp32), so that masked scores (-inf) times it stay -inf.
    const bool neg = a.qscale < 0.f;
    const float c = fmaxf(neg ? -a.qscale : a.qscale, 1.1754944e-38f);
    const float ic = 1.f / c;
    uint4 qv[NH];
    {
        const T *qp = a.q + eoff<D>(w, P.t, P.h, P.w) + 8 * lg;
        const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            qv[h] = *reinterpret_cast<const uint4 *>(qp + 32 * h);
            qv[h].x ^= flip; qv[h].y ^= flip; qv[h].z ^= flip; qv[h].w ^= flip;
        }
    }
    const LaneAddr<D> la(S::kPitch, lg, n);
    const uint4 ones = make_uint4(Mf<T>::kOne2, Mf<T>::kOne2, Mf<T>::kOne2, Mf<T>::kOne2);
    const f4 zero = f4{0.f, 0.f, 0.f, 0.f};

    f4 acc[ND], lsum = zero;
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = zero;
    float m = -1e30f;            // running maximum, scaled (log2 units)
    float thr = (m + kLazyRescale) * ic;  // unscaled score that triggers a rescale

    // frames: along T (3D grids) key planes outside a query plane's frame window
    // are skipped (by the workgroup when no query plane of the tile keeps them);
    // along H (2D grids) slab rows outside the lane's query row's are masked
    const bool fr_t = a.frame && a.frame_axis == 0, fr_h = a.frame && a.frame_axis == 1;
    // (the frame size of the wave's plane is uniform: readfirstlane keeps the
    // plane tests scalar)
    const int fk_t = fr_t ? __builtin_amdgcn_readfirstlane(frame_size(a.frame, w, 0, P.t)) : 0;
    const int fs_t = __builtin_amdgcn_readfirstlane(window_start(P.t, w.n[0], imax(fk_t, 1)));
    const int fk_h = fr_h ? frame_size(a.frame, w, 1, P.h) : 0;
    // key rows [hlo, hlo + hlen) of the lane's query: its window rows, cut to
    // its frame window on 2D grids with frames
    int hlo = wh, hlen = w.k[1];
    if (fr_h) {
        const int fs = window_start(P.h, nh, imax(fk_h, 1));
        const int hi = imin(wh + w.k[1], fs + fk_h);
        hlo = imax(wh, fs);
        hlen = imax(hi - hlo, 0);
    }
    // key plane tk in the window (and the frame window) of the wave's query plane
    auto wave_plane = [&](int tk) {
        return (unsigned)(tk - wt0) < (unsigned)w.k[0] &&
               (!fr_t || (unsigned)(tk - fs_t) < (unsigned)fk_t);
    };
    // key plane tk kept by some query plane of the tile
    auto plane_ok = [&](int tk) {
        if (!fr_t) return true;
        for (int z = w.o[0]; z <= tl; ++z)
            if ((unsigned)(tk - window_start(z, w.n[0], w.k[0])) < (unsigned)w.k[0] &&
                in_frame(tk, z, w.n[0], frame_size(a.frame, w, 0, z)))
                return true;
        return false;
    };
    const Stager<D, W, S::kPitch> st(w, wk.U2, g.box_w, wave, lane);
    auto stage = [&](int tk, int sl, char *buf, int) {
        st.stage(a.k, w, tk, wk.Uh + 4 * sl, buf);
        st.stage(a.v, w, tk, wk.Uh + 4 * sl, buf + slab);
    };
    auto walk = [&](int tk, int sl, const char *buf, int) {
        const int r0 = wk.Uh + 4 * sl;
        if (!wk.on || !wave_plane(tk) || r0 + 4 <= wk.wr0 || r0 >= wk.wr1) return;
        const char *Kc = buf, *Vc = buf + slab;
        // key rows of the slab inside the lane's query window
        bool hr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hr[r] = (unsigned)(r0 + r - hlo) < (unsigned)hlen;
        // a pair of blocks, or (TWO false) a wave's odd last block alone: its
        // second half of the reduction then has zero weights, so its scores
        // and exponentials are skipped and its V operand repeats the first
        // block (finite values times zero weights)
        auto step = [&](int col0, int second, bool two, auto two_c) {
            constexpr bool TWO = decltype(two_c)::value;
            const char *kb = Kc + col0 * NC * 16;
            f4 s0 = Mf<T>::mma(km_at(kb, la.km[0]), qv[0], zero), s1 = zero;
            if constexpr (TWO) s1 = Mf<T>::mma(km_at(kb + second, la.km[0]), qv[0], zero);
#pragma unroll
            for (int h = 1; h < NH; ++h) {
                s0 = Mf<T>::mma(km_at(kb, la.km[h]), qv[h], s0);
                if constexpr (TWO) s1 = Mf<T>::mma(km_at(kb + second, la.km[h]), qv[h], s1);
            }
            const bool w0 = (unsigned)(col0 + wrel) < (unsigned)w.k[2];
            const bool w1 = TWO && two && (unsigned)(col0 + 4 + wrel) < (unsigned)w.k[2];
            float x[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = (w0 && hr[r]) ? s0[r] : -INFINITY;
                x[4 + r] = (w1 && hr[r]) ? s1[r] : -INFINITY;
            }
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            if constexpr (TWO) mx = fmaxf(mx, fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            mx = xmax4(mx);
            if (__any(mx > thr)) {
                const float mn = mx > thr ? mx * c : m;
                const float alpha = fast_exp2(m - mn);
                m = mn;
                thr = (m + kLazyRescale) * ic;
#pragma unroll
                for (int d = 0; d < ND; ++d) acc[d] *= alpha;
                lsum *= alpha;
            }
            uint4 pb;
            pb.x = Mf<T>::pack(fast_exp2(fmaf(x[0], c, -m)), fast_exp2(fmaf(x[1], c, -m)));
            pb.y = Mf<T>::pack(fast_exp2(fmaf(x[2], c, -m)), fast_exp2(fmaf(x[3], c, -m)));
            if constexpr (TWO) {
                pb.z = Mf<T>::pack(fast_exp2(fmaf(x[4], c, -m)), fast_exp2(fmaf(x[5], c, -m)));
                pb.w = Mf<T>::pack(fast_exp2(fmaf(x[6], c, -m)), fast_exp2(fmaf(x[7], c, -m)));
            } else {
                pb.z = pb.w = 0u;
            }
            const char *vb = Vc + col0 * NC * 16;
#pragma unroll
            for (int d = 0; d < ND; ++d)
                acc[d] = Mf<T>::mma(tr_pair<TWO>(vb, second, la.tr[d]), pb, acc[d]);
            lsum = Mf<T>::mma(ones, pb, lsum);
        };
        int b = 0;
        for (; b + 1 < wk.nbw; b += 2) step(wk.aw + 4 * b, BLK, true, std::true_type{});
        if (b < wk.nbw) step(wk.aw + 4 * b, 0, false, std::false_type{});
    };
    slab_steps(t0, t1, wk.nslab, buf0, buf1, plane_ok, stage, walk, [](int) {});

    if (!wk.on || !P.active) return;
    // a query whose window is masked away entirely: zero output, lse -inf
    const float inv = lsum[0] > 0.f ? 1.f / lsum[0] : 0.f;
    T *op = a.o + eoff<D>(w, P.t, P.h, P.w) + 4 * lg;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        const float o4[4] = {acc[d][0] * inv, acc[d][1] * inv, acc[d][2] * inv, acc[d][3] * inv};
        Io<T>::store4(op + 16 * d, o4);
    }
    if (lg == 0)
        a.lse_out[roff(w, P.t, P.h, P.w)] =
            lsum[0] > 0.f ? (m + __log2f(lsum[0])) * kLn2 : -INFINITY;
}

// ============================================================================
// Backward, query side: delta = <dout, out> and dq.
template <typename T, int D, int W>
__global__ void __launch_bounds__(kTG, D == 32 && W <= 32 ? 8 : 2) dq_kernel(Args<T> a) {
    using S = Slabs<D, W>;
    __shared__ __align__(16) char buf0[S::kBuf];
    __shared__ __align__(16) char buf1[S::kBuf];
    constexpr int NC = D * 2 / 16, ND = D / 16, NH = D / 32, BLK = 4 * NC * 16;
    const Geom &g = a.g;
    TileCtx w;
    if (!decode(g, xcd_tile_id(blockIdx.x, g.n_tiles), w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lg = lane >> 4, n = lane & 15;
    const int nh = w.n[1], nw = w.n[2];
    constexpr int slab = S::kSlab;  // per buffer: the V slab, then the K slab
    // the odd last block alone (below) where its extra code still fits the
    // register budget of the launch bound
    constexpr bool kSplitOdd = true;

    // key planes [t0, t1] of the tile's query planes; [wt0, wt0 + k) of this wave's
    const int tl = tile_last_plane(g, w);
    const int t0 = window_start(w.o[0], w.n[0], w.k[0]);
    const int t1 = window_start(tl, w.n[0], w.k[0]) + w.k[0] - 1;
    const Walk wk = make_walk<false>(g, w, wave);
    const Pt P = patch_point(g, w, wave, n);
    const int wt0 = __builtin_amdgcn_readfirstlane(window_start(P.t, w.n[0], w.k[0]));
    const int wh = window_start(P.h, nh, w.k[1]);
    const int wrel = lg - (window_start(P.w, nw, w.k[2]) - wk.U2);
    const int64_t qo = eoff<D>(w, P.t, P.h, P.w);
    const int64_t ro = roff(w, P.t, P.h, P.w);
    uint4 qv[NH], dv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        qv[h] = *reinterpret_cast<const uint4 *>(a.q + qo + 8 * lg + 32 * h);
        dv[h] = *reinterpret_cast<const uint4 *>(a.dout + qo + 8 * lg + 32 * h);
    }
    // delta of the lane's query: its lane group's 8 (or 16) channels, summed
    // over the four lane groups
    float delta = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const uint4 ov = *reinterpret_cast<const uint4 *>(a.out + qo + 8 * lg + 32 * h);
        const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, dw[4] = {dv[h].x, dv[h].y, dv[h].z, dv[h].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            delta += Mf<T>::lo(ow[i]) * Mf<T>::lo(dw[i]) + Mf<T>::hi(ow[i]) * Mf<T>::hi(dw[i]);
    }
    delta = xsum4(delta);
    if (wk.on && P.active && lg == 0) a.delta[ro] = delta;
    const float nlse2 = -a.lse[ro] * kLog2e;
    const float c = a.qscale;
    const f4 ndelta = f4{-delta, -delta, -delta, -delta};
    const LaneAddr<D> la(S::kPitch, lg, n);
    const f4 zero = f4{0.f, 0.f, 0.f, 0.f};

    f4 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = zero;

    // frames: along T (3D grids) key planes outside a query plane's frame window
    // are skipped (by the workgroup when no query plane of the tile keeps them);
    // along H (2D grids) slab rows outside the lane's query row's are masked
    const bool fr_t = a.frame && a.frame_axis == 0, fr_h = a.frame && a.frame_axis == 1;
    // (the frame size of the wave's plane is uniform: readfirstlane keeps the
    // plane tests scalar)
    const int fk_t = fr_t ? __builtin_amdgcn_readfirstlane(frame_size(a.frame, w, 0, P.t)) : 0;
    const int fs_t = __builtin_amdgcn_readfirstlane(window_start(P.t, w.n[0], imax(fk_t, 1)));
    const int fk_h = fr_h ? frame_size(a.frame, w, 1, P.h) : 0;
    // key rows [hlo, hlo + hlen) of the lane's query: its window rows, cut to
    // its frame window on 2D grids with frames
    int hlo = wh, hlen = w.k[1];
    if (fr_h) {
        const int fs = window_start(P.h, nh, imax(fk_h, 1));
        const int hi = imin(wh + w.k[1], fs + fk_h);
        hlo = imax(wh, fs);
        hlen = imax(hi - hlo, 0);
    }
    // key plane tk in the window (and the frame window) of the wave's query plane
    auto wave_plane = [&](int tk) {
        return (unsigned)(tk - wt0) < (unsigned)w.k[0] &&
               (!fr_t || (unsigned)(tk - fs_t) < (unsigned)fk_t);
    };
    // key plane tk kept by some query plane of the tile
    auto plane_ok = [&](int tk) {
        if (!fr_t) return true;
        for (int z = w.o[0]; z <= tl; ++z)
            if ((unsigned)(tk - window_start(z, w.n[0], w.k[0])) < (unsigned)w.k[0] &&
                in_frame(tk, z, w.n[0], frame_size(a.frame, w, 0, z)))
                return true;
        return false;
    };
    const Stager<D, W, S::kPitch> st(w, wk.U2, g.box_w, wave, lane);
    auto stage = [&](int tk, int sl, char *buf, int) {
        st.stage(a.v, w, tk, wk.Uh + 4 * sl, buf);
        st.stage(a.k, w, tk, wk.Uh + 4 * sl, buf + slab);
    };
    auto walk = [&](int tk, int sl, const char *buf, int) {
        const int r0 = wk.Uh + 4 * sl;
        if (!wk.on || !wave_plane(tk) || r0 + 4 <= wk.wr0 || r0 >= wk.wr1) return;
        const char *Vc = buf, *Kc = buf + slab;
        bool hr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hr[r] = (unsigned)(r0 + r - hlo) < (unsigned)hlen;
        // a pair of blocks, or (TWO false) a wave's odd last block alone (its
        // second half of the reduction gets zero score gradients)
        auto step = [&](int col0, int second, bool two, auto two_c) {
            constexpr bool TWO = decltype(two_c)::value;
            const char *kb = Kc + col0 * NC * 16, *vb = Vc + col0 * NC * 16;
            // dP - delta: the products start from -delta
            f4 s0 = Mf<T>::mma(km_at(kb, la.km[0]), qv[0], zero);
            f4 p0 = Mf<T>::mma(km_at(vb, la.km[0]), dv[0], ndelta);
            f4 s1 = zero, p1 = zero;
            if constexpr (TWO) {
                s1 = Mf<T>::mma(km_at(kb + second, la.km[0]), qv[0], zero);
                p1 = Mf<T>::mma(km_at(vb + second, la.km[0]), dv[0], ndelta);
            }
#pragma unroll
            for (int h = 1; h < NH; ++h) {
                s0 = Mf<T>::mma(km_at(kb, la.km[h]), qv[h], s0);
                p0 = Mf<T>::mma(km_at(vb, la.km[h]), dv[h], p0);
                if constexpr (TWO) {
                    s1 = Mf<T>::mma(km_at(kb + second, la.km[h]), qv[h], s1);
                    p1 = Mf<T>::mma(km_at(vb + second, la.km[h]), dv[h], p1);
                }
            }
            const bool w0 = (unsigned)(col0 + wrel) < (unsigned)w.k[2];
            const bool w1 = TWO && two && (unsigned)(col0 + 4 + wrel) < (unsigned)w.k[2];
            float ds[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e0 = fast_exp2((w0 && hr[r]) ? fmaf(s0[r], c, nlse2) : -INFINITY);
                ds[r] = e0 * p0[r];
                if constexpr (TWO) {
                    const float e1 = fast_exp2((w1 && hr[r]) ? fmaf(s1[r], c, nlse2) : -INFINITY);
                    ds[4 + r] = e1 * p1[r];
                }
            }
            uint4 db;
            db.x = Mf<T>::pack(ds[0], ds[1]);
            db.y = Mf<T>::pack(ds[2], ds[3]);
            if constexpr (TWO) {
                db.z = Mf<T>::pack(ds[4], ds[5]);
                db.w = Mf<T>::pack(ds[6], ds[7]);
            } else {
                db.z = db.w = 0u;
            }
#pragma unroll
            for (int d = 0; d < ND; ++d)
                acc[d] = Mf<T>::mma(tr_pair<TWO>(kb, second, la.tr[d]), db, acc[d]);
        };
        if constexpr (kSplitOdd) {
            int b = 0;
            for (; b + 1 < wk.nbw; b += 2) step(wk.aw + 4 * b, BLK, true, std::true_type{});
            if (b < wk.nbw) step(wk.aw + 4 * b, 0, false, std::false_type{});
        } else {
            // the odd last block pairs with itself; the copy's weights are masked
            for (int b = 0; b < wk.nbw; b += 2) {
                const bool two = b + 1 < wk.nbw;
                step(wk.aw + 4 * b, two ? BLK : 0, two, std::true_type{});
            }
        }
    };
    slab_steps(t0, t1, wk.nslab, buf0, buf1, plane_ok, stage, walk, [](int) {});

    if (!wk.on || !P.active) return;
    T *dp = a.dq + qo + 4 * lg;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        const float o4[4] = {acc[d][0] * a.scale, acc[d][1] * a.scale, acc[d][2] * a.scale,
                             acc[d][3] * a.scale};
        Io<T>::store4(dp + 16 * d, o4);
    }
}

// ============================================================================
// Backward, key side: dk and dv by inverse-neighborhood gather (no atomics).
// The wave's patch holds keys; it walks the 4 x 4 query blocks of its keys'
// inverse windows: S = Q K^T (A = a query block, key-major; B = the wave's
// keys), P = exp2(S c - lse), dP = dO V^T, dS = P (dP - delta); then
// dV^T += dO^T P and dK^T += Q^T dS over pairs of query blocks.
// Four waves per SIMD up to 32-point slab rows: 128 VGPRs, two workgroups per
// CU also at head_dim 64; wider slabs are bound by their LDS.
template <typename T, int D, int W>
__global__ void __launch_bounds__(kTG, W <= 32 ? 4 : 2) dkdv_kernel(Args<T> a) {
    using S = Slabs<D, W>;
    __shared__ __align__(16) char buf0[S::kBuf];
    __shared__ __align__(16) char buf1[S::kBuf];
    constexpr int NC = D * 2 / 16, ND = D / 16, NH = D / 32, BLK = 4 * NC * 16;
    const Geom &g = a.g;
    TileCtx w;
    if (!decode(g, xcd_tile_id(blockIdx.x, g.n_tiles), w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lg = lane >> 4, n = lane & 15;
    const int nh = w.n[1], nw = w.n[2];
    constexpr int slab = S::kSlab;  // per buffer: the Q slab, then the dout slab
    // the odd last block alone (below) where its extra code still fits the
    // register budget of the launch bound
    constexpr bool kSplitOdd = D == 32;
    // (logsumexp * log2(e), delta) of the slab's points, one array per buffer
    __shared__ float2 rows0[4 * W], rows1[4 * W];

    // the workgroup's query planes [tq0, tq1], those of this wave's key plane
    // [iq0, iq1], and this wave's walk of the inverse windows
    const int tl = tile_last_plane(g, w);
    const int tq0 = inverse_first(w.o[0], w.n[0], w.k[0]);
    const int tq1 = inverse_last(tl, w.n[0], w.k[0]);
    const Walk wk = make_walk<true>(g, w, wave);
    const Pt P = patch_point(g, w, wave, n);  // the lane's key
    const int iq0 = __builtin_amdgcn_readfirstlane(inverse_first(P.t, w.n[0], w.k[0]));
    const int iq1 = __builtin_amdgcn_readfirstlane(inverse_last(P.t, w.n[0], w.k[0]));
    const int ih0 = inverse_first(P.h, nh, w.k[1]), ih1 = inverse_last(P.h, nh, w.k[1]);
    // query columns of this lane group relative to the key's inverse window
    const int irel = lg - (inverse_first(P.w, nw, w.k[2]) - wk.U2);
    const int iwn = inverse_last(P.w, nw, w.k[2]) - inverse_first(P.w, nw, w.k[2]);
    const int64_t ko = eoff<D>(w, P.t, P.h, P.w);
    uint4 kv[NH], vv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        kv[h] = *reinterpret_cast<const uint4 *>(a.k + ko + 8 * lg + 32 * h);
        vv[h] = *reinterpret_cast<const uint4 *>(a.v + ko + 8 * lg + 32 * h);
    }
    const float c = a.qscale;
    const LaneAddr<D> la(S::kPitch, lg, n);
    const f4 zero = f4{0.f, 0.f, 0.f, 0.f};

    f4 dka[ND], dva[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        dka[d] = zero;
        dva[d] = zero;
    }

    // frames: along T (3D grids) query planes whose frame window misses the key
    // plane are skipped (by the workgroup when it misses every key plane of the
    // tile); along H (2D grids) such query rows are masked
    const bool fr_t = a.frame && a.frame_axis == 0, fr_h = a.frame && a.frame_axis == 1;
    // query plane tq in the inverse window (and frame) of the wave's key plane
    auto wave_plane = [&](int tq) {
        return (unsigned)(tq - iq0) <= (unsigned)(iq1 - iq0) &&
               (!fr_t || in_frame(P.t, tq, w.n[0],
                                  __builtin_amdgcn_readfirstlane(frame_size(a.frame, w, 0, tq))));
    };
    // query plane tq whose frame window holds some key plane of the tile
    auto plane_ok = [&](int tq) {
        if (!fr_t) return true;
        const int fk = __builtin_amdgcn_readfirstlane(frame_size(a.frame, w, 0, tq));
        for (int z = w.o[0]; z <= tl; ++z)
            if (in_frame(z, tq, w.n[0], fk)) return true;
        return false;
    };
    float2 rv = make_float2(0.f, 0.f);  // the next slab's rows, in flight
    bool first = true;                  // the first step's rows are stored at once
    const Stager<D, W, S::kPitch> st(w, wk.U2, g.box_w, wave, lane);
    auto stage = [&](int tq, int sl, char *buf, int i) {
        const int r0 = wk.Uh + 4 * sl;
        st.stage(a.q, w, tq, r0, buf);
        st.stage(a.dout, w, tq, r0, buf + slab);
        rv = rows_load(a.lse, a.delta, w, tq, r0, wk.U2, g.box_w);
        if (first) rows_store(rv, g.box_w, i ? rows1 : rows0);
        first = false;
    };
    // a later step's rows go to LDS after the walk before it (their array was
    // last read a step earlier)
    auto done = [&](int i) { rows_store(rv, g.box_w, i ? rows1 : rows0); };
    auto walk = [&](int tq, int sl, const char *buf, int i) {
        const int r0 = wk.Uh + 4 * sl;
        if (!wk.on || !wave_plane(tq) || r0 + 4 <= wk.wr0 || r0 >= wk.wr1) return;
        const char *Qc = buf, *Oc = buf + slab;
        const float2 *Rc = i ? rows1 : rows0;
        // query rows of the slab inside the key's inverse window
        bool hr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hr[r] = (unsigned)(r0 + r - ih0) <= (unsigned)(ih1 - ih0);
        if (fr_h) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                hr[r] = hr[r] & in_frame(P.h, r0 + r, nh,
                                         frame_size(a.frame, w, 1, imin(r0 + r, nh - 1)));
        }
        // a pair of query blocks, or (TWO false) a wave's odd last block alone
        // (its second half of the reductions gets zero weights and zero score
        // gradients)
        auto step = [&](int col0, int second, bool two, auto two_c) {
            constexpr bool TWO = decltype(two_c)::value;
            const char *qb = Qc + col0 * NC * 16, *ob = Oc + col0 * NC * 16;
            f4 s0 = Mf<T>::mma(km_at(qb, la.km[0]), kv[0], zero);
            f4 p0 = Mf<T>::mma(km_at(ob, la.km[0]), vv[0], zero);
            f4 s1 = zero, p1 = zero;
            if constexpr (TWO) {
                s1 = Mf<T>::mma(km_at(qb + second, la.km[0]), kv[0], zero);
                p1 = Mf<T>::mma(km_at(ob + second, la.km[0]), vv[0], zero);
            }
#pragma unroll
            for (int h = 1; h < NH; ++h) {
                s0 = Mf<T>::mma(km_at(qb, la.km[h]), kv[h], s0);
                p0 = Mf<T>::mma(km_at(ob, la.km[h]), vv[h], p0);
                if constexpr (TWO) {
                    s1 = Mf<T>::mma(km_at(qb + second, la.km[h]), kv[h], s1);
                    p1 = Mf<T>::mma(km_at(ob + second, la.km[h]), vv[h], p1);
                }
            }
            // (-lse * log2 e, -delta) of the four rows of this lane group's query column
            const float4 *rp0 = reinterpret_cast<const float4 *>(Rc + 4 * (col0 + lg));
            const float4 l0a = rp0[0], l0b = rp0[1];
            float4 l1a = l0a, l1b = l0b;
            if constexpr (TWO) {
                const float4 *rp1 =
                    reinterpret_cast<const float4 *>(Rc + 4 * (two ? col0 + 4 + lg : col0 + lg));
                l1a = rp1[0];
                l1b = rp1[1];
            }
            const float ls0[4] = {l0a.x, l0a.z, l0b.x, l0b.z}, nd0[4] = {l0a.y, l0a.w, l0b.y, l0b.w};
            const float ls1[4] = {l1a.x, l1a.z, l1b.x, l1b.z}, nd1[4] = {l1a.y, l1a.w, l1b.y, l1b.w};
            const bool w0 = (unsigned)(col0 + irel) <= (unsigned)iwn;
            const bool w1 = TWO && two && (unsigned)(col0 + 4 + irel) <= (unsigned)iwn;
            float pr[8], ds[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[r] = fast_exp2((w0 && hr[r]) ? fmaf(s0[r], c, ls0[r]) : -INFINITY);
                if constexpr (TWO)
                    pr[4 + r] = fast_exp2((w1 && hr[r]) ? fmaf(s1[r], c, ls1[r]) : -INFINITY);
                ds[r] = pr[r] * (p0[r] + nd0[r]);
                if constexpr (TWO) ds[4 + r] = pr[4 + r] * (p1[r] + nd1[r]);
            }
            uint4 pb, db;
            pb.x = Mf<T>::pack(pr[0], pr[1]);
            pb.y = Mf<T>::pack(pr[2], pr[3]);
            db.x = Mf<T>::pack(ds[0], ds[1]);
            db.y = Mf<T>::pack(ds[2], ds[3]);
            if constexpr (TWO) {
                pb.z = Mf<T>::pack(pr[4], pr[5]);
                pb.w = Mf<T>::pack(pr[6], pr[7]);
                db.z = Mf<T>::pack(ds[4], ds[5]);
                db.w = Mf<T>::pack(ds[6], ds[7]);
            } else {
                pb.z = pb.w = db.z = db.w = 0u;
            }
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                dva[d] = Mf<T>::mma(tr_pair<TWO>(ob, second, la.tr[d]), pb, dva[d]);
                dka[d] = Mf<T>::mma(tr_pair<TWO>(qb, second, la.tr[d]), db, dka[d]);
            }
        };
        if constexpr (kSplitOdd) {
            int b = 0;
            for (; b + 1 < wk.nbw; b += 2) step(wk.aw + 4 * b, BLK, true, std::true_type{});
            if (b < wk.nbw) step(wk.aw + 4 * b, 0, false, std::false_type{});
        } else {
            // the odd last block pairs with itself; the copy's weights are masked
            for (int b = 0; b < wk.nbw; b += 2) {
                const bool two = b + 1 < wk.nbw;
                step(wk.aw + 4 * b, two ? BLK : 0, two, std::true_type{});
            }
        }
    };
    slab_steps(tq0, tq1, wk.nslab, buf0, buf1, plane_ok, stage, walk, done);

    if (!wk.on || !P.active) return;
    T *kp = a.dk + ko + 4 * lg;
    T *vp = a.dv + ko + 4 * lg;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        const float k4[4] = {dka[d][0] * a.scale, dka[d][1] * a.scale, dka[d][2] * a.scale,
                             dka[d][3] * a.scale};
        const float v4[4] = {dva[d][0], dva[d][1], dva[d][2], dva[d][3]};
        Io<T>::store4(kp + 16 * d, k4);
        Io<T>::store4(vp + 16 * d, v4);
    }
}

// Launch of kernel `kind` (0 forward, 1 dq, 2 dk/dv) for slab rows of up to
// a.g.wmax points (24, 32 or 48) on stream s; defined in na_m16.hip for bf16 /
// f16 and D 32 / 64.
template <typename T, int D>
hipError_t launch(int kind, const Args<T> &a, hipStream_t s);

}  // namespace m16
}  // namespace na
