// na_kernels.hpp -- neighborhood attention forward and backward kernels for
// gfx950 (wave64, fp32 MFMA 4x4x1, LDS-staged operands).
//
// Work decomposition. A workgroup of four waves owns a 1x8x8 tile of one
// residue class of one (batch, head): 64 points, one per lane, in sixteen 1x2x2
// patches (one per 4-lane MFMA block). In the forward and dq kernels the points
// are queries, in the dk/dv kernel keys. The workgroup stages, once, the box of
// the other side's points its tile needs (the union of the windows, or of the
// inverse windows) in LDS, then each block walks the 1x2x2 patches covering
// what its own four points need; the four waves split those patches between
// them and merge their partial results through LDS at the end.
//
// Why these shapes. A 4x4 MFMA block contracts 4 points against 4 points, so a
// 1x2x2 patch wastes little of a window: a 9x9 window is covered by 5x5 patches
// (100 computed vs 81 needed scores), a 3x5x5 window by 3x3x3 (108 vs 75); a
// 16-point tile (16x16 MFMA) would compute 144 resp. 192. The price is operand
// traffic: every 4x4x1 MFMA needs one fresh register per lane, so operands come
// from LDS (fast enough on gfx950), not from L1. Scores outside a point's
// window are masked by index arithmetic on the window starts, never by padding
// (software predication of these bounds is what the NATTEN maintainer names as
// the main overhead of 2D/3D fused kernels; here it is a few integer compares).
//
// Softmax. Scores are kept in log2 units (q pre-multiplied by scale*log2(e)) so
// exp2 is one instruction; each lane keeps the running maximum and sum of its
// own query, so no cross-lane reduction is needed in the softmax.
//
// Backward (the gather variant): the dq kernel recomputes P = exp2(S - lse)
// from the saved logsumexp, forms delta = <dout, out> for its queries
// (NATTEN's ComputeDelta, fused here), dS = P (dP - delta) and dq. The dk/dv
// kernel walks every key's inverse neighborhood (one contiguous range per
// axis, closed form in na_index.hpp) and writes dk, dv exactly once, with no
// atomics. With KVPAR the dk/dv pass also forms each query's dq contribution
// and adds it into an fp32 accumulator (the KV-parallel variant).
#pragma once

#include "na_common.hpp"

namespace na {

struct FwdArgs {
    Geometry g;
    const void *q, *k, *v;
    void *out;
    float *lse;
    float qscale;  // scale * log2(e)
    const int *frame;  // windows restricted along frame_axis (null: none)
    int frame_axis;
    const uint8_t *mask;  // window mask, K = mask_k bytes per query token (null: none)
    int mask_k;
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
    const int *frame;  // windows restricted along frame_axis (null: none)
    int frame_axis;
    const uint8_t *mask;  // window mask, K = mask_k bytes per query token (null: none)
    int mask_k;
    // dk/dv: when skip_ch > 0, skip the tiles whose 16 x 16 super-tile has an
    // inverse walk of at most skip_ch x skip_cw patches (the register-resident
    // dk/dv kernel covers those)
    int skip_ch, skip_cw;
    // KV-parallel with bounded copies: this launch runs the tiles of classes
    // [cls_lo, cls_lo + cls_n); a tile's class is its tile index along each
    // axis modulo cls_m (tiles of one class have disjoint query boxes), and
    // it adds its box into copy (class - cls_lo), copy_stride floats apart
    int cls_lo, cls_n, cls_m[3];
    int64_t copy_stride;
};

// dq contributions of a KV-parallel workgroup are summed exactly in LDS as
// 64-bit fixed point with 32 fraction bits: integer additions do not depend on
// their order, so the sums are the same on every run (|partial sums| < 2^31).
constexpr float kFixOne = 4294967296.0f;  // 2^32
constexpr float kFixInv = 1.0f / 4294967296.0f;

// Workgroups per CU the split kernels are compiled for: at head_dim 64 the
// per-lane rows and accumulators need more than the 256 registers of two
// workgroups per CU, so one workgroup takes the CU's whole register file and
// LDS (no scratch spills, boxes staged in one chunk).
template <int D>
constexpr int kSplitOccupancy = D >= 64 ? 1 : 2;

// Element `i` of a 3-array chosen by value: a runtime index into a small
// array would put the array in (slow, memory-backed) scratch.
__device__ __forceinline__ int get3(const int (&a)[3], int i) {
    return i == 0 ? a[0] : (i == 1 ? a[1] : a[2]);
}

// Rows of axis A a chunk of the staged box may hold: as many as the LDS budget
// allows for bytes_per_point, at least one.
__device__ __forceinline__ int chunk_rows(const Box &b, int A, int bytes_per_point, int budget) {
    const int ea = get3(b.e, A);
    const int plane = b.e[0] * b.e[1] * b.e[2] / ea;
    return imax(1, imin(ea, budget / (plane * bytes_per_point)));
}

// The chunk of box b starting at row r0 of axis A.
__device__ __forceinline__ Box chunk_of(const Box &b, int A, int r0, int rows) {
    Box c = b;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        if (x == A) {
            c.o[x] = b.o[x] + r0;
            c.e[x] = imin(rows, b.e[x] - r0);
        }
    }
    return c;
}

// A lane's addressing of a patch walk over a staged chunk. The walk starts at
// class point `start` (the first patch of the lane's block); entry e (0..3) of
// item (c0, c1, c2) is the point start + (c0, 2 c1 + e/2, 2 c2 + e%2). For a
// fixed entry, the LDS point index moves by an amount that is the same for all
// lanes (item_offset), and its swizzle only depends on c2 mod 4, so both are
// prepared per entry once per chunk.
struct Entry {
    int ptb;    // LDS byte offset of the entry's point at item (0, 0, 0)
    int tab;    // swizzle at c2 = j (mod 4) in bits [4j, 4j + 4)
};

template <int NC>
__device__ __forceinline__ Entry make_entry(const Box &b, const int (&start)[3], int e) {
    constexpr int PB = NC * 16;
    const int l0 = start[0] - b.o[0], l1 = start[1] - b.o[1] + (e >> 1);
    const int l2 = start[2] - b.o[2] + (e & 1);
    Entry en;
    en.ptb = ((l0 * b.e[1] + l1) * b.e[2] + l2) * PB;
    en.tab = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) en.tab |= swz<NC>(l1, l2 + 2 * j) << (4 * j);
    // keep the prepared values in registers (no re-derivation inside the walk)
    asm volatile("" : "+v"(en.ptb), "+v"(en.tab));
    return en;
}

// Item i of a walk of cnt patches per axis (row-major); all fields are the
// same for every lane.
struct Item {
    int c0, c1, c2;
    int offb;       // LDS byte offset of the item relative to item (0, 0, 0)
    int sh;         // 4 * (c2 mod 4): swizzle table shift
};

template <int PB>
__device__ __forceinline__ Item make_item(int i, const int (&cnt)[3], const Box &b) {
    Item it;
    it.c2 = i % cnt[2];
    it.c1 = (i / cnt[2]) % cnt[1];
    it.c0 = i / (cnt[2] * cnt[1]);
    it.offb = ((it.c0 * b.e[1] + 2 * it.c1) * b.e[2] + 2 * it.c2) * PB;
    it.sh = 4 * (it.c2 & 3);
    return it;
}

__device__ __forceinline__ unsigned umin(unsigned a, unsigned b) { return a < b ? a : b; }

// LDS byte address of chunk 0 of the entry's point at this item, with the
// swizzle folded in: chunk s is at  addr ^ (s << 4). limb (a byte offset)
// clamps the point into the staged chunk (walks over a chunk cut along H,
// masked entries; negative offsets wrap to large unsigned values).
__device__ __forceinline__ int entry_addr(const Entry &en, const Item &it, unsigned limb) {
    const unsigned pa = umin((unsigned)(en.ptb + it.offb), limb);
    return (int)pa | (((en.tab >> it.sh) & 15) << 4);
}

// Full point (D elements) at LDS byte address addr (see entry_addr).
template <typename T, int D>
__device__ __forceinline__ void lds_point_at(const char *lds, int addr, float (&d)[D]) {
    constexpr int PB = D * (int)sizeof(T), NC = PB / 16, EPC = 16 / (int)sizeof(T);
#pragma unroll
    for (int s = 0; s < NC; ++s) Io<T>::chunk(lds + (addr ^ (s << 4)), d + s * EPC);
}

// Elements [c*G, c*G + G) (G = D / 4) of the point at LDS byte address addr.
template <typename T, int D>
__device__ __forceinline__ void lds_quarter_at(const char *lds, int addr, int c, float (&d)[D / 4]) {
    constexpr int EPC = 16 / (int)sizeof(T), G = D / 4;
    if constexpr (G >= EPC) {
#pragma unroll
        for (int s = 0; s < G / EPC; ++s)
            Io<T>::chunk(lds + (addr ^ ((c * (G / EPC) + s) << 4)), d + s * EPC);
    } else {
        // G = 4 < EPC = 8 (bf16, D = 16): half a chunk
        const int chunk = (c * G) / EPC, half = (c * G) % EPC;
        Io<T>::quad(lds + (addr ^ (chunk << 4)) + half * (int)sizeof(T), d);
    }
}

// Validity bits of the four entries of an item: bit e set when entry e lies in
// the lane's window (or inverse window). m[a] has bit r set when relative
// position r along axis a (from the walk start) is valid.
__device__ __forceinline__ int entry_mask(const unsigned (&m)[3], const Item &it) {
    const unsigned t = (m[0] >> it.c0) & 1u;
    const unsigned row = (m[1] >> (2 * it.c1)) & (3u * t);
    const unsigned col = (m[2] >> (2 * it.c2)) & 3u;
    // bit e = row bit (e >> 1) & col bit (e & 1): col spread by the row bits
    return (int)(col * (row + (row & 2u)));
}


// Index of the block's patch along W inside the tile; blocks of one quarter
// wave with odd index visit the entries of a patch in the order e ^ 1 in their
// d-major reads (this is what makes those reads conflict-free, see swz).
__device__ __forceinline__ int entry_flip(int lane) { return (lane >> 2) & 1; }


// Output of the merged results: thread qd (0..3) of a point writes G = D / 4
// elements as 16-byte (or, for bf16 D = 16, 8-byte) pieces, piece j at element
// (4 j + qd) * W, so the four threads of a point write contiguous bytes in
// every store instruction (no partially written lines).
template <typename T, int D>
__device__ __forceinline__ constexpr int piece_elems() {
    return (D / 4) >= (16 / (int)sizeof(T)) ? 16 / (int)sizeof(T) : D / 4;
}
template <typename T, int D>
__device__ __forceinline__ int piece_offset(int j, int qd) {
    return (4 * j + qd) * piece_elems<T, D>();
}

// Reorder a 4-vector indexed by entry into the block's visiting order
// (entries e ^ flip): swap the members of each pair when flip is set.
__device__ __forceinline__ void swap_pairs(float (&v)[4], int flip) {
    const bool f = flip != 0;
    const float a0 = f ? v[1] : v[0], a1 = f ? v[0] : v[1];
    const float a2 = f ? v[3] : v[2], a3 = f ? v[2] : v[3];
    v[0] = a0; v[1] = a1; v[2] = a2; v[3] = a3;
}

// Chunk bookkeeping shared by the kernels: the items of a walk over a chunk
// cut along T are either wholly inside or outside it (all blocks of a tile
// share their T start); a cut along H masks entries one by one.
struct ChunkView {
    unsigned lim;    // largest valid point index for clamped reads
    bool chunked;    // the staged box is split
    int A;           // cut axis
};

// 4-bit mask of the entries of an item whose cut-axis row lies in the chunk.
__device__ __forceinline__ int chunk_mask(const ChunkView &cv, const Box &C, int start_a,
                                          const Item &it) {
    if (!cv.chunked) return 15;
    if (cv.A == 0) {
        const int r = start_a - C.o[0] + it.c0;
        return (r >= 0 && r < C.e[0]) ? 15 : 0;
    }
    const int r = start_a - C.o[1] + 2 * it.c1;
    const int lo = (r >= 0 && r < C.e[1]) ? 3 : 0, hi = (r + 1 >= 0 && r + 1 < C.e[1]) ? 12 : 0;
    return lo | hi;
}

// Window masks (the masked entry points). Byte j of the row of query token x
// (K bytes per token of one (batch, head) plane, tokens in row-major (T, H, W)
// grid order, shared by every batch element and head) is zero when x drops
// the j-th key of its window (window offsets in row-major (t, h, w) order).
// qc, kc: class coordinates of a query and of a key of its window.
__device__ __forceinline__ bool mask_keeps(const uint8_t *mask, int K, const Geometry &g,
                                           const TileCtx &w, const int (&qc)[3],
                                           const int (&kc)[3]) {
    int64_t tok = 0;
    int j = 0;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        tok = tok * g.ext[x] + (int64_t)qc[x] * w.d[x] + w.r[x];
        j = j * w.k[x] + (kc[x] - window_start(qc[x], w.n[x], w.k[x]));
    }
    return mask[tok * K + j] != 0;
}

// The entry bits mk of an item with the dropped pairs cleared. QUERY_LANE: the
// lane holds a query and the item's entries are keys of its window, walked
// from st; else the lane holds a key and the entries are queries of its
// inverse window, walked from st. Only entries already valid are looked up,
// so every mask byte read lies in the row of an in-grid query.
template <bool QUERY_LANE>
__device__ __forceinline__ int mask_entries(int mk, const uint8_t *mask, int K, const Geometry &g,
                                            const TileCtx &w, const int (&own)[3],
                                            const int (&st)[3], const Item &it) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (!((mk >> e) & 1)) continue;
        const int other[3] = {st[0] + it.c0, st[1] + 2 * it.c1 + (e >> 1),
                              st[2] + 2 * it.c2 + (e & 1)};
        const bool keep = QUERY_LANE ? mask_keeps(mask, K, g, w, own, other)
                                     : mask_keeps(mask, K, g, w, other, own);
        if (!keep) mk &= ~(1 << e);
    }
    return mk;
}

// ============================================================================
// Forward: out, lse.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads, kSplitOccupancy<D>) fwd_kernel(FwdArgs a) {
    extern __shared__ __align__(16) char smem[];
    constexpr int G = D / 4, PB = D * (int)sizeof(T), NC = PB / 16;
    TileCtx w;
    if (!decode_tile(a.g, xcd_tile_id(blockIdx.x, a.g.n_tiles), w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3, flip = entry_flip(lane);
    const LanePoint lp = lane_point(w, lane);

    // keys the tile needs (union of its queries' windows, padded to the walks)
    Box U;
    int us[3], cnt[3];
    unsigned vm[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        key_box(w.o[x], kTile[x], kPatch[x], w.n[x], w.k[x], &U.o[x], &U.e[x]);
        us[x] = window_start(lp.f[x], w.n[x], w.k[x]);
        vm[x] = bit_range(window_start(lp.p[x], w.n[x], w.k[x]) - us[x], w.k[x]);
        if (a.frame && x == a.frame_axis)
            vm[x] &= frame_bits(us[x], lp.p[x], w.n[x], frame_size(a.frame, w, x, lp.p[x]));
        cnt[x] = window_walk(w.k[x], kPatch[x]);
    }
    const int ncount = cnt[0] * cnt[1] * cnt[2];

    float qr[D];
    load_row<T, D>(static_cast<const T *>(a.q) + elem_off(w, lp.p), qr);
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] *= a.qscale;

    float m = -1e30f, l = 0.f;
    f4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};

    ChunkView cv;
    cv.A = a.g.chunk_axis;
    const int rows = chunk_rows(U, cv.A, 2 * PB, a.g.lds_budget);
    cv.chunked = rows < get3(U.e, cv.A);
    for (int r0 = 0; r0 < get3(U.e, cv.A); r0 += rows) {
        const Box C = chunk_of(U, cv.A, r0, rows);
        const int np = C.e[0] * C.e[1] * C.e[2];
        char *Ks = smem, *Vs = smem + np * PB;
        if (r0 > 0) __syncthreads();
        stage_box<T, D>(static_cast<const T *>(a.k), w, C, Ks);
        stage_box<T, D>(static_cast<const T *>(a.v), w, C, Vs);
        stage_wait();
        cv.lim = (cv.chunked && cv.A != 0) ? (unsigned)((np - 1) * PB) : 0xffffffffu;
        const Entry own = make_entry<NC>(C, us, c);
        Entry dm[4];
#pragma unroll
        for (int kap = 0; kap < 4; ++kap) dm[kap] = make_entry<NC>(C, us, kap ^ flip);

        for (int i = wave; i < ncount; i += kWaves) {
            const Item it = make_item<PB>(i, cnt, C);
            const int cm = chunk_mask(cv, C, get3(us, cv.A), it);
            if (cv.chunked && cv.A == 0 && cm == 0) continue;  // uniform along T
            int mk = entry_mask(vm, it) & cm;
            if (a.mask) mk = mask_entries<true>(mk, a.mask, a.mask_k, a.g, w, lp.p, us, it);
            // items every lane of the wave drops: no work (a masked tile's speedup)
            if (a.mask && !__any(mk != 0)) continue;
            // S_b[i][c] = <k_i, q_c>: this lane supplies key c of the patch
            f4 s;
            {
                float kr[D];
                lds_point_at<T, D>(Ks, entry_addr(own, it, cv.lim), kr);
                f4 s0 = f4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    s0 = mfma4(kr[d], qr[d], s0);
                    s1 = mfma4(kr[d + 1], qr[d + 1], s1);
                }
                s = s0 + s1;
            }
            float sv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e] = (mk >> e) & 1 ? s[e] : -INFINITY;
            // online softmax; the running maximum only moves (and the sums are
            // rescaled) when a score exceeds it by more than 2^8, so exp2 stays
            // below 256 and out = acc / l is unchanged
            const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            if (__any(mx > m + 8.f)) {
                const float mn = fmaxf(m, mx);
                const float alpha = fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] *= alpha;
                m = mn;
            }
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = fast_exp2(sv[e] - m);
            l += (p[0] + p[1]) + (p[2] + p[3]);
            swap_pairs(p, flip);

            // O_b[i][c] += v_e[i*G + g] * P[c][e]: this lane supplies the
            // quarter c of every key e of the patch (blocks visit e = kap ^ flip)
#pragma unroll
            for (int kap = 0; kap < 4; ++kap) {
                float vr[G];
                lds_quarter_at<T, D>(Vs, entry_addr(dm[kap], it, cv.lim), c, vr);
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = mfma4(vr[g], p[kap], acc[g]);
            }
        }
    }

    // merge the four waves' partial softmax states through LDS
    __syncthreads();
    float *mb = reinterpret_cast<float *>(smem);
    {
        float *mine = mb + (wave * 64 + lane) * (D + 3);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g) mine[i * G + g] = acc[g][i];
        mine[D] = m;
        mine[D + 1] = l;
    }
    __syncthreads();
    {
        const int L = threadIdx.x >> 2, qd = threadIdx.x & 3;
        float mw[kWaves], M = -1e30f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            mw[v] = mb[(v * 64 + L) * (D + 3) + D];
            M = fmaxf(M, mw[v]);
        }
        float Ls = 0.f, o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g] = 0.f;
        constexpr int PE = piece_elems<T, D>();
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float sc = exp2f(mw[v] - M);
            const float *src = mb + (v * 64 + L) * (D + 3);
            Ls += src[D + 1] * sc;
#pragma unroll
            for (int j = 0; j < G / PE; ++j)
#pragma unroll
                for (int x = 0; x < PE; ++x)
                    o[j * PE + x] += src[piece_offset<T, D>(j, qd) + x] * sc;
        }
        const LanePoint qp = lane_point(w, L);
        if (qp.active) {
            // a query whose window is masked away entirely: zero output, lse -inf
            const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) o[g] *= inv;
            T *O = static_cast<T *>(a.out) + elem_off(w, qp.p);
#pragma unroll
            for (int j = 0; j < G / PE; ++j)
#pragma unroll
                for (int x = 0; x < PE; x += 4)
                    Io<T>::store4(O + piece_offset<T, D>(j, qd) + x, o + j * PE + x);
            if (qd == 0) a.lse[row_off(w, qp.p)] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
        }
    }
}

// ============================================================================
// Backward, query side: delta and dq.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads, kSplitOccupancy<D>) dq_kernel(BwdArgs a) {
    extern __shared__ __align__(16) char smem[];
    constexpr int G = D / 4, PB = D * (int)sizeof(T), NC = PB / 16;
    TileCtx w;
    if (!decode_tile(a.g, xcd_tile_id(blockIdx.x, a.g.n_tiles), w)) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3, flip = entry_flip(lane);
    const LanePoint lp = lane_point(w, lane);

    Box U;
    int us[3], cnt[3];
    unsigned vm[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        key_box(w.o[x], kTile[x], kPatch[x], w.n[x], w.k[x], &U.o[x], &U.e[x]);
        us[x] = window_start(lp.f[x], w.n[x], w.k[x]);
        vm[x] = bit_range(window_start(lp.p[x], w.n[x], w.k[x]) - us[x], w.k[x]);
        if (a.frame && x == a.frame_axis)
            vm[x] &= frame_bits(us[x], lp.p[x], w.n[x], frame_size(a.frame, w, x, lp.p[x]));
        cnt[x] = window_walk(w.k[x], kPatch[x]);
    }
    const int ncount = cnt[0] * cnt[1] * cnt[2];

    const int64_t qo = elem_off(w, lp.p);
    float qr[D], dor[D];
    load_row<T, D>(static_cast<const T *>(a.q) + qo, qr);
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

    ChunkView cv;
    cv.A = a.g.chunk_axis;
    const int rows = chunk_rows(U, cv.A, 2 * PB, a.g.lds_budget);
    cv.chunked = rows < get3(U.e, cv.A);
    for (int r0 = 0; r0 < get3(U.e, cv.A); r0 += rows) {
        const Box C = chunk_of(U, cv.A, r0, rows);
        const int np = C.e[0] * C.e[1] * C.e[2];
        char *Ks = smem, *Vs = smem + np * PB;
        if (r0 > 0) __syncthreads();
        stage_box<T, D>(static_cast<const T *>(a.k), w, C, Ks);
        stage_box<T, D>(static_cast<const T *>(a.v), w, C, Vs);
        stage_wait();
        cv.lim = (cv.chunked && cv.A != 0) ? (unsigned)((np - 1) * PB) : 0xffffffffu;
        const Entry own = make_entry<NC>(C, us, c);
        Entry dm[4];
#pragma unroll
        for (int kap = 0; kap < 4; ++kap) dm[kap] = make_entry<NC>(C, us, kap ^ flip);

        for (int i = wave; i < ncount; i += kWaves) {
            const Item it = make_item<PB>(i, cnt, C);
            const int cm = chunk_mask(cv, C, get3(us, cv.A), it);
            if (cv.chunked && cv.A == 0 && cm == 0) continue;
            int mk = entry_mask(vm, it) & cm;
            if (a.mask) mk = mask_entries<true>(mk, a.mask, a.mask_k, a.g, w, lp.p, us, it);
            // items every lane of the wave drops: no work (a masked tile's speedup)
            if (a.mask && !__any(mk != 0)) continue;
            const int ao = entry_addr(own, it, cv.lim);
            f4 s, dp;
            {
                float kr[D];
                lds_point_at<T, D>(Ks, ao, kr);
                f4 s0 = f4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    s0 = mfma4(kr[d], qr[d], s0);
                    s1 = mfma4(kr[d + 1], qr[d + 1], s1);
                }
                s = s0 + s1;
            }
            {
                float vr[D];
                lds_point_at<T, D>(Vs, ao, vr);
                f4 d0 = f4{0.f, 0.f, 0.f, 0.f}, d1 = d0;
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    d0 = mfma4(vr[d], dor[d], d0);
                    d1 = mfma4(vr[d + 1], dor[d + 1], d1);
                }
                dp = d0 + d1;
            }
            float ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = (mk >> e) & 1 ? fast_exp2(s[e] - lse2) : 0.f;
                ds[e] = p * (dp[e] - delta);
            }
            // dQ_b[i][c] += k_e[i*G + g] * dS[c][e]
            swap_pairs(ds, flip);
#pragma unroll
            for (int kap = 0; kap < 4; ++kap) {
                float kd[G];
                lds_quarter_at<T, D>(Ks, entry_addr(dm[kap], it, cv.lim), c, kd);
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = mfma4(kd[g], ds[kap], acc[g]);
            }
        }
    }

    // sum the four waves' partial dq through LDS
    __syncthreads();
    float *mb = reinterpret_cast<float *>(smem);
    {
        float *mine = mb + (wave * 64 + lane) * (D + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g) mine[i * G + g] = acc[g][i];
    }
    __syncthreads();
    {
        const int L = threadIdx.x >> 2, qd = threadIdx.x & 3;
        float o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g] = 0.f;
        constexpr int PE = piece_elems<T, D>();
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float *src = mb + (v * 64 + L) * (D + 1);
#pragma unroll
            for (int j = 0; j < G / PE; ++j)
#pragma unroll
                for (int x = 0; x < PE; ++x) o[j * PE + x] += src[piece_offset<T, D>(j, qd) + x];
        }
        const LanePoint qp = lane_point(w, L);
        if (qp.active) {
#pragma unroll
            for (int g = 0; g < G; ++g) o[g] *= a.scale;
            T *DQ = static_cast<T *>(a.dq) + elem_off(w, qp.p);
#pragma unroll
            for (int j = 0; j < G / PE; ++j)
#pragma unroll
                for (int x = 0; x < PE; x += 4)
                    Io<T>::store4(DQ + piece_offset<T, D>(j, qd) + x, o + j * PE + x);
        }
    }
    if (wave == 0 && lp.active) a.delta[row_off(w, lp.p)] = delta;
}

// ============================================================================
// Backward, key side: dk and dv by inverse-neighborhood gather. MODE 0: only
// that. MODE 1 (KV-parallel): the same pass also produces each query's dq
// contributions from this tile's keys and adds them into the fp32 accumulator
// dq_acc with float atomics (not bitwise reproducible). MODE 2 (KV-parallel,
// deterministic): the contributions of each staged chunk of the query box are
// summed exactly in LDS (fixed point), then added with plain stores into the
// tile's class copy of the accumulator; no two tiles of one launch touch the
// same element of a copy.
// The KV-parallel pass keeps the block's keys for dq besides everything else
// and, with its LDS dq accumulator, runs one workgroup per CU anyway.
template <typename T, int D, int MODE>
__global__ void __launch_bounds__(kThreads, MODE != 0 ? 1 : kSplitOccupancy<D>) dkdv_kernel(BwdArgs a) {
    extern __shared__ __align__(16) char smem[];
    constexpr bool KVPAR = MODE != 0;
    constexpr int G = D / 4, PB = D * (int)sizeof(T), NC = PB / 16;
    TileCtx w;
    if (!decode_tile(a.g, xcd_tile_id(blockIdx.x, a.g.n_tiles), w)) return;
    float *copy = nullptr;
    if constexpr (MODE == 2) {
        const int cls = ((w.o[0] / kTile[0]) % a.cls_m[0] * a.cls_m[1] +
                         (w.o[1] / kTile[1]) % a.cls_m[1]) * a.cls_m[2] +
                        (w.o[2] / kTile[2]) % a.cls_m[2];
        if (cls < a.cls_lo || cls >= a.cls_lo + a.cls_n) return;
        copy = a.dq_acc + (int64_t)(cls - a.cls_lo) * a.copy_stride;
    }
    if (a.skip_ch > 0) {
        const int o1 = w.o[1] & ~15, o2 = w.o[2] & ~15;
        if (tile_inverse_walk(o1, 16, 2, w.n[1], w.k[1]) <= a.skip_ch &&
            tile_inverse_walk(o2, 16, 2, w.n[2], w.k[2]) <= a.skip_cw)
            return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 3, flip = entry_flip(lane);
    const LanePoint lp = lane_point(w, lane);  // here: this lane's key

    // queries the tile needs: the union of its keys' inverse windows
    Box U;
    int lo[3], cnt[3];
    unsigned vm[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        cnt[x] = tile_inverse_walk(w.o[x], kTile[x], kPatch[x], w.n[x], w.k[x]);
        query_box(w.o[x], kTile[x], kPatch[x], w.n[x], w.k[x], cnt[x], &U.o[x], &U.e[x]);
        lo[x] = inverse_first(lp.f[x], w.n[x], w.k[x]);
        const int ilo = inverse_first(lp.p[x], w.n[x], w.k[x]);
        vm[x] = bit_range(ilo - lo[x], inverse_last(lp.p[x], w.n[x], w.k[x]) - ilo + 1);
        if (a.frame && x == a.frame_axis)
            vm[x] &= frame_bits_inverse(a.frame, w, x, lo[x], lp.p[x], w.n[x], 32);
    }
    const int ncount = cnt[0] * cnt[1] * cnt[2];

    const int64_t ko = elem_off(w, lp.p);
    float kr[D], vr[D];
    load_row<T, D>(static_cast<const T *>(a.k) + ko, kr);
    load_row<T, D>(static_cast<const T *>(a.v) + ko, vr);
#pragma unroll
    for (int d = 0; d < D; ++d) kr[d] *= a.qscale;
    // KV-parallel: the block's four keys, quarter c of each, for dq += dS k
    float kq[KVPAR ? 4 : 1][KVPAR ? G : 1];
    if constexpr (KVPAR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int kj[3];
            patch_point(lp.f, j, kj);
#pragma unroll
            for (int x = 0; x < 3; ++x) kj[x] = imin(kj[x], w.n[x] - 1);
            load_row<T, G>(static_cast<const T *>(a.k) + elem_off(w, kj) + c * G, kq[j]);
        }
    }

    f4 dk[G], dv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        dk[g] = f4{0.f, 0.f, 0.f, 0.f};
        dv[g] = f4{0.f, 0.f, 0.f, 0.f};
    }
    // KV-parallel with an LDS accumulator: the tile's dq contributions are
    // summed over its query box U in LDS (points D + 1 floats apart), then
    // added to the global accumulator once per point and channel. Zeroed here;
    // the barrier of the first staging orders it before any addition.
    float *qacc = nullptr;
    if constexpr (MODE == 1) {
        if (a.g.dq_lds_off > 0) {
            qacc = reinterpret_cast<float *>(smem + a.g.dq_lds_off);
            const int n = U.e[0] * U.e[1] * U.e[2] * (D + 1);
            for (int i = threadIdx.x; i < n; i += kThreads) qacc[i] = 0.f;
        }
    }

    ChunkView cv;
    cv.A = a.g.chunk_axis;
    // MODE 2 keeps a 64-bit accumulator per point and channel of the chunk
    const int rows = chunk_rows(U, cv.A, 2 * PB + 8 + (MODE == 2 ? 8 * D : 0), a.g.lds_budget);
    cv.chunked = rows < get3(U.e, cv.A);
    for (int r0 = 0; r0 < get3(U.e, cv.A); r0 += rows) {
        const Box C = chunk_of(U, cv.A, r0, rows);
        const int np = C.e[0] * C.e[1] * C.e[2];
        char *Qs = smem, *Os = smem + np * PB;
        float2 *Rs = reinterpret_cast<float2 *>(smem + 2 * np * PB);
        unsigned long long *fix = reinterpret_cast<unsigned long long *>(smem + 2 * np * PB + 8 * np);
        if (r0 > 0) __syncthreads();
        if constexpr (MODE == 2) {
            // the barrier of this chunk's staging orders the clearing before any addition
            for (int i = threadIdx.x; i < np * D; i += kThreads) fix[i] = 0ull;
        }
        stage_box<T, D>(static_cast<const T *>(a.q), w, C, Qs);
        stage_box<T, D>(static_cast<const T *>(a.dout), w, C, Os);
        stage_rows(a.lse, a.delta, w, C, Rs);
        stage_wait();
        cv.lim = (cv.chunked && cv.A != 0) ? (unsigned)((np - 1) * PB) : 0xffffffffu;
        const Entry own = make_entry<NC>(C, lo, c);
        Entry dm[4], row[4];
#pragma unroll
        for (int kap = 0; kap < 4; ++kap) {
            dm[kap] = make_entry<NC>(C, lo, kap ^ flip);
            row[kap] = make_entry<NC>(C, lo, kap);
        }

        for (int i = wave; i < ncount; i += kWaves) {
            const Item it = make_item<PB>(i, cnt, C);
            const int cm = chunk_mask(cv, C, get3(lo, cv.A), it);
            if (cv.chunked && cv.A == 0 && cm == 0) continue;
            int mk = entry_mask(vm, it) & cm;
            if (a.mask) mk = mask_entries<false>(mk, a.mask, a.mask_k, a.g, w, lp.p, lo, it);
            // items every lane of the wave drops: no work (a masked tile's speedup)
            if (a.mask && !__any(mk != 0)) continue;
            // S_b[i][c] = <q_i, k_c>: this lane supplies query c of the patch
            const int ao = entry_addr(own, it, cv.lim);
            f4 s, dp;
            {
                float q_[D];
                lds_point_at<T, D>(Qs, ao, q_);
                f4 s0 = f4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    s0 = mfma4(q_[d], kr[d], s0);
                    s1 = mfma4(q_[d + 1], kr[d + 1], s1);
                }
                s = s0 + s1;
            }
            {
                float o_[D];
                lds_point_at<T, D>(Os, ao, o_);
                f4 d0 = f4{0.f, 0.f, 0.f, 0.f}, d1 = d0;
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    d0 = mfma4(o_[d], vr[d], d0);
                    d1 = mfma4(o_[d + 1], vr[d + 1], d1);
                }
                dp = d0 + d1;
            }
            float p[4], ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 ld = Rs[umin((unsigned)(row[e].ptb + it.offb), cv.lim) / PB];
                p[e] = (mk >> e) & 1 ? fast_exp2(s[e] - ld.x) : 0.f;
                ds[e] = p[e] * (dp[e] - ld.y);
            }
            // dV_b[i][c] += dout_e[i*G + g] * P[e][c];
            // dK_b[i][c] += q_e[i*G + g] * dS[e][c]
            float pf[4] = {p[0], p[1], p[2], p[3]}, dsf[4] = {ds[0], ds[1], ds[2], ds[3]};
            swap_pairs(pf, flip);
            swap_pairs(dsf, flip);
#pragma unroll
            for (int kap = 0; kap < 4; ++kap) {
                const int ad = entry_addr(dm[kap], it, cv.lim);
                float od[G], qd[G];
                lds_quarter_at<T, D>(Os, ad, c, od);
                lds_quarter_at<T, D>(Qs, ad, c, qd);
#pragma unroll
                for (int g = 0; g < G; ++g) dv[g] = mfma4(od[g], pf[kap], dv[g]);
#pragma unroll
                for (int g = 0; g < G; ++g) dk[g] = mfma4(qd[g], dsf[kap], dk[g]);
            }

            if constexpr (KVPAR) {
                // A lane whose key lies past the grid edge was clamped onto a
                // real key; it must not add that key's contribution twice.
                float dsk[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) dsk[j] = lp.active ? ds[j] : 0.f;
                // transpose dS inside the block: lane 4b+c gets
                // tr[j] = dS[query c][key j] (held by lane 4b+j, register c)
                float tr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int src = (lane & ~3) | j;
                    const float x0 = __shfl(dsk[0], src), x1 = __shfl(dsk[1], src);
                    const float x2 = __shfl(dsk[2], src), x3 = __shfl(dsk[3], src);
                    tr[j] = c == 0 ? x0 : c == 1 ? x1 : c == 2 ? x2 : x3;
                }
                // dQ_b[i][c] = sum_j k_j[i*G + g] * dS[c][j]
                f4 dq[G];
#pragma unroll
                for (int g = 0; g < G; ++g) dq[g] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g = 0; g < G; ++g) dq[g] = mfma4(kq[j][g], tr[j], dq[g]);
                const int qq[3] = {lo[0] + it.c0, lo[1] + 2 * it.c1 + (c >> 1),
                                   lo[2] + 2 * it.c2 + (c & 1)};
                const bool inside = qq[0] < w.n[0] && qq[1] < w.n[1] && qq[2] < w.n[2] &&
                                    ((cm >> c) & 1);
                if constexpr (MODE == 2) {
                    if (inside) {
                        unsigned long long *fp =
                            fix + (((qq[0] - C.o[0]) * C.e[1] + (qq[1] - C.o[1])) * C.e[2] +
                                   (qq[2] - C.o[2])) * D;
#pragma unroll
                        for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
                            for (int g = 0; g < G; ++g)
                                atomicAdd(fp + i2 * G + g,
                                          (unsigned long long)__float2ll_rn(dq[g][i2] * kFixOne));
                    }
                } else if (inside && qacc) {
                    float *ap = qacc + (((qq[0] - U.o[0]) * U.e[1] + (qq[1] - U.o[1])) * U.e[2] +
                                        (qq[2] - U.o[2])) * (D + 1);
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
                        for (int g = 0; g < G; ++g) atomicAdd(ap + i2 * G + g, dq[g][i2]);
                } else if (inside) {
                    float *accp = a.dq_acc + elem_off(w, qq);
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
                        for (int g = 0; g < G; ++g) atomicAdd(accp + i2 * G + g, dq[g][i2]);
                }
            }
        }
        if constexpr (MODE == 2) {
            // the chunk's exact sums into the tile's copy, one thread per element
            __syncthreads();
            const int plane = C.e[1] * C.e[2];
            for (int i = threadIdx.x; i < np * D; i += kThreads) {
                const int pt = i / D, d = i - pt * D;
                const int z = pt / plane, r = pt - z * plane, y = r / C.e[2], x = r - y * C.e[2];
                const int qq[3] = {C.o[0] + z, C.o[1] + y, C.o[2] + x};
                if (qq[0] < w.n[0] && qq[1] < w.n[1] && qq[2] < w.n[2]) {
                    float *dst = copy + elem_off(w, qq) + d;
                    *dst += (float)(long long)fix[i] * kFixInv;
                }
            }
        }
    }

    if constexpr (MODE == 1) {
        if (qacc) {
            // the box's sums into the global accumulator (points past the grid
            // never received any)
            __syncthreads();
            const int plane = U.e[1] * U.e[2], n = U.e[0] * plane * D;
            for (int i = threadIdx.x; i < n; i += kThreads) {
                const int pt = i / D, d = i - pt * D;
                const int z = pt / plane, r = pt - z * plane, y = r / U.e[2], x = r - y * U.e[2];
                const int qq[3] = {U.o[0] + z, U.o[1] + y, U.o[2] + x};
                const float v = qacc[pt * (D + 1) + d];
                if (qq[0] < w.n[0] && qq[1] < w.n[1] && qq[2] < w.n[2] && v != 0.f)
                    atomicAdd(a.dq_acc + elem_off(w, qq) + d, v);
            }
        }
    }

    // sum the four waves' partial dk, then dv, through LDS
    float *mb = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        __syncthreads();
        {
            float *mine = mb + (wave * 64 + lane) * (D + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g) mine[i * G + g] = round == 0 ? dk[g][i] : dv[g][i];
        }
        __syncthreads();
        const int L = threadIdx.x >> 2, qd = threadIdx.x & 3;
        float o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g] = 0.f;
        constexpr int PE = piece_elems<T, D>();
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float *src = mb + (v * 64 + L) * (D + 1);
#pragma unroll
            for (int j = 0; j < G / PE; ++j)
#pragma unroll
                for (int x = 0; x < PE; ++x) o[j * PE + x] += src[piece_offset<T, D>(j, qd) + x];
        }
        const LanePoint kp = lane_point(w, L);
        if (kp.active) {
            const float mul = round == 0 ? a.scale : 1.f;
#pragma unroll
            for (int g = 0; g < G; ++g) o[g] *= mul;
            T *dst = static_cast<T *>(round == 0 ? a.dk : a.dv) + elem_off(w, kp.p);
#pragma unroll
            for (int j = 0; j < G / PE; ++j)
#pragma unroll
                for (int x = 0; x < PE; x += 4)
                    Io<T>::store4(dst + piece_offset<T, D>(j, qd) + x, o + j * PE + x);
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

// Zero n4 float4s.
__global__ void __launch_bounds__(256) zero_kernel(float *p, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4) reinterpret_cast<float4 *>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// dq = scale * (copy 0 + copy 1 + ... + copy n-1), summed in that order, cast
// to the tensor type; four elements per thread.
template <typename T>
__global__ void __launch_bounds__(256) dq_copies_finalize_kernel(const float *acc, int ncopies,
                                                                 int64_t stride, T *dq, float scale,
                                                                 int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < ncopies; ++c) {
        float x[4];
        Io<float>::load4(acc + c * stride + 4 * i, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= scale;
    Io<T>::store4(dq + 4 * i, v);
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
