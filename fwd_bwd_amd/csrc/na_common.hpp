// na_common.hpp -- types, element I/O and per-wave geometry shared by the
// neighborhood-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "na_index.hpp"

namespace na {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16;  // storage of a bfloat16 value

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------------------
// Element I/O. Tensors are fp32 or bf16; arithmetic is always fp32. A "chunk"
// is 4 consecutive elements (16 bytes of fp32, 8 bytes of bf16).

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename T>
struct Io;

template <>
struct Io<float> {
    __device__ __forceinline__ static void load4(const float *p, float *d) {
        float4 v = *reinterpret_cast<const float4 *>(p);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __device__ __forceinline__ static void store4(float *p, const float *s) {
        *reinterpret_cast<float4 *>(p) = make_float4(s[0], s[1], s[2], s[3]);
    }
};

template <>
struct Io<bf16> {
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
// So with A = a key-indexed operand and B = a query-indexed one, lane 4b+c
// ends up holding the products of its own query c with the 4 keys of its
// block, one per register.
__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------------------------------
// Problem geometry, as the host hands it to every kernel. Axis 0 is T (1 for
// 2D problems), axis 1 is H, axis 2 is W.

// One wave covers a tile of 1 x 8 x 8 class coordinates, split into 16
// patches of 1 x 2 x 2 (one patch per 4-lane MFMA block).
constexpr int kPatch[3] = {1, 2, 2};
constexpr int kWaveTile[3] = {1, 8, 8};
constexpr int kWavesPerBlock = 4;

struct Geometry {
    int ext[3], ker[3], dil[3];
    int heads, batch, head_dim;
    int tiles[3];     // wave tiles per axis, over the largest residue class
    int nres;         // dil[0] * dil[1] * dil[2]
    int n_waves;      // batch * heads * nres * tiles[0] * tiles[1] * tiles[2]
};

// Where one wave works: batch element, head, residue class, tile origin, and
// the address arithmetic of that class.
struct WaveCtx {
    int n[3], k[3];     // class sizes and window sizes per axis
    int o[3];           // tile origin in class coordinates
    int64_t base;       // element offset of (b, class origin token, head, 0)
    int64_t st[3];      // element offset of one class step per axis
    int64_t lbase;      // lse / delta offset of (b, class origin token, head)
    int64_t lst[3];     // lse / delta offset of one class step per axis
};

// Decodes the wave id (tile fastest, then residue, head, batch). Returns false
// when the tile lies past the end of this residue class (the whole wave exits).
__device__ __forceinline__ bool decode_wave(const Geometry &g, int wave, WaveCtx &w) {
    int rem = wave;
    int tw = rem % g.tiles[2]; rem /= g.tiles[2];
    int th = rem % g.tiles[1]; rem /= g.tiles[1];
    int tt = rem % g.tiles[0]; rem /= g.tiles[0];
    int res = rem % g.nres; rem /= g.nres;
    int head = rem % g.heads; rem /= g.heads;
    int b = rem;
    int r[3];
    r[2] = res % g.dil[2];
    r[1] = (res / g.dil[2]) % g.dil[1];
    r[0] = res / (g.dil[2] * g.dil[1]);
    const int t_idx[3] = {tt, th, tw};
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        w.n[a] = class_size(g.ext[a], g.dil[a], r[a]);
        w.k[a] = g.ker[a];
        w.o[a] = t_idx[a] * kWaveTile[a];
        inside = inside && (w.o[a] < w.n[a]);
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

__device__ __forceinline__ int64_t elem_off(const WaveCtx &w, const int (&c)[3]) {
    return w.base + c[0] * w.st[0] + c[1] * w.st[1] + c[2] * w.st[2];
}
__device__ __forceinline__ int64_t row_off(const WaveCtx &w, const int (&c)[3]) {
    return w.lbase + c[0] * w.lst[0] + c[1] * w.lst[1] + c[2] * w.lst[2];
}

// Coordinates of entry c (0..3) of the 1x2x2 patch whose first point is f.
__device__ __forceinline__ void patch_point(const int (&f)[3], int c, int (&p)[3]) {
    p[0] = f[0];
    p[1] = f[1] + (c >> 1);
    p[2] = f[2] + (c & 1);
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) v = imax(v, __shfl_xor(v, m));
    return v;
}

}  // namespace na
