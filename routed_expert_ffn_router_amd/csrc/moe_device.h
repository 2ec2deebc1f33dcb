// moe_device.h -- device-side building blocks of libmoe (gfx950 only).
//
// Weight-format decoders (the formats of include/moe.h), dot products on the
// gfx950 dot2 instructions, and wavefront (64-lane) reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// --------------------------------------------------------------------------
// scalars
// --------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// OCP MX E8M0 scale 2^(e-127) as an exact fp32 (e = 0 is the subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : (e == 255 ? __uint_as_float(0x7FC00000u)
                                                           : __uint_as_float(e << 23));
}

// acc + a.lo*b.lo + a.hi*b.hi on bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// acc + a.lo*b.lo + a.hi*b.hi on fp16 pairs (v_dot2_f32_f16)
typedef _Float16 f16x2_dev_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_dev_t, a),
                                __builtin_bit_cast(f16x2_dev_t, b), acc, false);
}

// two E2M1 nibbles (byte `sel` of w, low nibble first) -> fp16 pair, exact
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

// two E2M1 nibbles (byte `sel` of w, low nibble first) -> bf16 pair, exact
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// --------------------------------------------------------------------------
// reductions over aligned groups of G lanes (G a power of two <= 64)
// --------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int G>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// --------------------------------------------------------------------------
// block -> (row tile, column block) of the grouped GEMMs, XCD-aware:
// workgroups go round-robin to the 8 XCDs (linear id b on XCD b % 8), each
// with its own L2.
//  * Grouped experts (rows first): XCD x takes the x-th eighth of the tile
//    list in order and walks all column blocks of a tile back to back.  An
//    expert's tiles are adjacent in the list, so they run together on one
//    XCD and its weights are fetched into one L2 once, not once per tile.
//  * One dense expert over many tiles (weight_major): XCD x takes column
//    blocks x, x + 8, ... (grid.x a multiple of 8) and walks all tiles of
//    one back to back, so its L2 keeps that block of weights.
// grid.y is a multiple of 8 and at least n_tiles.  False for a block past the
// real tiles.
// --------------------------------------------------------------------------
__device__ __forceinline__ bool block_tile(bool weight_major, int n_tiles, int *ti, int *bx) {
  const uint32_t nbx = gridDim.x, nby = gridDim.y;
  const uint32_t bid = blockIdx.y * nbx + blockIdx.x;
  const uint32_t jx = bid >> 3, x = bid & 7;
  if (weight_major) {
    *ti = (int)(jx % nby);
    *bx = (int)((jx / nby) * 8 + x);
    return *ti < n_tiles;
  }
  const int q = (int)(jx / nbx), per = (n_tiles + 7) >> 3;
  *ti = (int)x * per + q;
  *bx = (int)(jx % nbx);
  return q < per && *ti < n_tiles;
}

// --------------------------------------------------------------------------
// Q2K super-block (84 bytes): sc[16] | qs[64] | fp16 d | fp16 dmin
// --------------------------------------------------------------------------
constexpr int kQ2KBytes = 84;

// weight i of a block, exact: (d*scale)*q and dmin*min are exact in fp32,
// so the only rounding is the final subtraction
__device__ __forceinline__ float q2k_weight(const uint8_t *blk, int i) {
  const int s = i >> 4;
  const uint32_t scm = blk[s];
  const uint32_t q = (blk[16 + (i >> 2)] >> (2 * (i & 3))) & 3u;
  const uint32_t dm = *reinterpret_cast<const uint32_t *>(blk + 80);
  const float d = f16_bits_to_f32(dm & 0xFFFFu), dmin = f16_bits_to_f32(dm >> 16);
  const float hi = (d * (float)(scm & 15u)) * (float)q;
  const float lo = dmin * (float)(scm >> 4);
  return hi - lo;
}

// VQ2 weight: d * codebook[code][k%4]
__device__ __forceinline__ float vq2_weight(uint32_t code, int lane4, float d, const int8_t *cb) {
  return d * (float)cb[code * 4 + lane4];
}

// MXFP4 weight: E2M1(nibble) * 2^(e-127)
__device__ __forceinline__ float mxfp4_weight(uint32_t byte, int hi, uint32_t e) {
  uint32_t p = e2m1x2_to_bf16x2<0>(byte);
  float v = hi ? bf16_hi(p) : bf16_lo(p);
  return v * e8m0_to_f32(e);
}

}  // namespace moe
