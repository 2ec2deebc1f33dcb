// gemv_core.h -- building blocks of the decode GEMVs (see gemv.hip, decode.hip).
//
// A row of K weights is split over LPR lanes of a wavefront, each lane holding
// SPL interleaved pieces of 16 weights (see piece_k).  A Chunk holds the raw
// bits of one lane's pieces of one row; its dot_x / dot_a decode them in
// registers and multiply with the lane's activations:
//   dot_x: activations are bf16 pairs (token vectors x, gate/up input);
//   dot_a: activations are the SwiGLU output a in the per-format form ADown.
#pragma once
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kNCopy = 16;  // VQ2 codebook replicas in LDS, one bank pair each

// --------------------------------------------------------------------------
// wavefront reductions on DPP (no LDS round trip)
// --------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                             0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
// row of 16: quad xor 1, quad xor 2, half-row mirror, row mirror
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
// the same maximum / minimum in every lane, with VALU operations only: DPP
// within rows of 16, then the row-pair and half-wave swaps of gfx950
__device__ __forceinline__ int wave_max_all(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = max((int)r[0], (int)r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return max((int)q[0], (int)q[1]);
}
__device__ __forceinline__ int wave_min_all(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = min((int)r[0], (int)r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return min((int)q[0], (int)q[1]);
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// R per-row partial sums (R = 8 or 16) in every lane -> the R row totals,
// transposed: each step pairs lanes across one lane bit (the half-wave swap,
// the row-pair swap, then DPP inside rows of 16) and keeps half of the rows,
// so the R totals cost about 2R instructions instead of R full reductions.
// Lane l returns the total of row l / (64 / R).
template <int R>
__device__ __forceinline__ float rows_reduce(const float (&v)[R]) {
  static_assert(R == 8 || R == 16, "rows");
  const int lane = threadIdx.x & 63;
  float w[R / 2];
#pragma unroll
  for (int r = 0; r < R / 2; r++) {
    // lanes < 32 keep row r (both halves' sum), lanes >= 32 row r + R/2
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[r]),
                                                    __float_as_uint(v[r + R / 2]), false, false);
    w[r] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  float u[R / 4];
#pragma unroll
  for (int r = 0; r < R / 4; r++) {
    // even rows of 16 lanes keep w[r], odd ones w[r + R/4]
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[r]),
                                                    __float_as_uint(w[r + R / 4]), false, false);
    u[r] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  // lanes l and l ^ 8 (a rotation by 8 inside the row of 16)
  const bool b3 = lane & 8;
  float t[R / 8];
#pragma unroll
  for (int r = 0; r < R / 8; r++) {
    const float keep = b3 ? u[r + R / 8] : u[r], send = b3 ? u[r] : u[r + R / 8];
    t[r] = keep + dpp_f<0x128>(send);
  }
  float x;
  if constexpr (R == 16) {
    // lanes i and 7 - i of each half-row (the half-row mirror)
    const bool b2 = lane & 4;
    const float keep = b2 ? t[1] : t[0], send = b2 ? t[0] : t[1];
    x = keep + dpp_f<0x141>(send);
  } else {
    x = t[0] + dpp_f<0x141>(t[0]);
  }
  x += dpp_f<0xB1>(x);
  return x + dpp_f<0x4E>(x);
}

// sum over aligned groups of G lanes; G = 64 returns the full sum in all lanes
template <int G>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (G == 64) {
    return wave_sum_f(v);
  } else {
    return group_sum<G>(v);
  }
}

// --------------------------------------------------------------------------
// lane -> weight mapping
//
// A row of K weights is cut into K/16 "pieces" of 16 consecutive weights.
// The LPR lanes of a row group take pieces kl, kl + LPR, kl + 2 LPR, ...
// (kl = lane % LPR; SPL pieces each), so that the lanes of a wavefront read
// consecutive bytes of every format in each load instruction.
// --------------------------------------------------------------------------
template <int LPR>
__device__ __forceinline__ int piece_k(int kl, int i) {
  return 16 * (kl + LPR * i);
}

// Buffer resources: a wave-uniform base (SGPRs), a per-lane 32-bit offset that
// does not depend on the row, and a wave-uniform row offset (soffset).  Loads
// past num_records return 0.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufDword3 = 0x00020000;  // gfx9 raw buffer descriptor word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufDword3);
}
__device__ __forceinline__ uint32_t buf_u8(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ uint32_t buf_u16(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ u32x2_t buf_u64(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ u32x4_t buf_u128(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)so, 0);
}
// row offset as soffset when all lanes share the row (LPR == 64), else per lane
template <int LPR>
__device__ __forceinline__ void row_split(uint32_t row_off, uint32_t &vo, uint32_t &so) {
  if constexpr (LPR == 64) {
    so = __builtin_amdgcn_readfirstlane(row_off);
    vo = 0;
  } else {
    so = 0;
    vo = row_off;
  }
}

// split x into bf16 hi + bf16 lo (x - hi rounded), 16 significant bits together
__device__ __forceinline__ void split_bf16(float x, uint32_t &hi, uint32_t &lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// 16 floats at byte offset vo of an activation row
__device__ __forceinline__ void load_f32x16(__amdgpu_buffer_rsrc_t r, uint32_t vo, float *v) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const u32x4_t q = buf_u128(r, vo + 16 * i, 0);
    v[4 * i] = __uint_as_float(q.x), v[4 * i + 1] = __uint_as_float(q.y);
    v[4 * i + 2] = __uint_as_float(q.z), v[4 * i + 3] = __uint_as_float(q.w);
  }
}

// activations for the down projection: default fp32 values per piece
template <int FMT, int SPL, int LPR>
struct ADown {
  float v[SPL][16];
  __device__ __forceinline__ void load(const float *row, int kl) {
#pragma unroll
    for (int i = 0; i < SPL; i++) load_f32x16(make_rsrc(row, 0x7FFFFFFF), 4 * piece_k<LPR>(kl, i), v[i]);
  }
};

// Q2K: per piece (one sub-block), bf16 hi/lo pairs (a[p], a[p+8]) matching
// the code pairs one shift of a qs dword exposes, and the piece sum
template <int SPL, int LPR>
struct ADown<MOE_FMT_Q2K, SPL, LPR> {
  uint32_t hi[SPL][8], lo[SPL][8];
  float sum[SPL];
  __device__ __forceinline__ void load(const float *row, int kl) {
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float v[16];
      load_f32x16(make_rsrc(row, 0x7FFFFFFF), 4 * piece_k<LPR>(kl, i), v);
      float s = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; p++) {
        uint32_t h0, l0, h1, l1;
        split_bf16(v[p], h0, l0);
        split_bf16(v[p + 8], h1, l1);
        hi[i][p] = h0 | (h1 << 16);
        lo[i][p] = l0 | (l1 << 16);
        s += (bf16_bits_to_f32(h0) + bf16_bits_to_f32(l0)) +
             (bf16_bits_to_f32(h1) + bf16_bits_to_f32(l1));
      }
      sum[i] = s;
    }
  }
};

// BF16 weights: bf16 hi/lo pairs (a[2m], a[2m+1]) matching the weight dwords
template <int SPL, int LPR>
struct ADown<MOE_FMT_BF16, SPL, LPR> {
  uint32_t hi[SPL][8], lo[SPL][8];
  __device__ __forceinline__ void load(const float *row, int kl) {
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float v[16];
      load_f32x16(make_rsrc(row, 0x7FFFFFFF), 4 * piece_k<LPR>(kl, i), v);
#pragma unroll
      for (int m = 0; m < 8; m++) {
        uint32_t h0, l0, h1, l1;
        split_bf16(v[2 * m], h0, l0);
        split_bf16(v[2 * m + 1], h1, l1);
        hi[i][m] = h0 | (h1 << 16);
        lo[i][m] = l0 | (l1 << 16);
      }
    }
  }
  // activations already split into bf16 hi/lo arrays in natural order
  __device__ __forceinline__ void load_split(const uint16_t *hi_row, const uint16_t *lo_row,
                                             int kl) {
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(hi_row, 0x7FFFFFFF);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lo_row, 0x7FFFFFFF);
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const uint32_t vo = 2u * (uint32_t)piece_k<LPR>(kl, i);
      const u32x4_t h0 = buf_u128(rh, vo, 0), h1 = buf_u128(rh, vo + 16, 0);
      const u32x4_t l0 = buf_u128(rl, vo, 0), l1 = buf_u128(rl, vo + 16, 0);
      hi[i][0] = h0.x, hi[i][1] = h0.y, hi[i][2] = h0.z, hi[i][3] = h0.w;
      hi[i][4] = h1.x, hi[i][5] = h1.y, hi[i][6] = h1.z, hi[i][7] = h1.w;
      lo[i][0] = l0.x, lo[i][1] = l0.y, lo[i][2] = l0.z, lo[i][3] = l0.w;
      lo[i][4] = l1.x, lo[i][5] = l1.y, lo[i][6] = l1.z, lo[i][7] = l1.w;
    }
  }
};

// How a gate/up kernel stores the SwiGLU output a for the down kernel:
// kAF32: fp32; kASplit: bf16 hi/lo arrays in natural order (bf16 down);
// kAF16Q2K: fp16 (one array), each 16-value piece in the order of
// ADownQ2K16's pairs; kAF16: fp16 in natural order (MXFP4 down).
constexpr int kAF32 = 0, kASplit = 1, kAF16Q2K = 3, kAF16 = 4;
// value 4b + r of a piece sits at 4b + 2(r & 1) + (r >> 1): the pairs are
// (a[4b], a[4b+2]) and (a[4b+1], a[4b+3])
__device__ __forceinline__ int q2k16_pos(int i) {
  return (i & ~3) | ((i & 1) << 1) | ((i >> 1) & 1);
}

// fp16 activations in natural order: per piece the pairs (a[2m], a[2m+1])
template <int SPL, int LPR>
struct ADownF16 {
  uint32_t h[SPL][8];
  __device__ __forceinline__ void load(const uint16_t *row, int kl) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(row, 0x7FFFFFFF);
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const uint32_t vo = 2u * (uint32_t)piece_k<LPR>(kl, i);
      const u32x4_t a0 = buf_u128(r, vo, 0), a1 = buf_u128(r, vo + 16, 0);
      h[i][0] = a0.x, h[i][1] = a0.y, h[i][2] = a0.z, h[i][3] = a0.w;
      h[i][4] = a1.x, h[i][5] = a1.y, h[i][6] = a1.z, h[i][7] = a1.w;
    }
  }
};

// the two 2-bit codes held as E2M1 nibbles in byte b of w, as an exact fp16
// pair (E2M1 codes 0..3 are 0, 0.5, 1, 1.5; the scale 2 makes them 0..3)
__device__ __forceinline__ uint32_t q2_pair(uint32_t w, int b) {
  switch (b) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 3));
  }
}

// Q2K down against fp16 activations: per piece the 8 pairs in q2k16_pos
// order and the piece's sum (fp32)
template <int SPL, int LPR>
struct ADownQ2K16 {
  uint32_t h[SPL][8];
  float sum[SPL];
  __device__ __forceinline__ void load(const uint16_t *row, int kl) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(row, 0x7FFFFFFF);
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const uint32_t vo = 2u * (uint32_t)piece_k<LPR>(kl, i);
      const u32x4_t a0 = buf_u128(r, vo, 0), a1 = buf_u128(r, vo + 16, 0);
      h[i][0] = a0.x, h[i][1] = a0.y, h[i][2] = a0.z, h[i][3] = a0.w;
      h[i][4] = a1.x, h[i][5] = a1.y, h[i][6] = a1.z, h[i][7] = a1.w;
    }
  }
  // the piece sums, once the pairs are in
  __device__ __forceinline__ void sums() {
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float s = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; m++) s = dot2_f16(h[i][m], 0x3C003C00u, s);
      sum[i] = s;
    }
  }
};

// bf16 pairs of token `tok`'s pieces
template <int SPL, int LPR>
__device__ __forceinline__ void load_x_pieces(const uint16_t *x, int K, int tok, int kl,
                                              uint32_t (&xw)[SPL][8]) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(x, 0x7FFFFFFF);
  const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)tok * (uint32_t)K * 2u);
#pragma unroll
  for (int i = 0; i < SPL; i++) {
    const uint32_t vo = 2u * (uint32_t)piece_k<LPR>(kl, i);
    const u32x4_t q0 = buf_u128(r, vo, so), q1 = buf_u128(r, vo + 16, so);
    xw[i][0] = q0.x, xw[i][1] = q0.y, xw[i][2] = q0.z, xw[i][3] = q0.w;
    xw[i][4] = q1.x, xw[i][5] = q1.y, xw[i][6] = q1.z, xw[i][7] = q1.w;
  }
}

// --------------------------------------------------------------------------
// per-format lane chunks: SPL pieces of one row
// --------------------------------------------------------------------------

template <int FMT, int SPL, int LPR>
struct Chunk;

// VQ2: one code dword (4 codes = 16 weights) per piece + the piece's fp16 scale
template <int SPL, int LPR>
struct Chunk<MOE_FMT_VQ2, SPL, LPR> {
  uint32_t code[SPL];
  uint32_t d[SPL];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int kl) {
    const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_VQ2, w.N, w.K);
    const uint32_t sb = (uint32_t)expert_scale_bytes(MOE_FMT_VQ2, w.N, w.K);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(w.data + (size_t)e * db, db);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
    uint32_t vd, sd, vs, ss;
    row_split<LPR>((uint32_t)row * (uint32_t)(w.K / 4), vd, sd);
    row_split<LPR>((uint32_t)row * (uint32_t)(w.K / 128), vs, ss);
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const uint32_t k = (uint32_t)piece_k<LPR>(kl, i);
      code[i] = buf_u32(rd, vd + k / 4, sd);
      d[i] = buf_u16(rs, vs + (k / 256) * 2, ss);
    }
  }
  // cb: this lane's codebook copy in LDS (entry e at cb[e * NC], NC copies);
  // with NC == 32 the table itself (entry e, copy c at byte 256 e + 8 c) and
  // each lane reads copy lane % 32: the byte offset of code byte b is then
  // (byte << 8) | 8 (lane % 32), which one v_perm_b32 assembles (byte 1 from
  // the code word, byte 0 from the lane's copy offset, zeros above)
  template <int NT, int NC = kNCopy>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][SPL][8], const uint2 *cb,
                                        float (&out)[NT]) const {
    const uint32_t lane_off = (threadIdx.x & 31u) << 3;
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        uint2 c;
        if constexpr (NC == 32) {
          const uint32_t off =
              __builtin_amdgcn_perm(code[i], lane_off, 0x0C0C0000u | ((4u + b) << 8));
          c = *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(cb) + off);
        } else {
          c = cb[((code[i] >> (8 * b)) & 255u) * NC];
        }
#pragma unroll
        for (int t = 0; t < NT; t++) {
          acc[t] = dot2_bf16(xw[t][i][2 * b], c.x, acc[t]);
          acc[t] = dot2_bf16(xw[t][i][2 * b + 1], c.y, acc[t]);
        }
      }
      const float df = f16_bits_to_f32(d[i]);
#pragma unroll
      for (int t = 0; t < NT; t++) out[t] = fmaf(df, acc[t], out[t]);
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const ADown<MOE_FMT_VQ2, SPL, LPR> (&a)[NT],
                                        const uint2 *cb, float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const uint2 c = cb[((code[i] >> (8 * b)) & 255u) * kNCopy];
        const float c0 = bf16_lo(c.x), c1 = bf16_hi(c.x), c2 = bf16_lo(c.y), c3 = bf16_hi(c.y);
#pragma unroll
        for (int t = 0; t < NT; t++) {
          const float *v = &a[t].v[i][4 * b];
          acc[t] = fmaf(v[0], c0, acc[t]);
          acc[t] = fmaf(v[1], c1, acc[t]);
          acc[t] = fmaf(v[2], c2, acc[t]);
          acc[t] = fmaf(v[3], c3, acc[t]);
        }
      }
      const float df = f16_bits_to_f32(d[i]);
#pragma unroll
      for (int t = 0; t < NT; t++) out[t] = fmaf(df, acc[t], out[t]);
    }
  }
};

// Q2K: one sub-block per piece -- its qs dword, scale/min byte and the
// block's d/dmin dword
template <int SPL, int LPR>
struct Chunk<MOE_FMT_Q2K, SPL, LPR> {
  uint32_t qs[SPL];
  uint32_t sc[SPL];
  uint32_t dm[SPL];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int kl) {
    const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_Q2K, w.N, w.K);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(w.data + (size_t)e * db, db);
    if constexpr (LPR == 64) {
      // K % 1024 == 0: whole blocks per row; per-lane block/sub-block offsets
      // do not depend on the row
      const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)row * (uint32_t)(w.K / 256) *
                                                         (uint32_t)kQ2KBytes);
#pragma unroll
      for (int i = 0; i < SPL; i++) {
        const uint32_t p = (uint32_t)(kl + 64 * i);
        const uint32_t boff = (p / 16) * kQ2KBytes, j = p % 16;
        qs[i] = buf_u32(rd, boff + 16 + 4 * j, so);
        sc[i] = buf_u8(rd, boff + j, so);
        dm[i] = buf_u32(rd, boff + 80, so);
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPL; i++) {
        const uint32_t f = (uint32_t)row * (uint32_t)w.K + (uint32_t)piece_k<LPR>(kl, i);
        const uint32_t boff = (f / 256) * kQ2KBytes, j = (f % 256) / 16;
        qs[i] = buf_u32(rd, boff + 16 + 4 * j, 0);
        sc[i] = buf_u8(rd, boff + j, 0);
        dm[i] = buf_u32(rd, boff + 80, 0);
      }
    }
  }
  // sum x_i w_i = d*scale*sum(x q) - dmin*min*sum(x), per sub-block
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][SPL][8], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const float d = f16_bits_to_f32(dm[i] & 0xFFFFu), dmin = f16_bits_to_f32(dm[i] >> 16);
      const float ds = d * (float)(sc[i] & 15u), ms = dmin * (float)(sc[i] >> 4);
#pragma unroll
      for (int t = 0; t < NT; t++) {
        float sxq = 0.0f, sx = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; p++) {
          const uint32_t wx = xw[t][i][p / 2];
          const float xv = (p & 1) ? bf16_hi(wx) : bf16_lo(wx);
          sxq = fmaf(xv, (float)((qs[i] >> (2 * p)) & 3u), sxq);
          sx += xv;
        }
        out[t] = fmaf(ds, sxq, fmaf(-ms, sx, out[t]));
      }
    }
  }
  // against fp16 activations: each code widened to an E2M1 nibble (q reads
  // as q/2) and converted with the scale 2, so the pairs hold q exactly;
  // then d sc sum(a q) - dmin m sum(a) per sub-block
  __device__ __forceinline__ float dot_a16(const ADownQ2K16<SPL, LPR> &a) const {
    float out = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      // (d sc, dmin m) as one fp16 pair: the two nibbles as 1024 + n (exact
      // in fp16), minus 1024, times (d, dmin), rounded once each to fp16
      const uint32_t nib = (((sc[i] << 12) | sc[i]) & 0x000F000Fu) | 0x64006400u;
      const f16x2_dev_t sm = (__builtin_bit_cast(f16x2_dev_t, nib) - (_Float16)1024.0f) *
                             __builtin_bit_cast(f16x2_dev_t, dm[i]);
      const float ds = (float)sm[0], ms = (float)sm[1];
      const uint32_t nl = qs[i] & 0x33333333u, nh = (qs[i] >> 2) & 0x33333333u;
      float acc = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        acc = dot2_f16(a.h[i][2 * b], q2_pair(nl, b), acc);
        acc = dot2_f16(a.h[i][2 * b + 1], q2_pair(nh, b), acc);
      }
      out = fmaf(ds, acc, fmaf(-ms, a.sum[i], out));
    }
    return out;
  }
  // codes as bf16 pairs (128 + q_p, 128 + q_{p+8}) against the activation
  // pairs: sum a*(128+q) - 128*sum(a) = sum a*q
  template <int NT>
  __device__ __forceinline__ void dot_a(const ADown<MOE_FMT_Q2K, SPL, LPR> (&a)[NT],
                                        const uint2 *, float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const float d = f16_bits_to_f32(dm[i] & 0xFFFFu), dmin = f16_bits_to_f32(dm[i] >> 16);
      const float ds = d * (float)(sc[i] & 15u), ms = dmin * (float)(sc[i] >> 4);
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; p++) {
        const uint32_t qp = ((qs[i] >> (2 * p)) & 0x00030003u) | 0x43004300u;
#pragma unroll
        for (int t = 0; t < NT; t++) {
          acc[t] = dot2_bf16(a[t].hi[i][p], qp, acc[t]);
          acc[t] = dot2_bf16(a[t].lo[i][p], qp, acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; t++) {
        const float sxq = fmaf(-128.0f, a[t].sum[i], acc[t]);
        out[t] = fmaf(ds, sxq, fmaf(-ms, a[t].sum[i], out[t]));
      }
    }
  }
};

// MXFP4: 8 bytes of nibbles per piece and its E8M0 scale (one per 32 weights)
template <int SPL, int LPR>
struct Chunk<MOE_FMT_MXFP4, SPL, LPR> {
  uint32_t v[SPL][2];
  uint32_t sc[SPL];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int kl) {
    const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_MXFP4, w.N, w.K);
    const uint32_t sb = (uint32_t)expert_scale_bytes(MOE_FMT_MXFP4, w.N, w.K);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(w.data + (size_t)e * db, db);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
    uint32_t vd, sd, vs, ss;
    row_split<LPR>((uint32_t)row * (uint32_t)(w.K / 2), vd, sd);
    row_split<LPR>((uint32_t)row * (uint32_t)(w.K / 32), vs, ss);
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const uint32_t k = (uint32_t)piece_k<LPR>(kl, i);
      const u32x2_t q = buf_u64(rd, vd + k / 2, sd);
      v[i][0] = q.x, v[i][1] = q.y;
      sc[i] = buf_u8(rs, vs + k / 32, ss);
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][SPL][8], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint32_t p0 = e2m1x2_to_bf16x2<0>(v[i][j]), p1 = e2m1x2_to_bf16x2<1>(v[i][j]);
        const uint32_t p2 = e2m1x2_to_bf16x2<2>(v[i][j]), p3 = e2m1x2_to_bf16x2<3>(v[i][j]);
#pragma unroll
        for (int t = 0; t < NT; t++) {
          acc[t] = dot2_bf16(xw[t][i][4 * j + 0], p0, acc[t]);
          acc[t] = dot2_bf16(xw[t][i][4 * j + 1], p1, acc[t]);
          acc[t] = dot2_bf16(xw[t][i][4 * j + 2], p2, acc[t]);
          acc[t] = dot2_bf16(xw[t][i][4 * j + 3], p3, acc[t]);
        }
      }
      const float s = e8m0_to_f32(sc[i]);
#pragma unroll
      for (int t = 0; t < NT; t++) out[t] = fmaf(acc[t], s, out[t]);
    }
  }
  // against fp16 activations: the E2M1 pairs converted exactly to fp16 (scale
  // 1), one v_dot2_f32_f16 per pair, the block scale once per 32 weights
  __device__ __forceinline__ float dot_a16(const ADownF16<SPL, LPR> &a) const {
    float out = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        acc = dot2_f16(a.h[i][4 * j + 0], e2m1x2_to_f16x2<0>(v[i][j]), acc);
        acc = dot2_f16(a.h[i][4 * j + 1], e2m1x2_to_f16x2<1>(v[i][j]), acc);
        acc = dot2_f16(a.h[i][4 * j + 2], e2m1x2_to_f16x2<2>(v[i][j]), acc);
        acc = dot2_f16(a.h[i][4 * j + 3], e2m1x2_to_f16x2<3>(v[i][j]), acc);
      }
      out = fmaf(acc, e8m0_to_f32(sc[i]), out);
    }
    return out;
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const ADown<MOE_FMT_MXFP4, SPL, LPR> (&a)[NT],
                                        const uint2 *, float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint32_t p[4] = {e2m1x2_to_bf16x2<0>(v[i][j]), e2m1x2_to_bf16x2<1>(v[i][j]),
                               e2m1x2_to_bf16x2<2>(v[i][j]), e2m1x2_to_bf16x2<3>(v[i][j])};
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            acc[t] = fmaf(a[t].v[i][8 * j + 2 * q], bf16_lo(p[q]), acc[t]);
            acc[t] = fmaf(a[t].v[i][8 * j + 2 * q + 1], bf16_hi(p[q]), acc[t]);
          }
      }
      const float s = e8m0_to_f32(sc[i]);
#pragma unroll
      for (int t = 0; t < NT; t++) out[t] = fmaf(acc[t], s, out[t]);
    }
  }
};

// BF16 weights: 32 bytes (8 dwords) per piece
template <int SPL, int LPR>
struct Chunk<MOE_FMT_BF16, SPL, LPR> {
  uint32_t v[SPL][8];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int kl) {
    const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_BF16, w.N, w.K);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(w.data + (size_t)e * db, db);
    uint32_t vd, sd;
    row_split<LPR>((uint32_t)row * (uint32_t)w.K * 2u, vd, sd);
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const uint32_t vo = vd + 2u * (uint32_t)piece_k<LPR>(kl, i);
      const u32x4_t q0 = buf_u128(rd, vo, sd), q1 = buf_u128(rd, vo + 16, sd);
      v[i][0] = q0.x, v[i][1] = q0.y, v[i][2] = q0.z, v[i][3] = q0.w;
      v[i][4] = q1.x, v[i][5] = q1.y, v[i][6] = q1.z, v[i][7] = q1.w;
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][SPL][8], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; i++)
#pragma unroll
        for (int m = 0; m < 8; m++) acc = dot2_bf16(xw[t][i][m], v[i][m], acc);
      out[t] = acc;
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const ADown<MOE_FMT_BF16, SPL, LPR> (&a)[NT],
                                        const uint2 *, float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; i++)
#pragma unroll
        for (int m = 0; m < 8; m++) {
          acc = dot2_bf16(a[t].hi[i][m], v[i][m], acc);
          acc = dot2_bf16(a[t].lo[i][m], v[i][m], acc);
        }
      out[t] = acc;
    }
  }
};

// --------------------------------------------------------------------------
// shared helpers
// --------------------------------------------------------------------------

// VQ2 codebook -> LDS as bf16x4 entries, kNCopy interleaved copies so copy c
// of every entry sits in the same two banks; one entry per thread
__device__ __forceinline__ void fill_codebook(const int8_t *cb, uint2 *s_cb) {
  for (int e = threadIdx.x; e < 256; e += blockDim.x) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(cb)[e];
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; j++) b[j] = f32_to_bf16_bits((float)(int)(int8_t)((w >> (8 * j)) & 255u));
    const uint2 v = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
#pragma unroll
    for (int j = 0; j < kNCopy; j++) s_cb[e * kNCopy + ((j + e) & (kNCopy - 1))] = v;
  }
}

// the same fill in two steps, so that the load can be issued early: thread t
// loads entry t % 256 and later (codebook_entry_store_all) writes every copy
// of it
__device__ __forceinline__ uint32_t codebook_entry_load(const int8_t *cb) {
  return reinterpret_cast<const uint32_t *>(cb)[threadIdx.x & 255];
}
// entry threadIdx.x % 256, every one of NC copies (for 256 of the block's threads)
template <int NC = kNCopy>
__device__ __forceinline__ void codebook_entry_store_all(uint32_t w, uint2 *s_cb) {
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; j++) b[j] = f32_to_bf16_bits((float)(int)(int8_t)((w >> (8 * j)) & 255u));
  const uint2 v = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
  const int e = threadIdx.x & 255;
  // lanes write different copies in each step (consecutive entries are 128
  // bytes apart: the same copy for all lanes would hit one bank pair)
#pragma unroll
  for (int j = 0; j < NC; j++) s_cb[e * NC + ((j + threadIdx.x) & (NC - 1))] = v;
}

// rows per wave step so the raw bits in flight stay near 32 dwords per lane
// per projection (more rows for small chunks, fewer for bf16)
template <int FMT, int SPL>
constexpr int steps_for() {
  constexpr int dw = FMT == MOE_FMT_BF16 ? 8 * SPL : FMT == MOE_FMT_VQ2 ? 2 * SPL : 3 * SPL;
  return dw >= 32 ? 1 : dw >= 16 ? 2 : 4;
}

// lane geometry for a row length K
__host__ __device__ inline bool gemv_geometry(int K, int *spl, int *lpr) {
  if (K >= 1024 && K % 1024 == 0) {
    const int s = K / 1024;
    if (s == 1 || s == 2 || s == 4 || s == 8) {
      *spl = s;
      *lpr = 64;
      return true;
    }
    return false;  // other multiples: not instantiated
  }
  if (K == 512 || K == 256 || K == 128) {
    *spl = 1;
    *lpr = K / 16;
    return true;
  }
  return false;
}

// --------------------------------------------------------------------------
// row bodies: one wave, STEPS * (64/LPR) rows
// --------------------------------------------------------------------------

// a[r][row] = silu(gate_e[row] . x_t) * (up_e[row] . x_t) for bucket rows
// r in [r0, r1), token of row r = row_token[r] (or tok_fixed >= 0, or r)
template <int FMT, int SPL, int LPR, int STEPS, int NT, int PF = 2, int NC = kNCopy>
__device__ __forceinline__ void gateup_rows(const WView &gate, const WView &up, int H, int I,
                                            const uint16_t *x, int e, int r0, int r1,
                                            const int32_t *row_token, int tok_fixed, float *a,
                                            int row_base, const uint2 *cb, int am = kAF32,
                                            uint16_t *a_hi = nullptr, uint16_t *a_lo = nullptr) {
  constexpr int RPS = 64 / LPR;
  constexpr int D = PF < STEPS ? PF : STEPS;  // rows whose loads are in flight
  const int lane = threadIdx.x & 63;
  const int kl = lane % LPR;
  for (int rb = r0; rb < r1; rb += NT) {
    // keep the weight loads inside the token loop: hoisting them would hold
    // every row's bits in registers across iterations
    asm volatile("" ::: "memory");
    const int nt = min(NT, r1 - rb);
    Chunk<FMT, SPL, LPR> cg[D], cu[D];
#pragma unroll
    for (int s = 0; s < D; s++) {
      const int row = min(row_base + s * RPS, I - 1);
      cg[s].load(gate, e, row, kl);
      cu[s].load(up, e, row, kl);
    }
    uint32_t xw[NT][SPL][8];
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int r = rb + (t < nt ? t : 0);
      // every lane of the wave handles the same bucket rows: the token is uniform
      const int tok = __builtin_amdgcn_readfirstlane(
          tok_fixed >= 0 ? tok_fixed : (row_token ? row_token[r] : r));
      load_x_pieces<SPL, LPR>(x, H, tok, kl, xw[t]);
    }
    auto store = [&](int r, int row, float v) {
      if (am == kAF32) {
        a[(size_t)r * I + row] = v;
      } else if (am == kAF16Q2K || am == kAF16) {
        a_hi[(size_t)r * I + (am == kAF16Q2K ? q2k16_pos(row) : row)] =
            __builtin_bit_cast(uint16_t, (_Float16)v);
      } else {
        uint32_t h, l;
        split_bf16(v, h, l);
        const size_t pos = (size_t)r * I + row;
        a_hi[pos] = (uint16_t)h;
        a_lo[pos] = (uint16_t)l;
      }
    };
    // one token and four row pairs per wave, all loaded at once: the eight
    // sums are reduced together at the end (rows_reduce) instead of one full
    // reduction each
    constexpr bool kT = LPR == 64 && NT == 1 && STEPS == 4 && D == STEPS;
    float gs[kT ? STEPS : 1], us[kT ? STEPS : 1];
#pragma unroll
    for (int s = 0; s < STEPS; s++) {
      const int row = row_base + s * RPS;
      float g[NT], u[NT];
      if constexpr (FMT == MOE_FMT_VQ2) {
        cg[s % D].template dot_x<NT, NC>(xw, cb, g);
        cu[s % D].template dot_x<NT, NC>(xw, cb, u);
      } else {
        cg[s % D].template dot_x<NT>(xw, cb, g);
        cu[s % D].template dot_x<NT>(xw, cb, u);
      }
      if (s + D < STEPS) {  // refill this slot with the row D steps ahead
        const int nrow = min(row_base + (s + D) * RPS, I - 1);
        cg[s % D].load(gate, e, nrow, kl);
        cu[s % D].load(up, e, nrow, kl);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the pipeline depth: no hoisting of later loads
      if constexpr (kT) {
        gs[s] = g[0];
        us[s] = u[0];
      } else {
#pragma unroll
        for (int t = 0; t < NT; t++) {
          g[t] = lane_group_sum<LPR>(g[t]);
          u[t] = lane_group_sum<LPR>(u[t]);
        }
        if (kl == 0 && row < I) {
#pragma unroll
          for (int t = 0; t < NT; t++)
            if (t < nt) store(rb + t, row, silu_mul(g[t], u[t]));
        }
      }
    }
    if constexpr (kT) {
      const float vals[8] = {gs[0], gs[1], gs[2], gs[3], us[0], us[1], us[2], us[3]};
      // lane l: the total of value l / 8 (gate of step l / 8 below lane 32,
      // up above); the half-wave swap brings each up total next to its gate
      const float x = rows_reduce<8>(vals);
      const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                      false);
      const int row = row_base + (lane >> 3) * RPS;
      if (lane < 32 && (lane & 7) == 0 && row < I)
        store(rb, row, silu_mul(__uint_as_float(q[0]), __uint_as_float(q[1])));
    }
  }
}

// y[r][row] = down_e[row] . a[r] for bucket rows r in [r0, r1)
template <int FMT, int SPL, int LPR, int STEPS, int NT, int PF = 2>
__device__ __forceinline__ void down_rows(const WView &down, int H, int I, const float *a, int e,
                                          int r0, int r1, float *y, int row_base,
                                          const uint2 *cb) {
  constexpr int RPS = 64 / LPR;
  constexpr int D = PF < STEPS ? PF : STEPS;
  const int lane = threadIdx.x & 63;
  const int kl = lane % LPR;
  for (int rb = r0; rb < r1; rb += NT) {
    asm volatile("" ::: "memory");
    const int nt = min(NT, r1 - rb);
    Chunk<FMT, SPL, LPR> c[D];
#pragma unroll
    for (int s = 0; s < D; s++) c[s].load(down, e, min(row_base + s * RPS, H - 1), kl);
    ADown<FMT, SPL, LPR> av[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) av[t].load(a + (size_t)(rb + (t < nt ? t : 0)) * I, kl);
#pragma unroll
    for (int s = 0; s < STEPS; s++) {
      const int row = row_base + s * RPS;
      float yv[NT];
      c[s % D].template dot_a<NT>(av, cb, yv);
      if (s + D < STEPS) c[s % D].load(down, e, min(row_base + (s + D) * RPS, H - 1), kl);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NT; t++) yv[t] = lane_group_sum<LPR>(yv[t]);
      if (kl == 0 && row < H) {
#pragma unroll
        for (int t = 0; t < NT; t++)
          if (t < nt) y[(size_t)(rb + t) * H + row] = yv[t];
      }
    }
  }
}

}  // namespace moe
