// gemv.hip -- decode path: dequant-fused GEMVs over the experts' weights.
//
// Decode reads every selected expert's weights once per token batch, so it
// is bound by HBM bandwidth (the ds4 pages: routed experts dominate the
// model's size and generation pays for fetching them -- hysenlabs.com, "SSD
// streaming"; baiwuji.top, "SSD streaming").  The kernels stream the
// quantized bytes once, decode them in registers and reduce with wavefront
// shuffles; there is no matrix-core work here.
//
// Lane geometry: a row of K weights is split over LPR lanes, each holding a
// contiguous chunk of 16*SPL weights (SPL "sub-blocks" of 16).  For K >= 1024
// LPR = 64 (one row per wave step); smaller K packs 64/LPR rows per step.
// The activations of the lane's chunk stay in registers across all the rows a
// wave processes.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kNCopy = 16;  // replicas of the VQ2 codebook in LDS, one bank pair each

// --------------------------------------------------------------------------
// per-format lane chunks: raw bits of 16*SPL consecutive weights of one row
// --------------------------------------------------------------------------

template <int FMT, int SPL>
struct Chunk;

// VQ2: 4*SPL code bytes + one fp16 scale (16*SPL <= 256, so one group)
template <int SPL>
struct Chunk<MOE_FMT_VQ2, SPL> {
  uint32_t code[SPL];
  uint32_t d;
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k0) {
    const uint8_t *base = w.data + (size_t)e * expert_data_bytes(MOE_FMT_VQ2, w.N, w.K) +
                          (size_t)row * (w.K / 4) + k0 / 4;
    if constexpr (SPL % 4 == 0) {
#pragma unroll
      for (int i = 0; i < SPL; i += 4) {
        const uint4 v = reinterpret_cast<const uint4 *>(base)[i / 4];
        code[i] = v.x, code[i + 1] = v.y, code[i + 2] = v.z, code[i + 3] = v.w;
      }
    } else if constexpr (SPL % 2 == 0) {
#pragma unroll
      for (int i = 0; i < SPL; i += 2) {
        const uint2 v = reinterpret_cast<const uint2 *>(base)[i / 2];
        code[i] = v.x, code[i + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPL; i++) code[i] = reinterpret_cast<const uint32_t *>(base)[i];
    }
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(
        w.scales + (size_t)e * expert_scale_bytes(MOE_FMT_VQ2, w.N, w.K));
    d = sc[(size_t)row * (w.K / 256) + k0 / 256];
  }
  // x: bf16 pairs of the chunk; cb: LDS codebook (bf16x4 per entry, kNCopy copies)
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][8 * SPL], const uint2 *cb,
                                        float (&out)[NT]) const {
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++)
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const uint2 c = cb[((code[i] >> (8 * b)) & 255u) * kNCopy];
#pragma unroll
        for (int t = 0; t < NT; t++) {
          acc[t] = dot2_bf16(xw[t][8 * i + 2 * b], c.x, acc[t]);
          acc[t] = dot2_bf16(xw[t][8 * i + 2 * b + 1], c.y, acc[t]);
        }
      }
    const float df = f16_bits_to_f32(d);
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = df * acc[t];
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const float (&af)[NT][16 * SPL],
                                        const float (&as)[NT][SPL], const uint2 *cb,
                                        float (&out)[NT]) const {
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++)
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const uint2 c = cb[((code[i] >> (8 * b)) & 255u) * kNCopy];
        const float c0 = bf16_lo(c.x), c1 = bf16_hi(c.x), c2 = bf16_lo(c.y), c3 = bf16_hi(c.y);
#pragma unroll
        for (int t = 0; t < NT; t++) {
          const float *a = &af[t][16 * i + 4 * b];
          acc[t] = fmaf(a[0], c0, acc[t]);
          acc[t] = fmaf(a[1], c1, acc[t]);
          acc[t] = fmaf(a[2], c2, acc[t]);
          acc[t] = fmaf(a[3], c3, acc[t]);
        }
      }
    const float df = f16_bits_to_f32(d);
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = df * acc[t];
  }
};

// Q2K: SPL sub-blocks inside one 84-byte super-block
template <int SPL>
struct Chunk<MOE_FMT_Q2K, SPL> {
  uint32_t qs[SPL];
  uint32_t sc[SPL];
  uint32_t dm;
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k0) {
    const size_t f = (size_t)row * w.K + k0;
    const uint8_t *blk = w.data + (size_t)e * expert_data_bytes(MOE_FMT_Q2K, w.N, w.K) +
                         (f / 256) * kQ2KBytes;
    const int s0 = (int)(f % 256) / 16;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      qs[i] = reinterpret_cast<const uint32_t *>(blk + 16)[s0 + i];
      sc[i] = blk[s0 + i];
    }
    dm = reinterpret_cast<const uint32_t *>(blk)[20];
  }
  // sum_i x_i w_i = d*scale*sum(x q) - dmin*min*sum(x) per sub-block
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][8 * SPL], const uint2 *,
                                        float (&out)[NT]) const {
    const float d = f16_bits_to_f32(dm & 0xFFFFu), dmin = f16_bits_to_f32(dm >> 16);
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const float ds = d * (float)(sc[i] & 15u), ms = dmin * (float)(sc[i] >> 4);
#pragma unroll
      for (int t = 0; t < NT; t++) {
        float sxq = 0.0f, sx = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; p++) {
          const uint32_t wx = xw[t][8 * i + p / 2];
          const float xv = (p & 1) ? bf16_hi(wx) : bf16_lo(wx);
          sxq = fmaf(xv, (float)((qs[i] >> (2 * p)) & 3u), sxq);
          sx += xv;
        }
        out[t] = fmaf(ds, sxq, fmaf(-ms, sx, out[t]));
      }
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const float (&af)[NT][16 * SPL],
                                        const float (&as)[NT][SPL], const uint2 *,
                                        float (&out)[NT]) const {
    const float d = f16_bits_to_f32(dm & 0xFFFFu), dmin = f16_bits_to_f32(dm >> 16);
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      const float ds = d * (float)(sc[i] & 15u), ms = dmin * (float)(sc[i] >> 4);
#pragma unroll
      for (int t = 0; t < NT; t++) {
        float sxq = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; p++)
          sxq = fmaf(af[t][16 * i + p], (float)((qs[i] >> (2 * p)) & 3u), sxq);
        out[t] = fmaf(ds, sxq, fmaf(-ms, as[t][i], out[t]));
      }
    }
  }
};

// MXFP4: 8*SPL bytes of nibbles; one E8M0 scale per 32 weights
template <int SPL>
struct Chunk<MOE_FMT_MXFP4, SPL> {
  uint32_t v[2 * SPL];
  uint32_t sc;  // scale bytes, packed (SPL <= 8: at most 4 groups)
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k0) {
    const uint8_t *base = w.data + (size_t)e * expert_data_bytes(MOE_FMT_MXFP4, w.N, w.K) +
                          (size_t)row * (w.K / 2) + k0 / 2;
    if constexpr (SPL % 2 == 0) {
#pragma unroll
      for (int i = 0; i < 2 * SPL; i += 4) {
        const uint4 q = reinterpret_cast<const uint4 *>(base)[i / 4];
        v[i] = q.x, v[i + 1] = q.y, v[i + 2] = q.z, v[i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2 * SPL; i += 2) {
        const uint2 q = reinterpret_cast<const uint2 *>(base)[i / 2];
        v[i] = q.x, v[i + 1] = q.y;
      }
    }
    const uint8_t *s = w.scales + (size_t)e * expert_scale_bytes(MOE_FMT_MXFP4, w.N, w.K) +
                       (size_t)row * (w.K / 32) + k0 / 32;
    constexpr int NG = (SPL + 1) / 2;
    sc = 0;
#pragma unroll
    for (int g = 0; g < NG; g++) sc |= (uint32_t)s[g] << (8 * g);
  }
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][8 * SPL], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
    // dword j holds weights 8j..8j+7; 4 dwords per 32-weight group
#pragma unroll
    for (int g = 0; g < (2 * SPL + 3) / 4; g++) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 4 && 4 * g + jj < 2 * SPL; jj++) {
        const int j = 4 * g + jj;
        const uint32_t p0 = e2m1x2_to_bf16x2<0>(v[j]), p1 = e2m1x2_to_bf16x2<1>(v[j]);
        const uint32_t p2 = e2m1x2_to_bf16x2<2>(v[j]), p3 = e2m1x2_to_bf16x2<3>(v[j]);
#pragma unroll
        for (int t = 0; t < NT; t++) {
          acc[t] = dot2_bf16(xw[t][4 * j + 0], p0, acc[t]);
          acc[t] = dot2_bf16(xw[t][4 * j + 1], p1, acc[t]);
          acc[t] = dot2_bf16(xw[t][4 * j + 2], p2, acc[t]);
          acc[t] = dot2_bf16(xw[t][4 * j + 3], p3, acc[t]);
        }
      }
      const float s = e8m0_to_f32((sc >> (8 * g)) & 255u);
#pragma unroll
      for (int t = 0; t < NT; t++) out[t] = fmaf(acc[t], s, out[t]);
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const float (&af)[NT][16 * SPL],
                                        const float (&as)[NT][SPL], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) out[t] = 0.0f;
#pragma unroll
    for (int g = 0; g < (2 * SPL + 3) / 4; g++) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 4 && 4 * g + jj < 2 * SPL; jj++) {
        const int j = 4 * g + jj;
        uint32_t p[4] = {e2m1x2_to_bf16x2<0>(v[j]), e2m1x2_to_bf16x2<1>(v[j]),
                         e2m1x2_to_bf16x2<2>(v[j]), e2m1x2_to_bf16x2<3>(v[j])};
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            acc[t] = fmaf(af[t][8 * j + 2 * q], bf16_lo(p[q]), acc[t]);
            acc[t] = fmaf(af[t][8 * j + 2 * q + 1], bf16_hi(p[q]), acc[t]);
          }
      }
      const float s = e8m0_to_f32((sc >> (8 * g)) & 255u);
#pragma unroll
      for (int t = 0; t < NT; t++) out[t] = fmaf(acc[t], s, out[t]);
    }
  }
};

// BF16 weights: 16*SPL values = 8*SPL dwords
template <int SPL>
struct Chunk<MOE_FMT_BF16, SPL> {
  uint32_t v[8 * SPL];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k0) {
    const uint8_t *base = w.data + (size_t)e * expert_data_bytes(MOE_FMT_BF16, w.N, w.K) +
                          ((size_t)row * w.K + k0) * 2;
#pragma unroll
    for (int i = 0; i < 8 * SPL; i += 4) {
      const uint4 q = reinterpret_cast<const uint4 *>(base)[i / 4];
      v[i] = q.x, v[i + 1] = q.y, v[i + 2] = q.z, v[i + 3] = q.w;
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_x(const uint32_t (&xw)[NT][8 * SPL], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 8 * SPL; i++) acc = dot2_bf16(xw[t][i], v[i], acc);
      out[t] = acc;
    }
  }
  template <int NT>
  __device__ __forceinline__ void dot_a(const float (&af)[NT][16 * SPL],
                                        const float (&as)[NT][SPL], const uint2 *,
                                        float (&out)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; t++) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 8 * SPL; i++) {
        acc = fmaf(af[t][2 * i], bf16_lo(v[i]), acc);
        acc = fmaf(af[t][2 * i + 1], bf16_hi(v[i]), acc);
      }
      out[t] = acc;
    }
  }
};

// --------------------------------------------------------------------------
// shared pieces
// --------------------------------------------------------------------------

struct Bucket {
  int e, r0, r1;
};

// bucket of this block: from the plan (blockIdx.y-th active expert) or dense
__device__ __forceinline__ bool block_bucket(const int32_t *plan, int n_dense, Bucket *b) {
  if (plan) {
    const int a = blockIdx.y;
    if (a >= plan[0]) return false;
    b->e = plan[1 + 3 * a];
    b->r0 = plan[2 + 3 * a];
    b->r1 = plan[3 + 3 * a];
  } else {
    b->e = 0;
    b->r0 = 0;
    b->r1 = n_dense;
  }
  return true;
}

// VQ2 codebook -> LDS as bf16x4 entries, kNCopy copies interleaved so that
// copy c of every entry sits in the same two banks
__device__ __forceinline__ void fill_codebook(const int8_t *cb, uint2 *s_cb) {
  for (int i = threadIdx.x; i < 256 * kNCopy; i += blockDim.x) {
    const int e = i / kNCopy;
    const uint32_t w = reinterpret_cast<const uint32_t *>(cb)[e];
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int v = (int)(int8_t)((w >> (8 * j)) & 255u);
      b[j] = f32_to_bf16_bits((float)v);  // exact: |v| <= 128
    }
    s_cb[i] = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
  }
}

// bf16 pairs of x for the lane's chunk of NT tokens (rows rb.. of the bucket)
template <int SPL, int NT>
__device__ __forceinline__ void load_x(const uint16_t *x, int K, const int32_t *row_token, int rb,
                                       int nt, int k0, uint32_t (&xw)[NT][8 * SPL]) {
#pragma unroll
  for (int t = 0; t < NT; t++) {
    const int r = rb + (t < nt ? t : 0);
    const int tok = row_token ? row_token[r] : r;
    const uint4 *p = reinterpret_cast<const uint4 *>(x + (size_t)tok * K + k0);
#pragma unroll
    for (int i = 0; i < 2 * SPL; i++) {
      const uint4 q = p[i];
      xw[t][4 * i] = q.x, xw[t][4 * i + 1] = q.y, xw[t][4 * i + 2] = q.z, xw[t][4 * i + 3] = q.w;
    }
  }
}

// fp32 activations of the lane's chunk for NT bucket rows + sub-block sums
template <int SPL, int NT>
__device__ __forceinline__ void load_a(const float *a, int K, int rb, int nt, int k0,
                                       float (&af)[NT][16 * SPL], float (&as)[NT][SPL]) {
#pragma unroll
  for (int t = 0; t < NT; t++) {
    const int r = rb + (t < nt ? t : 0);
    const float4 *p = reinterpret_cast<const float4 *>(a + (size_t)r * K + k0);
#pragma unroll
    for (int i = 0; i < 4 * SPL; i++) {
      const float4 q = p[i];
      af[t][4 * i] = q.x, af[t][4 * i + 1] = q.y, af[t][4 * i + 2] = q.z, af[t][4 * i + 3] = q.w;
    }
#pragma unroll
    for (int i = 0; i < SPL; i++) {
      float s = 0.0f;
#pragma unroll
      for (int p2 = 0; p2 < 16; p2++) s += af[t][16 * i + p2];
      as[t][i] = s;
    }
  }
}

// --------------------------------------------------------------------------
// gate/up + SwiGLU
// --------------------------------------------------------------------------

struct GateUpArgs {
  WView gate, up;
  int H, I;
  const uint16_t *x;
  const int32_t *plan;
  int n_dense;
  const int32_t *row_token;
  float *a;
};

// block: 256 threads; rows per block = 4 waves * STEPS * (64 / LPR)
template <int FMT, int SPL, int LPR, int STEPS, int NT>
__global__ __launch_bounds__(256) void k_gateup(GateUpArgs p) {
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  Bucket b;
  if (!block_bucket(p.plan, p.n_dense, &b)) return;
  if constexpr (FMT == MOE_FMT_VQ2) {
    fill_codebook(p.gate.codebook, s_cb);
    __syncthreads();
  }
  constexpr int RPS = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = lane % LPR, rsub = lane / LPR;
  const int k0 = kl * 16 * SPL;
  const uint2 *cb = s_cb + (lane % kNCopy);
  const int row_base = (blockIdx.x * 4 + wave) * STEPS * RPS + rsub;
  for (int rb = b.r0; rb < b.r1; rb += NT) {
    const int nt = min(NT, b.r1 - rb);
    uint32_t xw[NT][8 * SPL];
    load_x<SPL, NT>(p.x, p.H, p.row_token, rb, nt, k0, xw);
    Chunk<FMT, SPL> cg[STEPS], cu[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; s++) {
      const int row = min(row_base + s * RPS, p.I - 1);
      cg[s].load(p.gate, b.e, row, k0);
      cu[s].load(p.up, b.e, row, k0);
    }
#pragma unroll
    for (int s = 0; s < STEPS; s++) {
      const int row = row_base + s * RPS;
      float g[NT], u[NT];
      cg[s].template dot_x<NT>(xw, cb, g);
      cu[s].template dot_x<NT>(xw, cb, u);
#pragma unroll
      for (int t = 0; t < NT; t++) {
        g[t] = group_sum<LPR>(g[t]);
        u[t] = group_sum<LPR>(u[t]);
      }
      if (kl == 0 && row < p.I) {
#pragma unroll
        for (int t = 0; t < NT; t++)
          if (t < nt) p.a[(size_t)(rb + t) * p.I + row] = silu_mul(g[t], u[t]);
      }
    }
  }
}

// --------------------------------------------------------------------------
// down: y[r][n] = down_e[n] . a[r]
// --------------------------------------------------------------------------

struct DownArgs {
  WView down;
  int H, I;
  const float *a;
  const int32_t *plan;
  int n_dense;
  float *y;
};

template <int FMT, int SPL, int LPR, int STEPS, int NT>
__global__ __launch_bounds__(256) void k_down(DownArgs p) {
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  Bucket b;
  if (!block_bucket(p.plan, p.n_dense, &b)) return;
  if constexpr (FMT == MOE_FMT_VQ2) {
    fill_codebook(p.down.codebook, s_cb);
    __syncthreads();
  }
  constexpr int RPS = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = lane % LPR, rsub = lane / LPR;
  const int k0 = kl * 16 * SPL;
  const uint2 *cb = s_cb + (lane % kNCopy);
  const int row_base = (blockIdx.x * 4 + wave) * STEPS * RPS + rsub;
  for (int rb = b.r0; rb < b.r1; rb += NT) {
    const int nt = min(NT, b.r1 - rb);
    float af[NT][16 * SPL], as[NT][SPL];
    load_a<SPL, NT>(p.a, p.I, rb, nt, k0, af, as);
    Chunk<FMT, SPL> c[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; s++) c[s].load(p.down, b.e, min(row_base + s * RPS, p.H - 1), k0);
#pragma unroll
    for (int s = 0; s < STEPS; s++) {
      const int row = row_base + s * RPS;
      float y[NT];
      c[s].template dot_a<NT>(af, as, cb, y);
#pragma unroll
      for (int t = 0; t < NT; t++) y[t] = group_sum<LPR>(y[t]);
      if (kl == 0 && row < p.H) {
#pragma unroll
        for (int t = 0; t < NT; t++)
          if (t < nt) p.y[(size_t)(rb + t) * p.H + row] = y[t];
      }
    }
  }
}

// --------------------------------------------------------------------------
// one token: down of every selected expert + weighted sum + shared, fused
// out[n] = shared_y[n] + sum_a row_w[a] * down_{e_a}[n] . a_rows[a]
// --------------------------------------------------------------------------

struct DownCombineArgs {
  WView down;
  int H, I;
  const float *a;
  const int32_t *plan;
  const float *row_w;
  const float *shared_y;
  float *out;
  uint16_t *out_bf16;
};

template <int FMT, int SPL, int STEPS>
__global__ __launch_bounds__(256) void k_down_combine1(DownCombineArgs p) {
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  if constexpr (FMT == MOE_FMT_VQ2) {
    fill_codebook(p.down.codebook, s_cb);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = lane * 16 * SPL;
  const uint2 *cb = s_cb + (lane % kNCopy);
  const int row_base = (blockIdx.x * 4 + wave) * STEPS;
  const int n_act = p.plan[0];
  float acc[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; s++) acc[s] = 0.0f;
  for (int a = 0; a < n_act; a++) {
    const int e = p.plan[1 + 3 * a], r = p.plan[2 + 3 * a];
    Chunk<FMT, SPL> c[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; s++) c[s].load(p.down, e, min(row_base + s, p.H - 1), k0);
    float af[1][16 * SPL], as[1][SPL];
    load_a<SPL, 1>(p.a, p.I, r, 1, k0, af, as);
    const float wr = p.row_w[r];
#pragma unroll
    for (int s = 0; s < STEPS; s++) {
      float y[1];
      c[s].template dot_a<1>(af, as, cb, y);
      acc[s] = fmaf(wr, y[0], acc[s]);
    }
  }
#pragma unroll
  for (int s = 0; s < STEPS; s++) {
    const float v = group_sum<64>(acc[s]);
    const int row = row_base + s;
    if (lane == 0 && row < p.H) {
      const float o = v + (p.shared_y ? p.shared_y[row] : 0.0f);
      p.out[row] = o;
      if (p.out_bf16) p.out_bf16[row] = (uint16_t)f32_to_bf16_bits(o);
    }
  }
}

// --------------------------------------------------------------------------
// host dispatch over formats and K
// --------------------------------------------------------------------------

namespace {

// lane geometry for a row length K: returns false when unsupported
bool geometry(int K, int *spl, int *lpr) {
  if (K >= 1024 && K % 1024 == 0 && K / 1024 <= 8 && (K / 1024) != 3 && (K / 1024) != 5 &&
      (K / 1024) != 6 && (K / 1024) != 7) {
    *spl = K / 1024;
    *lpr = 64;
    return true;
  }
  if (K == 512 || K == 256 || K == 128) {
    *spl = 1;
    *lpr = K / 16;
    return true;
  }
  return false;
}

// rows per wave step so that the raw bits in flight stay near 32 dwords per
// lane per projection (more for small chunks, fewer for bf16's 8 dwords per
// 16 weights)
template <int FMT, int SPL>
constexpr int steps_for() {
  constexpr int dw = FMT == MOE_FMT_BF16 ? 8 * SPL : FMT == MOE_FMT_VQ2 ? SPL + 1 : 2 * SPL + 1;
  return dw >= 32 ? 1 : dw >= 16 ? 2 : 4;
}

template <int FMT, int SPL, int LPR>
hipError_t gateup_inst(const GateUpArgs &a, int max_active, int ntok_hint, hipStream_t s) {
  constexpr int ST = steps_for<FMT, SPL>();
  constexpr int RPB = 4 * ST * (64 / LPR);
  dim3 grid((a.I + RPB - 1) / RPB, a.plan ? max_active : 1);
  if (ntok_hint >= 4)
    k_gateup<FMT, SPL, LPR, ST, 4><<<grid, 256, 0, s>>>(a);
  else
    k_gateup<FMT, SPL, LPR, ST, 1><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int FMT, int SPL, int LPR>
hipError_t down_inst(const DownArgs &a, int max_active, int ntok_hint, hipStream_t s) {
  constexpr int ST = steps_for<FMT, SPL>();
  constexpr int RPB = 4 * ST * (64 / LPR);
  dim3 grid((a.H + RPB - 1) / RPB, a.plan ? max_active : 1);
  if (ntok_hint >= 4)
    k_down<FMT, SPL, LPR, ST, 4><<<grid, 256, 0, s>>>(a);
  else
    k_down<FMT, SPL, LPR, ST, 1><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int FMT>
hipError_t gateup_fmt(const GateUpArgs &a, int max_active, int nh, hipStream_t s) {
  int spl, lpr;
  if (!geometry(a.H, &spl, &lpr)) return hipErrorInvalidValue;
  if (lpr == 64) {
    switch (spl) {
      case 1: return gateup_inst<FMT, 1, 64>(a, max_active, nh, s);
      case 2: return gateup_inst<FMT, 2, 64>(a, max_active, nh, s);
      case 4: return gateup_inst<FMT, 4, 64>(a, max_active, nh, s);
      case 8: return gateup_inst<FMT, 8, 64>(a, max_active, nh, s);
    }
  }
  switch (lpr) {
    case 8: return gateup_inst<FMT, 1, 8>(a, max_active, nh, s);
    case 16: return gateup_inst<FMT, 1, 16>(a, max_active, nh, s);
    case 32: return gateup_inst<FMT, 1, 32>(a, max_active, nh, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t down_fmt(const DownArgs &a, int max_active, int nh, hipStream_t s) {
  int spl, lpr;
  if (!geometry(a.I, &spl, &lpr)) return hipErrorInvalidValue;
  if (lpr == 64) {
    switch (spl) {
      case 1: return down_inst<FMT, 1, 64>(a, max_active, nh, s);
      case 2: return down_inst<FMT, 2, 64>(a, max_active, nh, s);
      case 4: return down_inst<FMT, 4, 64>(a, max_active, nh, s);
      case 8: return down_inst<FMT, 8, 64>(a, max_active, nh, s);
    }
  }
  switch (lpr) {
    case 8: return down_inst<FMT, 1, 8>(a, max_active, nh, s);
    case 16: return down_inst<FMT, 1, 16>(a, max_active, nh, s);
    case 32: return down_inst<FMT, 1, 32>(a, max_active, nh, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int SPL>
hipError_t dc_inst(const DownCombineArgs &a, hipStream_t s) {
  constexpr int ST = steps_for<FMT, SPL>();
  constexpr int RPB = 4 * ST;
  k_down_combine1<FMT, SPL, ST><<<(a.H + RPB - 1) / RPB, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int FMT>
hipError_t dc_fmt(const DownCombineArgs &a, hipStream_t s) {
  int spl, lpr;
  if (!geometry(a.I, &spl, &lpr) || lpr != 64) return hipErrorInvalidValue;
  switch (spl) {
    case 1: return dc_inst<FMT, 1>(a, s);
    case 2: return dc_inst<FMT, 2>(a, s);
    case 4: return dc_inst<FMT, 4>(a, s);
    case 8: return dc_inst<FMT, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool gemv_supported_k(int K) {
  int spl, lpr;
  return geometry(K, &spl, &lpr);
}

bool down_combine_supported(int I) {
  int spl, lpr;
  return geometry(I, &spl, &lpr) && lpr == 64;
}

hipError_t launch_gateup_gemv(const WView &gate, const WView &up, int H, int I,
                              const uint16_t *x, const int32_t *plan, int max_active,
                              const int32_t *row_token, float *a, hipStream_t s) {
  GateUpArgs g{gate, up, H, I, x, plan, max_active, row_token, a};
  // dense call: max_active carries the token count
  const int nh = plan ? 1 : max_active;
  switch (gate.fmt) {
    case MOE_FMT_BF16: return gateup_fmt<MOE_FMT_BF16>(g, max_active, nh, s);
    case MOE_FMT_Q2K: return gateup_fmt<MOE_FMT_Q2K>(g, max_active, nh, s);
    case MOE_FMT_VQ2: return gateup_fmt<MOE_FMT_VQ2>(g, max_active, nh, s);
    case MOE_FMT_MXFP4: return gateup_fmt<MOE_FMT_MXFP4>(g, max_active, nh, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_gemv(const WView &down, int H, int I, const float *a, const int32_t *plan,
                            int max_active, float *y, hipStream_t s) {
  DownArgs d{down, H, I, a, plan, max_active, y};
  const int nh = plan ? 1 : max_active;
  switch (down.fmt) {
    case MOE_FMT_BF16: return down_fmt<MOE_FMT_BF16>(d, max_active, nh, s);
    case MOE_FMT_Q2K: return down_fmt<MOE_FMT_Q2K>(d, max_active, nh, s);
    case MOE_FMT_VQ2: return down_fmt<MOE_FMT_VQ2>(d, max_active, nh, s);
    case MOE_FMT_MXFP4: return down_fmt<MOE_FMT_MXFP4>(d, max_active, nh, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_combine(const WView &down, int H, int I, int T, const float *a,
                               const int32_t *plan, int max_active, const int32_t *row_token,
                               const float *row_w, const float *shared_y, float *out,
                               uint16_t *out_bf16, hipStream_t s) {
  (void)row_token;
  (void)max_active;
  if (T != 1) return hipErrorInvalidValue;
  DownCombineArgs d{down, H, I, a, plan, row_w, shared_y, out, out_bf16};
  switch (down.fmt) {
    case MOE_FMT_BF16: return dc_fmt<MOE_FMT_BF16>(d, s);
    case MOE_FMT_Q2K: return dc_fmt<MOE_FMT_Q2K>(d, s);
    case MOE_FMT_VQ2: return dc_fmt<MOE_FMT_VQ2>(d, s);
    case MOE_FMT_MXFP4: return dc_fmt<MOE_FMT_MXFP4>(d, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
