// gemm.hip -- prefill: grouped per-expert GEMMs on the matrix cores.
//
// With many tokens every expert receives a bucket of rows and the expert FFN
// becomes a grouped GEMM (the ds4 pages: prefill amortises the expert weights
// over the batch -- hysenlabs.com "SSD streaming"; matrix-instruction expert
// kernels on newer devices -- hysenlabs.com "Model support and quantization").
// Each workgroup computes a 64-row x 128-column tile of one expert's bucket:
// the A rows (tokens gathered through the bucket, or the SwiGLU output in
// bucket order) and the weight tile are staged through LDS, the weights being
// dequantized as they are staged; 4 waves each run 32x32x16 MFMAs on a
// 32 x 64 sub-tile.
//
// Precision: gate/up multiply the bf16 tokens by exact bf16 weight values --
// VQ2 codebook entries are small integers (exact in bf16) and the fp16 scale
// of each 256-column group multiplies the fp32 partial sum of that group;
// MXFP4 and bf16 weights are exact in bf16.  Q2K gate/up and every down
// projection use fp16 operands (the SwiGLU output and the weights rounded to
// fp16), accumulating in fp32.
#include "gemv_core.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 64;          // bucket rows per tile
constexpr int kBN = 128;         // weight rows per tile (gate/up: 64 gate + 64 up)
constexpr int kBK = 64;          // reduction columns per stage
constexpr int kLdsK = kBK + 8;   // padded LDS row: 144 bytes
constexpr int kLdsW = kLdsK / 2; // ... in dwords
constexpr int kGemmThreads = 256;

enum { kOpBF16 = 0, kOpF16 = 1 };
enum { kModeGateUp = 0, kModeDown = 1 };

// tile list: tiles[0] = count; tile i = tiles[1 + 3i .. 3 + 3i] = {expert, r0, r1}
size_t gemm_tile_ints(int n_rows, int E) {
  return 1 + 3 * (size_t)((n_rows + kBM - 1) / kBM + E);
}

__global__ __launch_bounds__(1024) void k_tile_list(int E, int n_dense,
                                                     const int32_t *__restrict__ offsets,
                                                     int32_t *__restrict__ tiles) {
  __shared__ int s_tmp[16];
  if (!offsets) {  // one dense expert over rows [0, n_dense)
    const int n = (n_dense + kBM - 1) / kBM;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      tiles[1 + 3 * i] = 0;
      tiles[2 + 3 * i] = i * kBM;
      tiles[3 + 3 * i] = min(n_dense, (i + 1) * kBM);
    }
    if (threadIdx.x == 0) tiles[0] = n;
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (c + kBM - 1) / kBM;
    int inc = nt;  // inclusive scan over the wave
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    if (lane == 63) s_tmp[wv] = inc;
    __syncthreads();
    int wbase = 0, tot = 0;
    for (int i = 0; i < 16; i++) {
      wbase += i < wv ? s_tmp[i] : 0;
      tot += s_tmp[i];
    }
    __syncthreads();
    int pos = base + wbase + inc - nt;
    for (int t = 0; t < nt; t++, pos++) {
      const int r0 = offsets[e] + t * kBM;
      tiles[1 + 3 * pos] = e;
      tiles[2 + 3 * pos] = r0;
      tiles[3 + 3 * pos] = min(offsets[e + 1], r0 + kBM);
    }
    base += tot;
  }
  if (threadIdx.x == 0) tiles[0] = base;
}

struct GemmArgs {
  int K, N;                  // reduction length; columns of the layer's output (I or H)
  WView w0, w1;              // gate and up, or down (w0 == w1)
  const uint16_t *x;         // gate/up: bf16 tokens [T][K]
  const int32_t *row_token;  // gate/up: token of each bucket row (null: the row itself)
  const uint16_t *a16;       // down: fp16 SwiGLU output [n_rows][K]
  int a_rows;                // rows of x (gate/up: T) or of a16 (down: n_rows)
  const int32_t *tiles;
  uint16_t *a_out;           // gate/up: fp16 [n_rows][N]
  float *y_out;              // down: fp32 [n_rows][N]
};

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ uint32_t pack_b2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}
template <int OP>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return OP == kOpF16 ? pack_h2(a, b) : pack_b2(a, b);
}
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) { return pack_h2(bf16_lo(v), bf16_hi(v)); }

// ---------------------------------------------------------------------------
// B (weight) stage: 128 weight rows x 64 columns.  Thread t stages row t / 2,
// columns (t % 2) * 32 .. +32: it loads the packed bytes for the next stage
// while the MFMAs of the current one run, then decodes them into 16 dwords of
// operand pairs in LDS.
// ---------------------------------------------------------------------------
template <int FMT, int OP>
struct BStage {
  uint32_t raw[FMT == MOE_FMT_BF16 ? 16 : 8];
  uint32_t aux;

  __device__ __forceinline__ void load(const WView &w, int e, int row, int k) {
    const uint32_t db = (uint32_t)expert_data_bytes(FMT, w.N, w.K);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(w.data + (size_t)e * db, db);
    if constexpr (FMT == MOE_FMT_BF16) {
      const uint32_t vo = ((uint32_t)row * (uint32_t)w.K + (uint32_t)k) * 2u;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const u32x4_t q = buf_u128(r, vo + 16 * i, 0);
        raw[4 * i] = q.x, raw[4 * i + 1] = q.y, raw[4 * i + 2] = q.z, raw[4 * i + 3] = q.w;
      }
    } else if constexpr (FMT == MOE_FMT_VQ2) {  // one code byte per 4 weights
      const u32x2_t q = buf_u64(r, (uint32_t)row * (uint32_t)(w.K / 4) + (uint32_t)k / 4, 0);
      raw[0] = q.x, raw[1] = q.y;
    } else if constexpr (FMT == MOE_FMT_Q2K) {  // sub-blocks j, j+1 of one super-block
      const uint32_t blk = ((uint32_t)row * (uint32_t)(w.K / 256) + (uint32_t)k / 256) * kQ2KBytes;
      const uint32_t j = (k % 256) / 16;
      raw[0] = buf_u32(r, blk + 16 + 4 * j, 0);
      raw[1] = buf_u32(r, blk + 16 + 4 * j + 4, 0);
      raw[2] = buf_u32(r, blk + 80, 0);
      aux = buf_u16(r, blk + j, 0);
    } else {  // MXFP4: 16 bytes of nibbles + one E8M0 scale per 32
      const uint32_t sb = (uint32_t)expert_scale_bytes(FMT, w.N, w.K);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
      const u32x4_t q = buf_u128(r, (uint32_t)row * (uint32_t)(w.K / 2) + (uint32_t)k / 2, 0);
      raw[0] = q.x, raw[1] = q.y, raw[2] = q.z, raw[3] = q.w;
      aux = buf_u8(rs, (uint32_t)row * (uint32_t)(w.K / 32) + (uint32_t)k / 32, 0);
    }
  }

  __device__ __forceinline__ void store(uint32_t *dst, const uint2 *s_cb) const {
    uint32_t o[16];
    if constexpr (FMT == MOE_FMT_BF16) {
#pragma unroll
      for (int i = 0; i < 16; i++) o[i] = OP == kOpF16 ? bf16x2_to_f16x2(raw[i]) : raw[i];
    } else if constexpr (FMT == MOE_FMT_VQ2) {  // codebook integers; the group scale comes later
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const uint2 v = s_cb[(raw[c / 4] >> (8 * (c % 4))) & 255u];
        o[2 * c] = v.x, o[2 * c + 1] = v.y;
      }
    } else if constexpr (FMT == MOE_FMT_Q2K) {
      const float d = f16_bits_to_f32(raw[2] & 0xFFFFu), dmin = f16_bits_to_f32(raw[2] >> 16);
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const uint32_t scm = (aux >> (8 * s)) & 255u;
        const float ds = d * (float)(scm & 15u), ms = dmin * (float)(scm >> 4);
#pragma unroll
        for (int p = 0; p < 16; p += 2) {
          const float w0 = ds * (float)((raw[s] >> (2 * p)) & 3u) - ms;
          const float w1 = ds * (float)((raw[s] >> (2 * p + 2)) & 3u) - ms;
          o[8 * s + p / 2] = pack2<OP>(w0, w1);
        }
      }
    } else {  // MXFP4
      const float sc = e8m0_to_f32(aux);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t p0 = e2m1x2_to_bf16x2<0>(raw[j]), p1 = e2m1x2_to_bf16x2<1>(raw[j]);
        const uint32_t p2 = e2m1x2_to_bf16x2<2>(raw[j]), p3 = e2m1x2_to_bf16x2<3>(raw[j]);
        o[4 * j] = pack2<OP>(bf16_lo(p0) * sc, bf16_hi(p0) * sc);
        o[4 * j + 1] = pack2<OP>(bf16_lo(p1) * sc, bf16_hi(p1) * sc);
        o[4 * j + 2] = pack2<OP>(bf16_lo(p2) * sc, bf16_hi(p2) * sc);
        o[4 * j + 3] = pack2<OP>(bf16_lo(p3) * sc, bf16_hi(p3) * sc);
      }
    }
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int i = 0; i < 4; i++) d4[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
};

// A stage: 64 rows x 64 columns; thread t stages row t / 4, columns (t % 4) * 16 .. +16
template <int MODE, int OP>
struct AStage {
  uint32_t raw[8];
  // rows past the bucket carry an offset beyond the buffer: the loads read zeros
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int k) {
    const uint32_t vo = row_off + (uint32_t)k * 2u;
    const u32x4_t q0 = buf_u128(r, vo, 0), q1 = buf_u128(r, vo + 16, 0);
    raw[0] = q0.x, raw[1] = q0.y, raw[2] = q0.z, raw[3] = q0.w;
    raw[4] = q1.x, raw[5] = q1.y, raw[6] = q1.z, raw[7] = q1.w;
  }
  __device__ __forceinline__ void store(uint32_t *dst) const {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      o[i] = (MODE == kModeGateUp && OP == kOpF16) ? bf16x2_to_f16x2(raw[i]) : raw[i];
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
    d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
};

template <int OP>
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  if constexpr (OP == kOpBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// the grouped GEMM: grid.x = column tiles of the layer, grid.y = bucket tiles
// ---------------------------------------------------------------------------
template <int MODE, int FMT, int OP>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs p) {
  __shared__ uint32_t s_a[2][kBM * kLdsW];
  __shared__ uint32_t s_b[2][kBN * kLdsW];
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 : 1];
  // XCD-aware order: workgroups go round-robin to the 8 XCDs, so linear id b
  // runs on XCD b % 8.  Give XCD x the tiles x, x + 8, ... and walk all column
  // blocks of one tile back to back there, so its L2 fetches each A tile once.
  // (grid.y is a multiple of 8.)
  const uint32_t nbx = gridDim.x;
  const uint32_t b = blockIdx.y * nbx + blockIdx.x;
  const uint32_t j = b >> 3;
  const int ti = (int)((j / nbx) * 8 + (b & 7));
  const int bx = (int)(j % nbx);
  if (ti >= p.tiles[0]) return;
  const int e = __builtin_amdgcn_readfirstlane(p.tiles[1 + 3 * ti]);
  const int r0 = __builtin_amdgcn_readfirstlane(p.tiles[2 + 3 * ti]);
  const int r1 = __builtin_amdgcn_readfirstlane(p.tiles[3 + 3 * ti]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int kCols = MODE == kModeGateUp ? kBN / 2 : kBN;  // output columns per tile
  const int n0 = bx * kCols;

  if constexpr (FMT == MOE_FMT_VQ2) {  // codebook entries as exact operand pairs
    const uint32_t cw = reinterpret_cast<const uint32_t *>(p.w0.codebook)[tid];
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = (float)(int)(int8_t)((cw >> (8 * j)) & 255u);
    s_cb[tid] = make_uint2(pack2<OP>(v[0], v[1]), pack2<OP>(v[2], v[3]));
  }

  // A staging: bucket row tid / 4
  const int arow = tid >> 2, ak = (tid & 3) * 16;
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)p.K * 2u;
  uint32_t a_off = a_bytes;  // past the end: zeros
  if (r0 + arow < r1) {
    const int src = (MODE == kModeGateUp && p.row_token) ? p.row_token[r0 + arow] : r0 + arow;
    a_off = (uint32_t)src * (uint32_t)p.K * 2u;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(MODE == kModeGateUp ? p.x : p.a16, a_bytes);
  // B staging: tile row tid / 2 (waves 2, 3 stage the up rows of a gate/up tile)
  const int brow = tid >> 1, bk = (tid & 1) * 32;
  const bool b_up = MODE == kModeGateUp && wave >= 2;
  const WView &bw = b_up ? p.w1 : p.w0;
  const int wrow = MODE == kModeGateUp ? n0 + (brow & (kBN / 2 - 1)) : n0 + brow;

  // kPD stages in flight: stage s is staged in registers slot s % kPD from the
  // time its loads are issued until it is decoded into LDS, kPD - 1 stages
  // before the MFMAs read it, which covers the HBM latency
  constexpr int kPD = 4;
  AStage<MODE, OP> sa[kPD];
  BStage<FMT, OP> sb[kPD];
  const int nk = p.K / kBK;
#pragma unroll
  for (int u = 0; u < kPD; u++) {  // nk >= kPD (K >= 256)
    sa[u].load(ra, a_off, u * kBK + ak);
    sb[u].load(bw, e, wrow, u * kBK + bk);
  }
  if constexpr (FMT == MOE_FMT_VQ2) __syncthreads();
  sa[0].store(&s_a[0][arow * kLdsW + ak / 2]);
  sb[0].store(&s_b[0][brow * kLdsW + bk / 2], s_cb);
  {  // stages past the end re-read the last one (never used; keeps the loads unconditional)
    const int st = min(kPD, nk - 1);
    sa[0].load(ra, a_off, st * kBK + ak);
    sb[0].load(bw, e, wrow, st * kBK + bk);
  }
  __syncthreads();

  // the lane's two B columns: gate/up -> (gate, up) of column n0 + 32 wn + lane % 32;
  // down -> columns n0 + 64 wn + lane % 32 and that + 32
  const int cl = lane & 31;
  const int bc0 = MODE == kModeGateUp ? 32 * wn + cl : 64 * wn + cl;
  const int bc1 = MODE == kModeGateUp ? kBN / 2 + 32 * wn + cl : 64 * wn + 32 + cl;
  const int arow_frag = 32 * wm + cl;
  const int kh = 8 * (lane >> 5);
  // a wave whose 32 rows all lie past the bucket's end skips its MFMAs
  const bool active = r0 + 32 * wm < r1;

  constexpr bool kGroupScale = FMT == MOE_FMT_VQ2;
  // VQ2: the fp16 scales of the lane's two weight rows, all K / 256 <= 16 groups
  uint32_t gsc0[kGroupScale ? 8 : 1] = {}, gsc1[kGroupScale ? 8 : 1] = {};
  if constexpr (kGroupScale) {
    const int wr0 = n0 + (MODE == kModeGateUp ? 32 * wn + cl : 64 * wn + cl);
    const int wr1 = MODE == kModeGateUp ? wr0 : wr0 + 32;
    const WView &v1 = MODE == kModeGateUp ? p.w1 : p.w0;
    const uint32_t sbb = (uint32_t)expert_scale_bytes(FMT, p.w0.N, p.w0.K);
    const uint32_t rb = (uint32_t)(p.K / 256) * 2u;  // scale bytes per row
    const __amdgpu_buffer_rsrc_t s0 = make_rsrc(p.w0.scales + (size_t)e * sbb, sbb);
    const __amdgpu_buffer_rsrc_t s1 = make_rsrc(v1.scales + (size_t)e * sbb, sbb);
#pragma unroll
    for (int q = 0; q < 8; q++) {
      // past the row's K / 256 groups this reads the next row (or zeros past
      // the expert): never used, and it keeps the loads unconditional
      gsc0[q] = buf_u32(s0, (uint32_t)wr0 * rb + 4 * q, 0);
      gsc1[q] = buf_u32(s1, (uint32_t)wr1 * rb + 4 * q, 0);
    }
  }
  f32x16_t acc0 = {}, acc1 = {}, part0 = {}, part1 = {};
  for (int it0 = 0; it0 < nk; it0 += kPD) {
#pragma unroll
    for (int u = 0; u < kPD; u++) {
      const int it = it0 + u;  // nk % kPD == 0 (K % 256 == 0)
      const uint32_t *A = s_a[it & 1];
      const uint32_t *B = s_b[it & 1];
      if (active) {
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ks++) {
          const int kk = ks * 16 + kh;
          const uint4 af = *reinterpret_cast<const uint4 *>(&A[arow_frag * kLdsW + kk / 2]);
          const uint4 bf0 = *reinterpret_cast<const uint4 *>(&B[bc0 * kLdsW + kk / 2]);
          const uint4 bf1 = *reinterpret_cast<const uint4 *>(&B[bc1 * kLdsW + kk / 2]);
          if constexpr (kGroupScale) {
            part0 = mfma32<OP>(af, bf0, part0);
            part1 = mfma32<OP>(af, bf1, part1);
          } else {
            acc0 = mfma32<OP>(af, bf0, acc0);
            acc1 = mfma32<OP>(af, bf1, acc1);
          }
        }
        if constexpr (kGroupScale) {
          if ((it + 1) % (256 / kBK) == 0) {  // a 256-column group is complete: scale and fold
            const int kb = it / (256 / kBK);
            const uint32_t h0 = gsc0[kb >> 1], h1 = gsc1[kb >> 1];
            const float d0 = f16_bits_to_f32((kb & 1) ? h0 >> 16 : h0 & 0xFFFFu);
            const float d1 = f16_bits_to_f32((kb & 1) ? h1 >> 16 : h1 & 0xFFFFu);
#pragma unroll
            for (int i = 0; i < 16; i++) {
              acc0[i] = fmaf(d0, part0[i], acc0[i]);
              acc1[i] = fmaf(d1, part1[i], acc1[i]);
              part0[i] = 0.0f;
              part1[i] = 0.0f;
            }
          }
        }
      }
      // decode stage it + 1 into the other buffer, then refill its slot
      const int slot = (u + 1) % kPD;
      // (after the last stage this fills the idle buffer with a repeat: unread)
      sa[slot].store(&s_a[(it + 1) & 1][arow * kLdsW + ak / 2]);
      sb[slot].store(&s_b[(it + 1) & 1][brow * kLdsW + bk / 2], s_cb);
      const int st = min(it + 1 + kPD, nk - 1);
      sa[slot].load(ra, a_off, st * kBK + ak);
      sb[slot].load(bw, e, wrow, st * kBK + bk);
      __syncthreads();
    }
  }

  // result i of the lane: tile row 32 wm + (i % 4) + 8 (i / 4) + 4 (lane / 32)
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int r = r0 + 32 * wm + (i & 3) + 8 * (i >> 2) + 4 * (lane >> 5);
    if (r >= r1) continue;
    if constexpr (MODE == kModeGateUp) {
      const float a = silu_mul(acc0[i], acc1[i]);
      p.a_out[(size_t)r * p.N + n0 + 32 * wn + cl] = __builtin_bit_cast(uint16_t, (_Float16)a);
    } else {
      float *yr = p.y_out + (size_t)r * p.N + n0 + 64 * wn + cl;
      yr[0] = acc0[i];
      yr[32] = acc1[i];
    }
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------

// K a multiple of 256 (whole Q2K / VQ2 groups; at least kPD stages); VQ2 keeps
// all its K / 256 group scales of a row in registers: K <= 4096
bool gemm_supported(int H, int I, int fmt_gate, int fmt_down) {
  if (H < 256 || I < 256 || H % 256 || I % 256) return false;
  if (fmt_gate == MOE_FMT_VQ2 && H > 4096) return false;
  if (fmt_down == MOE_FMT_VQ2 && I > 4096) return false;
  return true;
}

namespace {

template <int MODE>
hipError_t gemm_fmt(const GemmArgs &a, int fmt, int op, dim3 grid, hipStream_t s) {
#define MOE_GEMM_CASE(F, O)                                \
  if (fmt == F && op == O) {                               \
    launch(k_gemm<MODE, F, O>, dim3(grid), dim3(kGemmThreads), s, a);   \
    return hipGetLastError();                              \
  }
  MOE_GEMM_CASE(MOE_FMT_BF16, kOpBF16)
  MOE_GEMM_CASE(MOE_FMT_BF16, kOpF16)
  MOE_GEMM_CASE(MOE_FMT_VQ2, kOpBF16)
  MOE_GEMM_CASE(MOE_FMT_VQ2, kOpF16)
  MOE_GEMM_CASE(MOE_FMT_Q2K, kOpF16)
  MOE_GEMM_CASE(MOE_FMT_MXFP4, kOpBF16)
  MOE_GEMM_CASE(MOE_FMT_MXFP4, kOpF16)
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                           int T, const uint16_t *x, const int32_t *offsets, const int32_t *sorted_token,
                           int n_rows, int32_t *tiles, uint16_t *a16, float *y, hipStream_t s,
                           void (*mark)(void *, const char *), void *mark_ctx,
                           const char *const names[3]) {
  if (!gemm_supported(H, I, gate.fmt, down.fmt) || n_rows < 1 || T < 1) return hipErrorInvalidValue;
  const int E = offsets ? gate.E : 0;
  const int max_tiles = ((n_rows + kBM - 1) / kBM + E + 7) / 8 * 8;
  if (mark) mark(mark_ctx, names[0]);
  launch(k_tile_list, dim3(1), dim3(1024), s, E, n_rows, offsets, tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  GemmArgs g{};
  g.K = H, g.N = I, g.w0 = gate, g.w1 = up, g.x = x, g.a_rows = T;
  g.row_token = offsets ? sorted_token : nullptr;
  g.tiles = tiles, g.a_out = a16;
  if (mark) mark(mark_ctx, names[1]);
  err = gemm_fmt<kModeGateUp>(g, gate.fmt, gate.fmt == MOE_FMT_Q2K ? kOpF16 : kOpBF16,
                              dim3(I / (kBN / 2), max_tiles), s);
  if (err != hipSuccess) return err;

  GemmArgs d{};
  d.K = I, d.N = H, d.w0 = down, d.w1 = down, d.a16 = a16, d.a_rows = n_rows, d.tiles = tiles;
  d.y_out = y;
  if (mark) mark(mark_ctx, names[2]);
  return gemm_fmt<kModeDown>(d, down.fmt, kOpF16, dim3(H / kBN, max_tiles), s);
}

}  // namespace moe
