// gemm_fp4.hip -- MXFP4 experts on gfx950's native FP4 matrix instructions.
//
// The A8 variant of the MXFP4 layer (hysenlabs.com "Model support and
// quantization": an MXFP4 variant keeps the released FP4 expert weights):
// the activations entering each routed projection are quantized to OCP
// MX-FP8 (E4M3 elements, one E8M0 scale per 32 along K) and multiplied with
// the raw FP4 weights and their E8M0 scales by
// v_mfma_scale_f32_16x16x128_f8f6f4 -- no weight is ever decoded by VALU.
//
// MX-FP8 of a 32-element group (OCP MX v1.0): scale X = 2^(floor(log2 amax)
// - 8), 8 being E4M3's largest exponent; element = E4M3 nearest to v / X,
// ties to an even mantissa, saturating at 448; amax == 0 gives scale byte 0
// and zero elements.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (probed on the device
// with random operands, matched exactly):
//   A (E4M3, 32 bytes per lane): lane l holds row l % 16, byte i is
//     k = 64 (i / 16) + 16 (l / 16) + i % 16;
//   B (E2M1, 16 bytes per lane): lane l holds column l % 16, nibble i (low
//     nibble first) is k = 32 (l / 16) + i;
//   scales: byte 0 of lane r + 16 j scales row (column) r over k in
//     [32 j, 32 j + 32);
//   D: register i of lane l is row 4 (l / 16) + i, column l % 16.
//
// Workgroups are laid out as in gemm.hip: BM bucket rows of one expert
// against 256 weight rows (gate/up: 128 gate + 128 up; down: 256 outputs),
// 4 waves of 64 weight rows; the activation rows are staged in LDS per K
// step of 128, the weight bytes go straight from memory into the operand
// registers.  Gate/up's epilogue applies SwiGLU and quantizes the result to
// MX-FP8 (a wave's 32 columns of a row are exactly one scale group).
#include <type_traits>

#include "gemv_core.h"
#include "lds_dma.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4a_t __attribute__((ext_vector_type(4)));

enum { kModeGateUp = 0, kModeDown = 1 };
constexpr int kA8K = 128;                // K per MFMA and per LDS stage
constexpr int kA8Row = kA8K + 16;        // padded LDS row, bytes
constexpr int kA8Threads = 256;

// ---------------------------------------------------------------------------
// MX-FP8 quantization
// ---------------------------------------------------------------------------

// E8M0 scale byte of a group from its largest magnitude
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  if (!(amax > 0.0f)) return 0u;
  int ex;
  (void)frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
  const int e8 = ex - 1 - 8 + 127;
  return (uint32_t)(e8 < 0 ? 0 : e8 > 254 ? 254 : e8);
}

// E4M3 code nearest to y (ties to an even mantissa), saturating at 448
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f)  // below 2^-6: subnormal codes m * 2^-9 (m = 8 is 2^-6)
    return sign | (uint32_t)rintf(a * 512.0f);
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // -6 .. 8
  const float m = rintf((a * __builtin_ldexpf(1.0f, -e) - 1.0f) * 8.0f);
  // m == 8 carries into the exponent; a < 448 keeps the code below NaN
  return sign | (uint32_t)(((e + 7) << 3) + (int)m);
}

// x: bf16 [rows][K] -> q: E4M3 [rows][K], s: E8M0 [rows][K / 32].  Thread t
// takes 8 consecutive values; the 4 threads of a group are adjacent lanes.
__global__ __launch_bounds__(256) void k_mx8_quant(int rows, int K, const uint16_t *__restrict__ x,
                                                   uint8_t *__restrict__ q,
                                                   uint8_t *__restrict__ s) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long n8 = (long)rows * (K / 8);
  const bool live = t < n8;
  const long tt = live ? t : 0;
  const uint4 w = *reinterpret_cast<const uint4 *>(x + tt * 8);
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  float v[8], amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = bf16_lo(ww[i]);
    v[2 * i + 1] = bf16_hi(ww[i]);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const uint32_t e8 = mx8_scale_byte(amax);
  const int sh = 127 - (int)e8;  // v / X
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    lo |= (amax > 0.0f ? e4m3_code(__builtin_ldexpf(v[i], sh)) : 0u) << (8 * i);
    hi |= (amax > 0.0f ? e4m3_code(__builtin_ldexpf(v[4 + i], sh)) : 0u) << (8 * i);
  }
  if (live) {
    *reinterpret_cast<uint2 *>(q + tt * 8) = make_uint2(lo, hi);
    if ((tt & 3) == 0) s[tt / 4] = (uint8_t)e8;
  }
}

// ---------------------------------------------------------------------------
// the GEMM
// ---------------------------------------------------------------------------

struct A8Args {
  int K, N;                  // reduction length; columns of the layer's output (I or H)
  WView w0, w1;              // gate and up, or down (w0 == w1); MXFP4
  const uint8_t *aq;         // E4M3 activation rows [a_rows][K]
  const uint8_t *as;         // their E8M0 scales [a_rows][K / 32]
  const int32_t *row_token;  // gate/up: row of aq for each bucket row (null: the row itself)
  int a_rows;
  const int32_t *tiles;
  int weight_major;
  uint8_t *out_q, *out_s;  // gate/up: MX-FP8 SwiGLU output [n_rows][N], [n_rows][N / 32]
  float *a_f32;            // gate/up, optional: the SwiGLU output before quantization [n_rows][N]
  float *y_out;            // down: fp32 [n_rows][N]
};

template <int MODE>
constexpr int a8_block_cols() { return MODE == kModeGateUp ? 128 : 256; }

template <int MODE, int BM>
__global__ __launch_bounds__(kA8Threads) void k_gemm_a8(A8Args p) {
  constexpr int MB = BM / 16;
  constexpr int NB = 4;
  constexpr int kTPR = kA8Threads / BM;  // threads per staged row
  constexpr int kBPT = kA8K / kTPR;      // bytes per thread and stage: 32 (BM 64) or 8 (BM 16)
  constexpr int kPA = 4;                 // A stages in flight in registers
  constexpr int kPB = 2;                 // B steps in flight
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][BM * kA8Row];
  __shared__ uint32_t s_as[2][BM];  // the 4 scale bytes of each row and stage

  // XCD-aware block order (block_tile)
  int ti, bx;
  if (!block_tile(p.weight_major, p.tiles[0], &ti, &bx)) return;
  const int e = __builtin_amdgcn_readfirstlane(p.tiles[1 + 3 * ti]);
  const int r0 = __builtin_amdgcn_readfirstlane(p.tiles[2 + 3 * ti]);
  const int r1 = __builtin_amdgcn_readfirstlane(p.tiles[3 + 3 * ti]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = bx * a8_block_cols<MODE>();
  const int nk = p.K / kA8K;

  // A staging: row tid / kTPR, bytes (tid % kTPR) * kBPT ..; the row's scale
  // dword by its first thread.  Rows past the bucket read zeros (offset past
  // the end of the buffer).
  const int arow = tid / kTPR, acol = (tid % kTPR) * kBPT;
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)p.K;
  const uint32_t s_bytes = (uint32_t)p.a_rows * (uint32_t)(p.K / 32);
  uint32_t a_off = a_bytes, s_off = s_bytes;
  if (r0 + arow < r1) {
    const int src = p.row_token ? p.row_token[r0 + arow] : r0 + arow;
    a_off = (uint32_t)src * (uint32_t)p.K + (uint32_t)acol;
    s_off = (uint32_t)src * (uint32_t)(p.K / 32);
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.aq, a_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.as, s_bytes);
  struct AStg {
    uint32_t v[kBPT / 4];
    uint32_t sc;
  };
  auto a_load = [&](AStg &st, int it) {
    const uint32_t ko = (uint32_t)it * kA8K;
    if constexpr (kBPT == 64) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const u32x4_t x = buf_u128(ra, a_off + ko + 16 * q, 0);
        st.v[4 * q] = x.x, st.v[4 * q + 1] = x.y, st.v[4 * q + 2] = x.z, st.v[4 * q + 3] = x.w;
      }
    } else if constexpr (kBPT == 32) {
      const u32x4_t x0 = buf_u128(ra, a_off + ko, 0), x1 = buf_u128(ra, a_off + ko + 16, 0);
      st.v[0] = x0.x, st.v[1] = x0.y, st.v[2] = x0.z, st.v[3] = x0.w;
      st.v[4] = x1.x, st.v[5] = x1.y, st.v[6] = x1.z, st.v[7] = x1.w;
    } else {
      const u32x2_t x0 = buf_u64(ra, a_off + ko, 0);
      st.v[0] = x0.x, st.v[1] = x0.y;
    }
    st.sc = buf_u32(rs, s_off + ko / 32, 0);
  };
  auto a_store = [&](const AStg &st, int buf) {
    uint8_t *dst = &s_a[buf][arow * kA8Row + acol];
    if constexpr (kBPT == 64) {
#pragma unroll
      for (int q = 0; q < 4; q++)
        *reinterpret_cast<uint4 *>(dst + 16 * q) =
            make_uint4(st.v[4 * q], st.v[4 * q + 1], st.v[4 * q + 2], st.v[4 * q + 3]);
    } else if constexpr (kBPT == 32) {
      *reinterpret_cast<uint4 *>(dst) = make_uint4(st.v[0], st.v[1], st.v[2], st.v[3]);
      *reinterpret_cast<uint4 *>(dst + 16) = make_uint4(st.v[4], st.v[5], st.v[6], st.v[7]);
    } else {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(st.v[0], st.v[1]);
    }
    if (tid % kTPR == 0) s_as[buf][arow] = st.sc;
  };

  // this lane's weight rows, one per column block (gate/up: blocks 0, 1 gate
  // rows, 2, 3 the up rows of the same columns)
  constexpr int kWaveCols = MODE == kModeGateUp ? 32 : 64;
  int wrow[NB];
  const WView *wv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    if constexpr (MODE == kModeGateUp) {
      wrow[nb] = n0 + kWaveCols * wave + 16 * (nb % 2) + lr;
      wv[nb] = nb < 2 ? &p.w0 : &p.w1;
    } else {
      wrow[nb] = n0 + kWaveCols * wave + 16 * nb + lr;
      wv[nb] = &p.w0;
    }
  }
  const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_MXFP4, p.w0.N, p.w0.K);
  const uint32_t sb = (uint32_t)expert_scale_bytes(MOE_FMT_MXFP4, p.w0.N, p.w0.K);
  struct BStg {
    uint32_t q[NB][4];
    uint32_t sc[NB];
  };
  auto b_load = [&](BStg &st, int it) {
    const uint32_t k0 = (uint32_t)it * kA8K + 32u * (uint32_t)lg;
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(wv[nb]->data + (size_t)e * db, db);
      const __amdgpu_buffer_rsrc_t rsc = make_rsrc(wv[nb]->scales + (size_t)e * sb, sb);
      const u32x4_t v = buf_u128(rd, (uint32_t)wrow[nb] * (uint32_t)(p.K / 2) + k0 / 2, 0);
      st.q[nb][0] = v.x, st.q[nb][1] = v.y, st.q[nb][2] = v.z, st.q[nb][3] = v.w;
      st.sc[nb] = buf_u8(rsc, (uint32_t)wrow[nb] * (uint32_t)(p.K / 32) + k0 / 32, 0);
    }
  };

  AStg sa[kPA];
  BStg sbq[kPB];
#pragma unroll
  for (int u = 0; u < kPA; u++) a_load(sa[u], min(u, nk - 1));
#pragma unroll
  for (int u = 0; u < kPB; u++) b_load(sbq[u], min(u, nk - 1));
  a_store(sa[0], 0);
  a_load(sa[0], min(kPA, nk - 1));
  __syncthreads();

  const int m_active = (r1 - r0 + 15) >> 4;
  f32x4a_t acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[m][nb] = (f32x4a_t){0.0f, 0.0f, 0.0f, 0.0f};

  // one K step; the stage rings are indexed by compile-time slots, so the
  // loop body covers lcm(kPA, kPB) = 4 steps (K % 512 == 0)
  auto step = [&](int it, int ua, int ub) {
    const int buf = it & 1;
    const uint8_t *A = s_a[buf];
    i32x8_t af[MB];
    uint32_t asc[MB];
#pragma unroll
    for (int m = 0; m < MB; m++) {
      const uint8_t *row = A + (16 * m + lr) * kA8Row;
      const uint4 x0 = *reinterpret_cast<const uint4 *>(row + 16 * lg);
      const uint4 x1 = *reinterpret_cast<const uint4 *>(row + 64 + 16 * lg);
      af[m] = (i32x8_t){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                        (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      asc[m] = (s_as[buf][16 * m + lr] >> (8 * lg)) & 0xFFu;
    }
    BStg &bq = sbq[ub];
#pragma unroll
    for (int m = 0; m < MB; m++) {
      if (MB > 1 && m >= m_active) continue;
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const i32x8_t bfrag = {(int)bq.q[nb][0], (int)bq.q[nb][1], (int)bq.q[nb][2],
                               (int)bq.q[nb][3], 0, 0, 0, 0};
        acc[m][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[m], bfrag, acc[m][nb], 0, 4, 0, (int)asc[m], 0, (int)bq.sc[nb]);
      }
    }
    b_load(bq, min(it + kPB, nk - 1));
    // A: stage it + 1 into the other buffer, refill its slot
    a_store(sa[ua], buf ^ 1);
    a_load(sa[ua], min(it + 1 + kPA, nk - 1));
    __syncthreads();
  };
  for (int it0 = 0; it0 < nk; it0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; u++) step(it0 + u, (u + 1) % kPA, u % kPB);
  }

  // result register i of the lane: row 16 m + 4 (lane / 16) + i, column lane % 16
#pragma unroll
  for (int m = 0; m < MB; m++) {
    if (m >= m_active) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = r0 + 16 * m + 4 * lg + i;
      if constexpr (MODE == kModeGateUp) {
        float a[2];
        a[0] = silu_mul(acc[m][0][i], acc[m][2][i]);
        a[1] = silu_mul(acc[m][1][i], acc[m][3][i]);
        // the row's 32 columns of this wave are one MX-FP8 group: the 16
        // lanes of this lane group hold them
        float amax = fmaxf(fabsf(a[0]), fabsf(a[1]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const uint32_t e8 = mx8_scale_byte(amax);
        const int sh = 127 - (int)e8;
        if (r < r1) {
          const size_t base = (size_t)r * p.N + n0 + kWaveCols * wave;
#pragma unroll
          for (int c = 0; c < 2; c++)
            p.out_q[base + 16 * c + lr] =
                (uint8_t)(amax > 0.0f ? e4m3_code(__builtin_ldexpf(a[c], sh)) : 0u);
          if (p.a_f32) {
#pragma unroll
            for (int c = 0; c < 2; c++) p.a_f32[base + 16 * c + lr] = a[c];
          }
          if (lr == 0) p.out_s[(size_t)r * (p.N / 32) + (n0 + kWaveCols * wave) / 32] = (uint8_t)e8;
        }
      } else {
        if (r < r1) {
#pragma unroll
          for (int nb = 0; nb < NB; nb++)
            p.y_out[(size_t)r * p.N + n0 + kWaveCols * wave + 16 * nb + lr] = acc[m][nb][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tiles of BM = 128 or 192 rows with every operand moved into LDS by direct
// loads (as the dense bf16 GEMM).  A block of 8 waves computes BM bucket rows
// of one expert against 256 weight rows: wave (h, c) = (w / 4, w % 4) takes
// rows BM/2 h + [0, BM/2) and the columns of k_gemm_a8's wave c (gate/up:
// columns 32 c + [0, 32) of gate and of up, one MX-FP8 scale group; down:
// outputs 64 c + [0, 64)), BM/32 x 4 accumulators of 16 x 16, which stay in
// VGPRs at two waves per SIMD.  Each weight byte is staged once per tile: with
// 192 rows a bucket of up to 192 rows (prefill 4096: 128 +- 11) reads its
// expert's weights once.  Three K stages of 128 in LDS:
//   A codes, BM rows x 128 bytes, 16-byte chunks XOR-swizzled by
//     (row / 2) % 8; the MFMA's A lane (row r, lane group g) reads chunks g
//     and 4 + g of its row;
//   B nibbles, 256 rows x 64 bytes stored chunk-major (chunk g of every row,
//     then chunk g + 1), so the 16 lanes of a lane group read consecutive
//     16-byte slots; B lane (column n, group g) reads chunk g of row n;
//   the E8M0 scale dwords of A and B rows (4 k-blocks of 32 per stage).
// Every wave issues the same direct loads per stage, so one vmcnt immediate
// serves all: BM/64 runs of A, 2 runs of B, and the scales (128: one load,
// 32 A rows on waves 0-3, 64 B rows on waves 4-7; 192: 24 A rows and 32 B
// rows on every wave).  The loop is compiled once per count of live 16-row
// blocks of the wave's half (0, 2, 4, or 6 with 192 rows; a wave with none
// still loads and keeps the barriers).
// ---------------------------------------------------------------------------
constexpr int kA8DmaThreads = 512;

template <int MODE, int BM>
__global__ __launch_bounds__(kA8DmaThreads, 1) void k_a8_dma(A8Args p) {
  static_assert(BM == 128 || BM == 192, "tile rows");
  constexpr int NB = 4, kStg = 3, kWB = 256;
  constexpr int RH = BM / 2, MB = RH / 16;   // rows per wave half, 16-row blocks
  constexpr int kAR = BM / 64;               // A runs (8 rows of 128 bytes) per wave
  constexpr int kAB = kA8K, kBB = kA8K / 2;  // A and B bytes per row and stage
  // direct loads per wave and stage: A runs, 2 B runs, and the scales (128:
  // one load, A rows on waves 0-3, B rows on 4-7; 192: an A and a B load on
  // every wave)
  constexpr int kDma = kAR + 2 + (BM == 128 ? 1 : 2);
  __shared__ __attribute__((aligned(16))) uint8_t s_a[kStg][BM * kAB];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[kStg][kWB * kBB];
  __shared__ __attribute__((aligned(16))) uint32_t s_as[kStg][BM];
  __shared__ __attribute__((aligned(16))) uint32_t s_bs[kStg][kWB];

  int ti, bx;
  if (!block_tile(p.weight_major, p.tiles[0], &ti, &bx)) return;
  const int e = __builtin_amdgcn_readfirstlane(p.tiles[1 + 3 * ti]);
  const int r0 = __builtin_amdgcn_readfirstlane(p.tiles[2 + 3 * ti]);
  const int r1 = __builtin_amdgcn_readfirstlane(p.tiles[3 + 3 * ti]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wh = wave >> 2, wc = wave & 3;  // row half, column group
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = bx * a8_block_cols<MODE>();
  const int nk = p.K / kA8K;
  const uint32_t ks = (uint32_t)(p.K / 32);  // scale bytes per row

  // A: the source row of bucket row r (rows past the bucket repeat its last
  // row; their results are not stored)
  auto a_src = [&](int row) {
    const int r = min(r0 + row, r1 - 1);
    return p.row_token ? p.row_token[r] : r;
  };
  const i32x4r_t ra = rsrc_words(p.aq, (uint32_t)p.a_rows * (uint32_t)p.K);
  const i32x4r_t ras = rsrc_words(p.as, (uint32_t)p.a_rows * ks);
  const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_MXFP4, p.w0.N, p.w0.K);
  const uint32_t sb = (uint32_t)expert_scale_bytes(MOE_FMT_MXFP4, p.w0.N, p.w0.K);
  const i32x4r_t rb0 = rsrc_words(p.w0.data + (size_t)e * db, db);
  const i32x4r_t rb1 = rsrc_words(p.w1.data + (size_t)e * db, db);
  const i32x4r_t rs0 = rsrc_words(p.w0.scales + (size_t)e * sb, sb);
  const i32x4r_t rs1 = rsrc_words(p.w1.scales + (size_t)e * sb, sb);
  // weight row of LDS B row b (gate/up: rows below 128 gate, the rest up)
  auto w_row = [&](int b) { return n0 + (MODE == kModeGateUp ? (b & 127) : b); };

  // A runs kAR w + u (rows 8 j + lane / 8); B runs 2w, 2w + 1: run j is chunk
  // j / 4 of rows 64 (j % 4) + lane.  Scale loads, 128: waves 0-3 A rows
  // 32 w + lane (lanes < 32), waves 4-7 B rows 64 (w - 4) + lane; 192: A rows
  // 24 w + lane (lanes < 24) and B rows 32 w + lane (lanes < 32)
  uint32_t avo[kAR], bvo[2], svo, svo_b = 0;
#pragma unroll
  for (int u = 0; u < kAR; u++) {
    const int j = kAR * wave + u;
    const int row = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    avo[u] = (uint32_t)a_src(row) * (uint32_t)p.K + 16u * (uint32_t)c;
  }
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int j = 2 * wave + u;
    bvo[u] = (uint32_t)w_row(64 * (j & 3) + lane) * (uint32_t)(p.K / 2) + 16u * (uint32_t)(j >> 2);
  }
  bool s_up;  // this wave's B scale rows are up rows (128..255)
  if constexpr (BM == 128) {
    if (wave < 4)
      svo = (uint32_t)a_src(32 * wave + (lane & 31)) * ks;
    else
      svo = (uint32_t)w_row(64 * (wave - 4) + lane) * ks;
    s_up = MODE == kModeGateUp && wave >= 6;
  } else {
    svo = (uint32_t)a_src(24 * wave + min(lane, 23)) * ks;
    svo_b = (uint32_t)w_row(32 * wave + (lane & 31)) * ks;
    s_up = MODE == kModeGateUp && wave >= 4;
  }

  auto issue = [&](int it) {
    const int buf = it % kStg;
    const uint32_t ka = (uint32_t)it * kAB, kb = (uint32_t)it * kBB, kc = (uint32_t)it * 4u;
#pragma unroll
    for (int u = 0; u < kAR; u++)
      lds_load16(ra, lds_offset(&s_a[buf][(kAR * wave + u) * 1024]), avo[u] + ka);
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int j = 2 * wave + u;
      lds_load16(MODE == kModeGateUp && (j & 3) >= 2 ? rb1 : rb0,
                 lds_offset(&s_b[buf][(j >> 2) * (kWB * 16) + (j & 3) * 1024]), bvo[u] + kb);
    }
    if constexpr (BM == 128) {
      if (wave < 4) {
        if (lane < 32) lds_load4(ras, lds_offset(&s_as[buf][32 * wave]), svo + kc);
      } else {
        lds_load4(s_up ? rs1 : rs0, lds_offset(&s_bs[buf][64 * (wave - 4)]), svo + kc);
      }
    } else {
      if (lane < 24) lds_load4(ras, lds_offset(&s_as[buf][24 * wave]), svo + kc);
      if (lane < 32) lds_load4(s_up ? rs1 : rs0, lds_offset(&s_bs[buf][32 * wave]), svo_b + kc);
    }
  };

  f32x4a_t acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[m][nb] = (f32x4a_t){0.0f, 0.0f, 0.0f, 0.0f};

  issue(0);
  if (nk > 1) issue(1);
  if (nk > 1)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  // live 16-row blocks of this wave's half
  const int m_active = min(max((r1 - r0 - RH * wh + 15) >> 4, 0), MB);
  auto kloop = [&](auto ma_c) {
    constexpr int MA = decltype(ma_c)::value;
    for (int it = 0; it < nk; it++) {
      if (it + 2 < nk) issue(it + 2);
      if constexpr (MA > 0) {
        const int buf = it % kStg;
        const uint8_t *A = s_a[buf];
        const uint8_t *B = s_b[buf];
        i32x8_t bfr[NB];
        int bsc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          const int b = MODE == kModeGateUp ? (nb < 2 ? 0 : 128) + 32 * wc + 16 * (nb & 1) + lr
                                            : 64 * wc + 16 * nb + lr;
          const uint4 v = *reinterpret_cast<const uint4 *>(B + lg * (kWB * 16) + b * 16);
          bfr[nb] = (i32x8_t){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          bsc[nb] = (int)((s_bs[buf][b] >> (8 * lg)) & 0xFFu);
        }
#pragma unroll
        for (int m = 0; m < MA; m++) {
          const int row = RH * wh + 16 * m + lr;
          const uint8_t *ar = A + row * kAB;
          const int sw = (row >> 1) & 7;
          const uint4 x0 = *reinterpret_cast<const uint4 *>(ar + 16 * (lg ^ sw));
          const uint4 x1 = *reinterpret_cast<const uint4 *>(ar + 16 * ((4 + lg) ^ sw));
          const i32x8_t af = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                              (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          const int asc = (int)((s_as[buf][row] >> (8 * lg)) & 0xFFu);
#pragma unroll
          for (int nb = 0; nb < NB; nb++)
            acc[m][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af, bfr[nb], acc[m][nb], 0, 4, 0, asc, 0, bsc[nb]);
        }
      }
      if (it + 1 < nk) {
        if (it + 2 < nk)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
      }
    }
  };
  if (m_active == 0)
    kloop(std::integral_constant<int, 0>{});
  else if (m_active <= 2)
    kloop(std::integral_constant<int, 2>{});
  else if (MB == 4 || m_active <= 4)
    kloop(std::integral_constant<int, 4>{});
  else
    kloop(std::integral_constant<int, MB>{});

  // result register i of the lane: row 16 m + 4 (lane / 16) + i of the half,
  // column lane % 16
  constexpr int kWaveCols = MODE == kModeGateUp ? 32 : 64;
#pragma unroll
  for (int m = 0; m < MB; m++) {
    if (m >= m_active) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = r0 + RH * wh + 16 * m + 4 * lg + i;
      if constexpr (MODE == kModeGateUp) {
        float a[2];
        a[0] = silu_mul(acc[m][0][i], acc[m][2][i]);
        a[1] = silu_mul(acc[m][1][i], acc[m][3][i]);
        // the row's 32 columns of this wave are one MX-FP8 group: the 16
        // lanes of this lane group hold them
        float amax = fmaxf(fabsf(a[0]), fabsf(a[1]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const uint32_t e8 = mx8_scale_byte(amax);
        const int sh = 127 - (int)e8;
        if (r < r1) {
          const size_t base = (size_t)r * p.N + n0 + kWaveCols * wc;
#pragma unroll
          for (int c = 0; c < 2; c++)
            p.out_q[base + 16 * c + lr] =
                (uint8_t)(amax > 0.0f ? e4m3_code(__builtin_ldexpf(a[c], sh)) : 0u);
          if (p.a_f32) {
#pragma unroll
            for (int c = 0; c < 2; c++) p.a_f32[base + 16 * c + lr] = a[c];
          }
          if (lr == 0) p.out_s[(size_t)r * (p.N / 32) + (n0 + kWaveCols * wc) / 32] = (uint8_t)e8;
        }
      } else {
        if (r < r1) {
#pragma unroll
          for (int nb = 0; nb < NB; nb++)
            p.y_out[(size_t)r * p.N + n0 + kWaveCols * wc + 16 * nb + lr] = acc[m][nb][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool a8_supported(int H, int I, const WView &gate, const WView &up, const WView &down) {
  return gate.fmt == MOE_FMT_MXFP4 && up.fmt == MOE_FMT_MXFP4 && down.fmt == MOE_FMT_MXFP4 &&
         H % 512 == 0 && I % 512 == 0;
}

size_t a8_ws_bytes(int T, int H, int I, int n_rows) {
  auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
  return up((size_t)T * H) + up((size_t)T * H / 32) + up((size_t)n_rows * I) +
         up((size_t)n_rows * I / 32);
}

void a8_layout(int T, int H, int I, int n_rows, size_t *codes_off, size_t *scales_off) {
  auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
  *codes_off = up((size_t)T * H) + up((size_t)T * H / 32);
  *scales_off = *codes_off + up((size_t)n_rows * I);
}

namespace {

template <int BM>
hipError_t a8_bm(const WView &gate, const WView &up, const WView &down, int H, int I, int T,
                 const int32_t *offsets, const int32_t *sorted_token, int n_rows, int32_t *tiles,
                 const uint8_t *xq, const uint8_t *xs, uint8_t *aq, uint8_t *as, float *a_trace,
                 float *y, hipStream_t s, void (*mark)(void *, const char *), void *mark_ctx,
                 const char *const names[3]) {
  const int E = offsets ? gate.E : 0;
  // tiles: sum over the active experts of ceil(rows / BM) <= n_rows / BM + the
  // active count, which is at most min(E, n_rows) (blocks past the real count
  // exit at once, but each still takes a slot and a load)
  const int max_tiles = ((n_rows + BM - 1) / BM + std::min(E, n_rows) + 7) / 8 * 8;
  if (mark) mark(mark_ctx, names[0]);
  hipError_t err = launch_tile_list(E, n_rows, BM, offsets, tiles, s);
  if (err != hipSuccess) return err;

  A8Args g{};
  g.K = H, g.N = I, g.w0 = gate, g.w1 = up, g.aq = xq, g.as = xs, g.a_rows = T;
  g.row_token = offsets ? sorted_token : nullptr;
  g.tiles = tiles, g.out_q = aq, g.out_s = as, g.a_f32 = a_trace;
  g.weight_major = !offsets && (I / a8_block_cols<kModeGateUp>()) % 8 == 0 && max_tiles >= 16;
  if (mark) mark(mark_ctx, names[1]);
  if constexpr (BM >= 128)
    err = launch(k_a8_dma<kModeGateUp, BM>, dim3(I / a8_block_cols<kModeGateUp>(), max_tiles),
                 dim3(kA8DmaThreads), s, g);
  else
    err = launch(k_gemm_a8<kModeGateUp, BM>, dim3(I / a8_block_cols<kModeGateUp>(), max_tiles),
                 dim3(kA8Threads), s, g);
  if (err != hipSuccess) return err;

  A8Args d{};
  d.K = I, d.N = H, d.w0 = down, d.w1 = down, d.aq = aq, d.as = as, d.a_rows = n_rows;
  d.tiles = tiles, d.y_out = y;
  d.weight_major = !offsets && (H / a8_block_cols<kModeDown>()) % 8 == 0 && max_tiles >= 16;
  if (mark) mark(mark_ctx, names[2]);
  if constexpr (BM >= 128)
    return launch(k_a8_dma<kModeDown, BM>, dim3(H / a8_block_cols<kModeDown>(), max_tiles),
                  dim3(kA8DmaThreads), s, d);
  else
    return launch(k_gemm_a8<kModeDown, BM>, dim3(H / a8_block_cols<kModeDown>(), max_tiles),
                  dim3(kA8Threads), s, d);
}

}  // namespace

hipError_t launch_a8_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                         int T, const uint16_t *x, const int32_t *offsets,
                         const int32_t *sorted_token, int n_rows, int32_t *tiles, void *ws,
                         float *a_trace, float *y, hipStream_t s,
                         void (*mark)(void *, const char *), void *mark_ctx,
                         const char *const names[4]) {
  if (!a8_supported(H, I, gate, up, down) || n_rows < 1 || T < 1) return hipErrorInvalidValue;
  if ((size_t)T * H >= ((size_t)1 << 31) || (size_t)n_rows * I >= ((size_t)1 << 31))
    return hipErrorInvalidValue;
  auto up256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  size_t codes_off, scales_off;
  a8_layout(T, H, I, n_rows, &codes_off, &scales_off);
  uint8_t *w = static_cast<uint8_t *>(ws);
  uint8_t *xq = w;
  uint8_t *xs = xq + up256((size_t)T * H);
  uint8_t *aq = w + codes_off;
  uint8_t *as = w + scales_off;
  if (mark) mark(mark_ctx, names[3]);
  const long n8 = (long)T * (H / 8);
  hipError_t err =
      launch(k_mx8_quant, dim3((unsigned)((n8 + 255) / 256)), dim3(256), s, T, H, x, xq, xs);
  if (err != hipSuccess) return err;
  const int active = offsets ? (gate.E < n_rows ? gate.E : n_rows) : 1;
  // 192-row tiles from 112 rows per active expert: a bucket of up to 192 rows
  // (prefill 4096: 128 +- 11) is one tile, so each expert's weights stream
  // once instead of once more for the few rows past 128; 128-row tiles from
  // 96 rows: the weights stream about once per bucket rather than once per 64
  // rows
  if (n_rows >= 112 * active)
    return a8_bm<192>(gate, up, down, H, I, T, offsets, sorted_token, n_rows, tiles, xq, xs, aq,
                      as, a_trace, y, s, mark, mark_ctx, names);
  if (n_rows >= 96 * active)
    return a8_bm<128>(gate, up, down, H, I, T, offsets, sorted_token, n_rows, tiles, xq, xs, aq,
                      as, a_trace, y, s, mark, mark_ctx, names);
  if (n_rows >= 32 * active)
    return a8_bm<64>(gate, up, down, H, I, T, offsets, sorted_token, n_rows, tiles, xq, xs, aq,
                     as, a_trace, y, s, mark, mark_ctx, names);
  return a8_bm<16>(gate, up, down, H, I, T, offsets, sorted_token, n_rows, tiles, xq, xs, aq, as,
                   a_trace, y, s, mark, mark_ctx, names);
}

// MX-FP8 quantization alone (for tests of the quantizer)
hipError_t launch_mx8_quant(int rows, int K, const uint16_t *x, uint8_t *q, uint8_t *sc,
                            hipStream_t s) {
  if (K % 32 || rows < 0) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const long n8 = (long)rows * (K / 8);
  return launch(k_mx8_quant, dim3((unsigned)((n8 + 255) / 256)), dim3(256), s, rows, K, x, q, sc);
}

}  // namespace moe
