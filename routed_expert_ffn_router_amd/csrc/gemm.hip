// gemm.hip -- batched tokens: grouped per-expert GEMMs on the matrix cores.
//
// With several tokens per expert the expert FFN becomes a grouped GEMM (the
// ds4 pages: prefill amortises the expert weights over the batch --
// hysenlabs.com "SSD streaming"; matrix-instruction expert kernels on newer
// devices -- hysenlabs.com "Model support and quantization").  Each workgroup
// computes BM bucket rows of one expert against 256 weight rows (gate/up: 128
// gate + 128 up; down: 256 outputs), BM 16 or 64 by the rows per active
// expert, 128 for one dense expert.  Each of the 4 waves owns 64 weight rows for all BM rows and
// dequantizes them straight into MFMA operand registers -- every weight is
// decoded once per tile and never passes through LDS; only the activation
// rows (gathered tokens, or the SwiGLU output in bucket order) are staged in
// LDS and shared by the waves.  v_mfma_f32_16x16x32 throughout.
//
// K is walked in groups of 256 (one Q2K super-block, one VQ2 scale group),
// each cut into 4 stages of 64: a lane loads its weights once per group (the
// contiguous run of 64 it covers over the group's stages, see BGroup) and
// decodes one stage ahead of the matrix instructions that consume it.  The
// MFMA reduction slots are a relabelling of k; A and B use the same one.
//
// Operand precision: bf16 tokens x exact bf16 weights for MXFP4 and bf16
// gate/up; fp16 for VQ2 and Q2K gate/up (tokens converted exactly, weights
// rounded once to fp16) and for every down projection (the SwiGLU output in
// fp16).  Accumulation in fp32.
#include "gemv_core.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kBKs = 64;                  // K per stage
constexpr int kLdsRow = kBKs + 8;         // padded LDS row (16-bit elements): 144 bytes
constexpr int kLdsRowW = kLdsRow / 2;     // ... in dwords
constexpr int kGemmThreads = 256;
// MFMA column blocks (16 weight rows each) per wave
template <int FMT>
constexpr int col_blocks() { return 4; }

constexpr int kMinBM = 16;

enum { kOpBF16 = 0, kOpF16 = 1 };
enum { kModeGateUp = 0, kModeDown = 1 };

// output columns of one block (4 waves): gate/up a columns, down outputs
template <int MODE, int FMT>
constexpr int block_cols() { return MODE == kModeGateUp ? 32 * col_blocks<FMT>() : 64 * col_blocks<FMT>(); }

// tile list: tiles[0] = count; tile i = tiles[1 + 3i .. 3 + 3i] = {expert, r0, r1}
size_t gemm_tile_ints(int n_rows, int E) {
  return 1 + 3 * (size_t)((n_rows + kMinBM - 1) / kMinBM + E);
}

__global__ __launch_bounds__(1024) void k_tile_list(int E, int n_dense, int bm,
                                                     const int32_t *__restrict__ offsets,
                                                     int32_t *__restrict__ tiles) {
  __shared__ int s_tmp[16];
  if (!offsets) {  // one dense expert over rows [0, n_dense)
    const int n = (n_dense + bm - 1) / bm;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      tiles[1 + 3 * i] = 0;
      tiles[2 + 3 * i] = i * bm;
      tiles[3 + 3 * i] = min(n_dense, (i + 1) * bm);
    }
    if (threadIdx.x == 0) tiles[0] = n;
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (c + bm - 1) / bm;
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
      const int r0 = offsets[e] + t * bm;
      tiles[1 + 3 * pos] = e;
      tiles[2 + 3 * pos] = r0;
      tiles[3 + 3 * pos] = min(offsets[e + 1], r0 + bm);
    }
    base += tot;
  }
  if (threadIdx.x == 0) tiles[0] = base;
}

struct GemmArgs {
  int K, N;                  // reduction length; columns of the layer's output (I or H)
  WView w0, w1;              // gate and up, or down (w0 == w1)
  const uint16_t *x;         // gate/up: tokens [T][K] in the operand type (bf16 or fp16)
  const int32_t *row_token;  // gate/up: token of each bucket row (null: the row itself)
  const uint16_t *a16;       // down: fp16 SwiGLU output [n_rows][K]
  int a_rows;                // rows of x (gate/up: T) or of a16 (down: n_rows)
  const int32_t *tiles;
  int weight_major;          // tile order: weights-first (one dense expert) or rows-first
  int a_swap;                // gate/up: a_out in Q2K slot order (swap12 within each 4 columns)
  uint16_t *a_out;           // gate/up: fp16 [n_rows][N]
  float *y_out;              // down: fp32 [n_rows][N]
};

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) { return pack_h2(bf16_lo(v), bf16_hi(v)); }
// the slot of value i when each group of 4 is ordered (0, 2, 1, 3)
__device__ __forceinline__ int swap12(int i) { return (i & ~3) | ((i & 1) << 1) | ((i >> 1) & 1); }

// ---------------------------------------------------------------------------
// B: the weights of one row that a lane covers, raw bits -> operand pairs.
//
// K is cut into groups of 256 (one Q2K super-block, one VQ2 scale group) and
// each group into 4 stages.  Stage s of a group holds the columns 64 j + 16 s
// + [0, 16), j = 0..3, and lane group g = lane / 16 takes chunk j = g: over
// the 4 stages of a group it covers the contiguous run 64 g + [0, 64) of its
// row, which it loads at once (VQ2: 16 bytes of codes and the group's scale;
// Q2K: 16 bytes of 2-bit codes, its 4 sub-blocks' scale bytes and d|dmin;
// MXFP4: 32 bytes and 2 scales).  bf16 weights (64 bytes a run) are loaded
// per stage instead.
// ---------------------------------------------------------------------------
template <int FMT, int OP>
struct BGroup {
  uint32_t q[FMT == MOE_FMT_MXFP4 ? 8 : 4];
  uint32_t s0, s1;  // VQ2: fp16 scale; Q2K: 4 scale/min bytes, d|dmin; MXFP4: 2 E8M0 bytes

  // k0: first column of the lane's run (a multiple of 64)
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k0) {
    const uint32_t db = (uint32_t)expert_data_bytes(FMT, w.N, w.K);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(w.data + (size_t)e * db, db);
    if constexpr (FMT == MOE_FMT_VQ2) {
      const uint32_t sb = (uint32_t)expert_scale_bytes(FMT, w.N, w.K);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
      const u32x4_t v = buf_u128(r, (uint32_t)row * (uint32_t)(w.K / 4) + (uint32_t)k0 / 4, 0);
      q[0] = v.x, q[1] = v.y, q[2] = v.z, q[3] = v.w;
      s0 = buf_u16(rs, ((uint32_t)row * (uint32_t)(w.K / 256) + (uint32_t)k0 / 256) * 2u, 0);
    } else if constexpr (FMT == MOE_FMT_Q2K) {
      const uint32_t blk = ((uint32_t)row * (uint32_t)(w.K / 256) + (uint32_t)k0 / 256) * kQ2KBytes;
      const uint32_t j = (k0 % 256) / 16;  // first of the 4 sub-blocks
      // (84-byte blocks keep only 4-byte alignment: dword loads)
      q[0] = buf_u32(r, blk + 16 + 4 * j, 0);
      q[1] = buf_u32(r, blk + 20 + 4 * j, 0);
      q[2] = buf_u32(r, blk + 24 + 4 * j, 0);
      q[3] = buf_u32(r, blk + 28 + 4 * j, 0);
      s0 = buf_u32(r, blk + j, 0);
      s1 = buf_u32(r, blk + 80, 0);
    } else {  // MXFP4
      const uint32_t sb = (uint32_t)expert_scale_bytes(FMT, w.N, w.K);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
      const uint32_t vo = (uint32_t)row * (uint32_t)(w.K / 2) + (uint32_t)k0 / 2;
      const u32x4_t a = buf_u128(r, vo, 0), b = buf_u128(r, vo + 16, 0);
      q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w, q[4] = b.x, q[5] = b.y, q[6] = b.z, q[7] = b.w;
      s0 = buf_u16(rs, (uint32_t)row * (uint32_t)(w.K / 32) + (uint32_t)k0 / 32, 0);
    }
  }

  // stage S of the group: the run's weights 16 S .. 16 S + 15; out[i] holds
  // weights (2i, 2i + 1) of those as an OP pair (Q2K: in swap12 order)
  __device__ __forceinline__ void decode(int S, uint32_t (&out)[8], const uint2 *cb) const {
    if constexpr (FMT == MOE_FMT_VQ2) {
      // fp16 codebook integers (exact) times the fp16 scale, rounded once
      const f16x2_t d2 = {__builtin_bit_cast(_Float16, (uint16_t)s0),
                          __builtin_bit_cast(_Float16, (uint16_t)s0)};
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const uint2 v = cb[((q[S] >> (8 * c)) & 255u) * kNCopy];
        out[2 * c] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.x) * d2);
        out[2 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.y) * d2);
      }
    } else if constexpr (FMT == MOE_FMT_Q2K) {
      // w = (d sc) q - dmin m: the codes widened to E2M1 nibbles (q reads as
      // q/2) and converted with the scale 2 give q exactly as fp16 pairs;
      // one fused multiply-add with d sc and -dmin m (each rounded to fp16)
      // rounds the weight once.  Nibble order pairs weights (4b, 4b+2) and
      // (4b+1, 4b+3): the A operand is stored in that order (swap12).
      const uint32_t scm = (s0 >> (8 * S)) & 255u;
      const float d = f16_bits_to_f32(s1 & 0xFFFFu), dmin = f16_bits_to_f32(s1 >> 16);
      const float ds = d * (float)(scm & 15u), ms = dmin * (float)(scm >> 4);
      const f16x2_t ds2 = {(_Float16)ds, (_Float16)ds};
      const f16x2_t nms2 = {(_Float16)(-ms), (_Float16)(-ms)};
      const uint32_t x = q[S];
      const uint32_t nl = x & 0x33333333u, nh = (x >> 2) & 0x33333333u;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const f16x2_t p0 = __builtin_bit_cast(f16x2_t, q2_pair(nl, b));
        const f16x2_t p1 = __builtin_bit_cast(f16x2_t, q2_pair(nh, b));
        out[2 * b] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(p0, ds2, nms2));
        out[2 * b + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(p1, ds2, nms2));
      }
    } else {  // MXFP4: E2M1 x 2^(e - 127), converted with the scale applied
      const float sc = e8m0_to_f32((s0 >> (8 * (S / 2))) & 255u);
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint32_t v = q[2 * S + j];
        if constexpr (OP == kOpBF16) {
          out[4 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 0));
          out[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 1));
          out[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 2));
          out[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 3));
        } else {
          out[4 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, sc, 0));
          out[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, sc, 1));
          out[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, sc, 2));
          out[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, sc, 3));
        }
      }
    }
  }
};

// bf16 weights: one stage's 16 weights of the row (the run 64 g + 16 S + [0, 16))
template <int OP>
struct BStageBf16 {
  uint32_t q[8];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k) {
    const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_BF16, w.N, w.K);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(w.data + (size_t)e * db, db);
    const uint32_t vo = ((uint32_t)row * (uint32_t)w.K + (uint32_t)k) * 2u;
    const u32x4_t a = buf_u128(r, vo, 0), b = buf_u128(r, vo + 16, 0);
    q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w, q[4] = b.x, q[5] = b.y, q[6] = b.z, q[7] = b.w;
  }
  __device__ __forceinline__ void decode(uint32_t (&out)[8]) const {
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = OP == kOpF16 ? bf16x2_to_f16x2(q[i]) : q[i];
  }
};

// A stage (already in the operand type): BM rows x 64 LDS columns; thread t stages row t / (256 / BM) and
// the BM / 4 LDS columns from acol.  LDS column c of stage it holds
// k = kb(it) + 64 (c / 16) + c % 16 with kb(it) = 256 (it / 4) + 16 (it % 4),
// so a thread's columns are one run of 4 (BM 16) or runs of 16 (BM 64, 128)
// 64 apart in k.  Rows past the bucket read zeros (an offset past the buffer).
template <int MODE, int OP, int BM>
struct AStage {
  static constexpr int kCPT = BM / 4;   // columns per thread
  static constexpr int kDw = kCPT / 2;  // dwords per thread: 2, 8 or 16
  uint32_t raw[kDw];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int kb, int acol) {
    if constexpr (kCPT == 4) {
      const u32x2_t a = buf_u64(r, row_off + (uint32_t)(kb + 64 * (acol / 16) + acol % 16) * 2u, 0);
      raw[0] = a.x, raw[1] = a.y;
    } else {
#pragma unroll
      for (int q = 0; q < kCPT / 16; q++) {
        const uint32_t vo = row_off + (uint32_t)(kb + 64 * (acol / 16 + q)) * 2u;
        const u32x4_t a = buf_u128(r, vo, 0), b = buf_u128(r, vo + 16, 0);
        raw[8 * q] = a.x, raw[8 * q + 1] = a.y, raw[8 * q + 2] = a.z, raw[8 * q + 3] = a.w;
        raw[8 * q + 4] = b.x, raw[8 * q + 5] = b.y, raw[8 * q + 6] = b.z, raw[8 * q + 7] = b.w;
      }
    }
  }
  __device__ __forceinline__ void store(uint32_t *dst) const {
    if constexpr (kDw == 2) {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(raw[0], raw[1]);
    } else {
      uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
      for (int i = 0; i < kDw / 4; i++)
        d4[i] = make_uint4(raw[4 * i], raw[4 * i + 1], raw[4 * i + 2], raw[4 * i + 3]);
    }
  }
};

// the bf16 weight column a lane of k group g loads in stage it
__device__ __forceinline__ int a_k_b16(int it, int g) { return 256 * (it >> 2) + 64 * g + 16 * (it & 3); }

template <int OP>
__device__ __forceinline__ f32x4v_t mfma16(uint4 a, uint4 b, f32x4v_t c) {
  if constexpr (OP == kOpBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// the grouped GEMM: grid.x = column blocks of the layer, grid.y = bucket tiles
// ---------------------------------------------------------------------------
template <int MODE, int FMT, int OP, int BM>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs p) {
  constexpr int MB = BM / 16;  // MFMA row blocks
  constexpr int NB = col_blocks<FMT>();
  constexpr int kPA = 4;       // A stages in flight (one group)
  constexpr bool kGroupB = FMT != MOE_FMT_BF16;
  __shared__ uint32_t s_a[2][BM * kLdsRowW];
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  // XCD-aware order: workgroups go round-robin to the 8 XCDs (linear id b on
  // XCD b % 8).  Grouped experts (a tile or two each): XCD x takes tiles x,
  // x + 8, ... and walks all column blocks of a tile back to back, so its L2
  // fetches each tile's rows once.  One dense expert over many tiles: XCD x
  // takes column blocks x, x + 8, ... and walks all tiles of one back to back,
  // so its L2 keeps that block of weights.  (grid.y, and grid.x in the dense
  // order, are multiples of 8.)
  const uint32_t nbx = gridDim.x, nby = gridDim.y;
  const uint32_t bid = blockIdx.y * nbx + blockIdx.x;
  const uint32_t jx = bid >> 3;
  const int ti = p.weight_major ? (int)(jx % nby) : (int)((jx / nbx) * 8 + (bid & 7));
  const int bx = p.weight_major ? (int)((jx / nby) * 8 + (bid & 7)) : (int)(jx % nbx);
  if (ti >= p.tiles[0]) return;
  const int e = __builtin_amdgcn_readfirstlane(p.tiles[1 + 3 * ti]);
  const int r0 = __builtin_amdgcn_readfirstlane(p.tiles[2 + 3 * ti]);
  const int r1 = __builtin_amdgcn_readfirstlane(p.tiles[3 + 3 * ti]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;  // MFMA row/column within a block; k group
  const int n0 = bx * block_cols<MODE, FMT>();

  if constexpr (FMT == MOE_FMT_VQ2) {  // codebook as exact fp16 integers, kNCopy copies
    const uint32_t cw = reinterpret_cast<const uint32_t *>(p.w0.codebook)[tid];
    uint32_t h[2];
#pragma unroll
    for (int j = 0; j < 2; j++)
      h[j] = pack_h2((float)(int)(int8_t)((cw >> (16 * j)) & 255u),
                     (float)(int)(int8_t)((cw >> (16 * j + 8)) & 255u));
#pragma unroll
    for (int j = 0; j < kNCopy; j++)  // a different copy per lane and step: no bank conflicts
      s_cb[tid * kNCopy + ((j + tid) & (kNCopy - 1))] = make_uint2(h[0], h[1]);
  }

  // A staging: row tid / (256 / BM), LDS columns acol .. acol + BM / 4 - 1
  constexpr int kTPR = kGemmThreads / BM;  // threads per A row
  constexpr int kCPT = kBKs / kTPR;        // columns per thread
  const int arow = tid / kTPR, acol = (tid % kTPR) * kCPT;
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)p.K * 2u;
  uint32_t a_off = a_bytes;  // past the end: zeros
  if (r0 + arow < r1) {
    const int src = (MODE == kModeGateUp && p.row_token) ? p.row_token[r0 + arow] : r0 + arow;
    a_off = (uint32_t)src * (uint32_t)p.K * 2u;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(MODE == kModeGateUp ? p.x : p.a16, a_bytes);
  const int nk = p.K / kBKs;  // stages, a multiple of 4 (K % 256 == 0)
  const int ng = nk / 4;      // groups
  auto a_kb = [&](int it) { return 256 * (it >> 2) + 16 * (it & 3); };

  // this lane's weight rows, one per column block nb: gate/up: the first half
  // of the blocks gate rows, the second half the up rows of the same a columns
  constexpr int kWaveCols = MODE == kModeGateUp ? 8 * NB : 16 * NB;  // output columns per wave
  int wrow[NB];
  const WView *wv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    if constexpr (MODE == kModeGateUp) {
      wrow[nb] = n0 + kWaveCols * wave + 16 * (nb % (NB / 2)) + lr;
      wv[nb] = nb < NB / 2 ? &p.w0 : &p.w1;
    } else {
      wrow[nb] = n0 + kWaveCols * wave + 16 * nb + lr;
      wv[nb] = &p.w0;
    }
  }

  AStage<MODE, OP, BM> sa[kPA];
  BGroup<FMT, OP> gb0[NB], gb1[NB];  // group ring (quantized formats)
  BStageBf16<OP> sb16[2][NB];        // stage ring (bf16): two stages ahead
#pragma unroll
  for (int u = 0; u < kPA; u++) sa[u].load(ra, a_off, a_kb(u), acol);
  if constexpr (kGroupB) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) gb0[nb].load(*wv[nb], e, wrow[nb], 64 * lg);
  } else {
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int nb = 0; nb < NB; nb++) sb16[u][nb].load(*wv[nb], e, wrow[nb], a_k_b16(u, lg));
  }
  sa[0].store(&s_a[0][arow * kLdsRowW + acol / 2]);
  // stages past the end re-read the last one (never used; keeps the loads unconditional)
  sa[0].load(ra, a_off, a_kb(min(kPA, nk - 1)), acol);
  __syncthreads();  // A stage 0 and the codebook

  const int m_active = (r1 - r0 + 15) >> 4;  // row blocks holding bucket rows
  f32x4v_t acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[m][nb] = (f32x4v_t){0.0f, 0.0f, 0.0f, 0.0f};
  const uint2 *cb = s_cb + (lane & (kNCopy - 1));

  // B operands of two stages: the MFMAs of stage `it` read bp[it & 1] while
  // stage it + 1 is decoded into the other slot, so the decode's LDS lookups
  // and VALU work overlap the matrix instructions instead of preceding them
  uint32_t bp[2][NB][8];
  if constexpr (kGroupB) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) gb0[nb].decode(0, bp[0][nb], cb);
  }

  // one group: 4 stages; its B comes from `cur`, the next group's goes to `nxt`
  auto group = [&](int G, BGroup<FMT, OP>(&cur)[NB], BGroup<FMT, OP>(&nxt)[NB]) {
    if constexpr (kGroupB) {
      const int gn = min(G + 1, ng - 1);
#pragma unroll
      for (int nb = 0; nb < NB; nb++) nxt[nb].load(*wv[nb], e, wrow[nb], 256 * gn + 64 * lg);
    }
#pragma unroll
    for (int S = 0; S < 4; S++) {
      const int it = 4 * G + S;
      // this stage's A fragments, all read before the matrix instructions
      const uint32_t *A = s_a[it & 1];
      uint4 af[2][MB];
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int m = 0; m < MB; m++)
          af[t][m] =
              *reinterpret_cast<const uint4 *>(&A[(16 * m + lr) * kLdsRowW + (16 * lg + 8 * t) / 2]);
      if constexpr (kGroupB) {
        // the next stage: stage S + 1 of this group, or stage 0 of the next
        // (past the last group: a decode of the clamped reload, never used)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          if (S < 3)
            cur[nb].decode(S + 1, bp[(S + 1) & 1][nb], cb);
          else
            nxt[nb].decode(0, bp[(S + 1) & 1][nb], cb);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) sb16[S & 1][nb].decode(bp[S & 1][nb]);
        const int st = min(it + 2, nk - 1);
#pragma unroll
        for (int nb = 0; nb < NB; nb++) sb16[S & 1][nb].load(*wv[nb], e, wrow[nb], a_k_b16(st, lg));
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
#pragma unroll
        for (int m = 0; m < MB; m++) {
          if (MB > 1 && m >= m_active) continue;
#pragma unroll
          for (int nb = 0; nb < NB; nb++) {
            const uint32_t *b = bp[S & 1][nb];
            const uint4 bf = make_uint4(b[4 * t], b[4 * t + 1], b[4 * t + 2], b[4 * t + 3]);
            acc[m][nb] = mfma16<OP>(af[t][m], bf, acc[m][nb]);
          }
        }
      }
      // A: stage it + 1 into the other buffer, refill its slot
      const int an = (S + 1) & 3;
      sa[an].store(&s_a[(it + 1) & 1][arow * kLdsRowW + acol / 2]);
      sa[an].load(ra, a_off, a_kb(min(it + 1 + kPA, nk - 1)), acol);
      __syncthreads();
    }
  };
  for (int G = 0; G < ng; G += 2) {
    group(G, gb0, gb1);
    if (G + 1 < ng) group(G + 1, gb1, gb0);
  }

  // result register i of the lane: row 16 m + 4 (lane / 16) + i, column lane % 16
#pragma unroll
  for (int m = 0; m < MB; m++) {
    if (m >= m_active) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = r0 + 16 * m + 4 * lg + i;
      if (r >= r1) continue;
      if constexpr (MODE == kModeGateUp) {
#pragma unroll
        for (int c = 0; c < NB / 2; c++) {
          const float a = silu_mul(acc[m][c][i], acc[m][c + NB / 2][i]);
          const int col = n0 + kWaveCols * wave + 16 * c + lr;
          p.a_out[(size_t)r * p.N + (p.a_swap ? swap12(col) : col)] =
              __builtin_bit_cast(uint16_t, (_Float16)a);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
          p.y_out[(size_t)r * p.N + n0 + kWaveCols * wave + 16 * nb + lr] = acc[m][nb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dense and skinny (one expert, T <= 64 rows, bf16 weights: the shared expert
// of a small batch).  Block: 16 output columns; its 8 waves split K, each
// streaming its share of the 16 (gate/up: 16 + 16) weight rows straight into
// MFMA operands, A (the T rows) straight from global memory; the 8 partial
// tiles are summed in wave order through LDS, then the SwiGLU / output.
// ---------------------------------------------------------------------------
constexpr int kSkWaves = 8;

struct SkinnyArgs {
  int T, K, N;
  const uint16_t *w0, *w1;  // bf16 [N][K] (gate, up) or (down, -)
  const uint16_t *a;        // gate/up: bf16 x [T][K]; down: fp16 SwiGLU output [T][K]
  uint16_t *a_out;          // gate/up: fp16 [T][N]
  float *y_out;             // down: fp32 [T][N]
};

template <int MODE, int MB>
__global__ __launch_bounds__(64 * kSkWaves) void k_skinny(SkinnyArgs p) {
  constexpr int NB = MODE == kModeGateUp ? 2 : 1;  // gate + up, or down
  constexpr int OP = MODE == kModeGateUp ? kOpBF16 : kOpF16;
  constexpr int kPD = MB > 2 ? 2 : 4;              // stages in flight
  __shared__ f32x4v_t s_red[kSkWaves][MB][NB][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int c0 = blockIdx.x * 16;
  const int ns = p.K / kBKs, per = ns / kSkWaves, st0 = wave * per;  // ns % 8 == 0
  const uint32_t wbytes = (uint32_t)p.N * (uint32_t)p.K * 2u;
  const __amdgpu_buffer_rsrc_t rw0 = make_rsrc(p.w0, wbytes);
  const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(NB == 2 ? p.w1 : p.w0, wbytes);
  const uint32_t abytes = (uint32_t)p.T * (uint32_t)p.K * 2u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, abytes);
  const uint32_t wo = ((uint32_t)(c0 + lr) * (uint32_t)p.K + 16u * lg) * 2u;
  uint32_t ao[MB];
#pragma unroll
  for (int m = 0; m < MB; m++) {
    const int t = 16 * m + lr;
    ao[m] = t < p.T ? ((uint32_t)t * (uint32_t)p.K + 16u * lg) * 2u : abytes;  // past T: zeros
  }
  u32x4_t bw[kPD][NB][2], av[kPD][MB][2];
  auto load = [&](int slot, int st) {
    const uint32_t ko = (uint32_t)st * kBKs * 2u;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      bw[slot][0][h] = buf_u128(rw0, wo + ko + 16 * h, 0);
      if constexpr (NB == 2) bw[slot][1][h] = buf_u128(rw1, wo + ko + 16 * h, 0);
#pragma unroll
      for (int m = 0; m < MB; m++) av[slot][m][h] = buf_u128(ra, ao[m] + ko + 16 * h, 0);
    }
  };
  f32x4v_t acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[m][nb] = (f32x4v_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kPD; u++) load(u, st0 + min(u, per - 1));
  for (int i0 = 0; i0 < per; i0 += kPD) {
#pragma unroll
    for (int u = 0; u < kPD; u++) {
      if (i0 + u < per) {
#pragma unroll
        for (int t = 0; t < 2; t++) {
#pragma unroll
          for (int nb = 0; nb < NB; nb++) {
            const u32x4_t w = bw[u][nb][t];
            const uint4 bf = OP == kOpF16
                                 ? make_uint4(bf16x2_to_f16x2(w.x), bf16x2_to_f16x2(w.y),
                                              bf16x2_to_f16x2(w.z), bf16x2_to_f16x2(w.w))
                                 : make_uint4(w.x, w.y, w.z, w.w);
#pragma unroll
            for (int m = 0; m < MB; m++) {
              const u32x4_t x = av[u][m][t];
              acc[m][nb] = mfma16<OP>(make_uint4(x.x, x.y, x.z, x.w), bf, acc[m][nb]);
            }
          }
        }
        load(u, st0 + min(i0 + u + kPD, per - 1));
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++) s_red[wave][m][nb][lane] = acc[m][nb];
  __syncthreads();
  if (wave != 0) return;
  // result register i of the lane: row 16 m + 4 (lane / 16) + i, column c0 + lane % 16
#pragma unroll
  for (int m = 0; m < MB; m++) {
    f32x4v_t v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      v[nb] = s_red[0][m][nb][lane];
#pragma unroll
      for (int w = 1; w < kSkWaves; w++) v[nb] += s_red[w][m][nb][lane];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int t = 16 * m + 4 * lg + i;
      if (t >= p.T) continue;
      if constexpr (MODE == kModeGateUp)
        p.a_out[(size_t)t * p.N + c0 + lr] = __builtin_bit_cast(uint16_t, (_Float16)silu_mul(v[0][i], v[1][i]));
      else
        p.y_out[(size_t)t * p.N + c0 + lr] = v[0][i];
    }
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------

// bf16 tokens -> fp16 operands (round to nearest even; exact for every bf16
// value inside the fp16 normal range), once per call instead of once per
// column block of the gate/up GEMM.  SWAP: each group of 4 in swap12 order
// (the Q2K weights' slot order)
template <bool SWAP>
__global__ __launch_bounds__(256) void k_tokens_f16(long n8, const uint4 *__restrict__ x,
                                                     uint4 *__restrict__ x16) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = x[i];
  if constexpr (SWAP)
    x16[i] = make_uint4(pack_h2(bf16_lo(v.x), bf16_lo(v.y)), pack_h2(bf16_hi(v.x), bf16_hi(v.y)),
                        pack_h2(bf16_lo(v.z), bf16_lo(v.w)), pack_h2(bf16_hi(v.z), bf16_hi(v.w)));
  else
    x16[i] = make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
                        bf16x2_to_f16x2(v.w));
}

// K a multiple of 256 (whole Q2K / VQ2 groups; a whole number of register
// stages), output columns a multiple of the block's (128 a columns, 256 down)
hipError_t launch_tile_list(int E, int n_dense, int bm, const int32_t *offsets, int32_t *tiles,
                            hipStream_t s) {
  return launch(k_tile_list, dim3(1), dim3(1024), s, offsets ? E : 0, n_dense, bm, offsets, tiles);
}

bool gemm_supported(int H, int I, int fmt_gate, int fmt_down) {
  (void)fmt_gate, (void)fmt_down;
  return H >= 256 && I >= 256 && H % 256 == 0 && I % 256 == 0;
}

namespace {

// grid.x: the layer's output columns over the block's; grid.y: tiles
template <int MODE, int BM>
hipError_t gemm_fmt(const GemmArgs &a, int fmt, int op, int tiles, hipStream_t s) {
#define MOE_GEMM_CASE(F, O)                                                              \
  if (fmt == F && op == O) {                                                             \
    return launch(k_gemm<MODE, F, O, BM>, dim3(a.N / block_cols<MODE, F>(), tiles),      \
                  dim3(kGemmThreads), s, a);                                             \
  }
  MOE_GEMM_CASE(MOE_FMT_BF16, kOpBF16)
  MOE_GEMM_CASE(MOE_FMT_BF16, kOpF16)
  MOE_GEMM_CASE(MOE_FMT_VQ2, kOpF16)
  MOE_GEMM_CASE(MOE_FMT_Q2K, kOpF16)
  MOE_GEMM_CASE(MOE_FMT_MXFP4, kOpBF16)
  MOE_GEMM_CASE(MOE_FMT_MXFP4, kOpF16)
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

int gateup_op(int fmt) {
  return fmt == MOE_FMT_VQ2 || fmt == MOE_FMT_Q2K ? kOpF16 : kOpBF16;
}

template <int BM>
hipError_t gemm_bm(const WView &gate, const WView &up, const WView &down, int H, int I, int T,
                   const uint16_t *x, const int32_t *offsets, const int32_t *sorted_token,
                   int n_rows, int32_t *tiles, uint16_t *a16, uint16_t *x16, float *y,
                   hipStream_t s, void (*mark)(void *, const char *), void *mark_ctx,
                   const char *const names[4]) {
  const int E = offsets ? gate.E : 0;
  // tiles: sum over the active experts of ceil(rows / BM) <= n_rows / BM + the
  // active count, which is at most min(E, n_rows) (blocks past the real count
  // exit at once, but each still takes a slot and a load)
  const int max_tiles = ((n_rows + BM - 1) / BM + std::min(E, n_rows) + 7) / 8 * 8;
  if (mark) mark(mark_ctx, names[0]);
  hipError_t err = launch(k_tile_list, dim3(1), dim3(1024), s, E, n_rows, BM, offsets, tiles);
  if (err != hipSuccess) return err;

  if (gateup_op(gate.fmt) == kOpF16) {
    if (mark) mark(mark_ctx, names[3]);
    const long n8 = (long)T * H / 8;  // H % 256 == 0
    const auto kern = gate.fmt == MOE_FMT_Q2K ? k_tokens_f16<true> : k_tokens_f16<false>;
    err = launch(kern, dim3((unsigned)((n8 + 255) / 256)), dim3(256), s, n8,
                 reinterpret_cast<const uint4 *>(x), reinterpret_cast<uint4 *>(x16));
    if (err != hipSuccess) return err;
    x = x16;
  }

  GemmArgs g{};
  g.K = H, g.N = I, g.w0 = gate, g.w1 = up, g.x = x, g.a_rows = T;
  g.row_token = offsets ? sorted_token : nullptr;
  g.tiles = tiles, g.a_out = a16;
  g.a_swap = down.fmt == MOE_FMT_Q2K;
  // one dense expert with many row tiles: keep each weight block in an L2
  g.weight_major = !offsets && (I / block_cols<kModeGateUp, MOE_FMT_BF16>()) % 8 == 0 && max_tiles >= 16;
  if (mark) mark(mark_ctx, names[1]);
  err = gemm_fmt<kModeGateUp, BM>(g, gate.fmt, gateup_op(gate.fmt), max_tiles, s);
  if (err != hipSuccess) return err;

  GemmArgs d{};
  d.K = I, d.N = H, d.w0 = down, d.w1 = down, d.a16 = a16, d.a_rows = n_rows, d.tiles = tiles;
  d.weight_major = !offsets && (H / block_cols<kModeDown, MOE_FMT_BF16>()) % 8 == 0 && max_tiles >= 16;
  d.y_out = y;
  if (mark) mark(mark_ctx, names[2]);
  return gemm_fmt<kModeDown, BM>(d, down.fmt, kOpF16, max_tiles, s);
}

}  // namespace

template <int MB>
static hipError_t skinny_mb(const WView &gate, const WView &up, const WView &down, int H, int I,
                            int T, const uint16_t *x, uint16_t *a16, float *y, hipStream_t s,
                            void (*mark)(void *, const char *), void *mark_ctx,
                            const char *const names[4]) {
  SkinnyArgs g{T, H, I, reinterpret_cast<const uint16_t *>(gate.data),
               reinterpret_cast<const uint16_t *>(up.data), x, a16, nullptr};
  if (mark) mark(mark_ctx, names[1]);
  hipError_t err = launch(k_skinny<kModeGateUp, MB>, dim3(I / 16), dim3(64 * kSkWaves), s, g);
  if (err != hipSuccess) return err;
  SkinnyArgs d{T, I, H, reinterpret_cast<const uint16_t *>(down.data), nullptr, a16, nullptr, y};
  if (mark) mark(mark_ctx, names[2]);
  return launch(k_skinny<kModeDown, MB>, dim3(H / 16), dim3(64 * kSkWaves), s, d);
}

bool skinny_supported(int H, int I, int T, const WView &gate, const WView &down) {
  return gate.fmt == MOE_FMT_BF16 && down.fmt == MOE_FMT_BF16 && gate.E == 1 && T >= 1 &&
         T <= 64 && H % (kBKs * kSkWaves) == 0 && I % (kBKs * kSkWaves) == 0;
}

hipError_t launch_skinny_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                             int T, const uint16_t *x, uint16_t *a16, float *y, hipStream_t s,
                             void (*mark)(void *, const char *), void *mark_ctx,
                             const char *const names[4]) {
  if (!skinny_supported(H, I, T, gate, down)) return hipErrorInvalidValue;
  if (T <= 16) return skinny_mb<1>(gate, up, down, H, I, T, x, a16, y, s, mark, mark_ctx, names);
  if (T <= 32) return skinny_mb<2>(gate, up, down, H, I, T, x, a16, y, s, mark, mark_ctx, names);
  return skinny_mb<4>(gate, up, down, H, I, T, x, a16, y, s, mark, mark_ctx, names);
}

hipError_t launch_gemm_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                           int T, const uint16_t *x, const int32_t *offsets,
                           const int32_t *sorted_token, int n_rows, int32_t *tiles, uint16_t *a16,
                           uint16_t *x16, float *y, hipStream_t s,
                           void (*mark)(void *, const char *), void *mark_ctx,
                           const char *const names[4]) {
  if (!gemm_supported(H, I, gate.fmt, down.fmt) || n_rows < 1 || T < 1) return hipErrorInvalidValue;
  if (gateup_op(gate.fmt) == kOpF16 && !x16) return hipErrorInvalidValue;
  // rows per tile: 128 for one dense expert of 96 rows or more (one wave per
  // SIMD, each weight read for more rows), 64 from 32 rows per active expert,
  // else 16.  Grouped experts stay at 64 even with 128 rows each: two tiles
  // at two waves per SIMD beat one at one (prefill 4096, 128 rows per
  // expert: VQ2 gate/up 1848 -> 1488 us, MXFP4 2175 -> 1779 us)
  const int active = offsets ? (gate.E < n_rows ? gate.E : n_rows) : 1;
  if (!offsets && n_rows >= 96)
    return gemm_bm<128>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16,
                        x16, y, s, mark, mark_ctx, names);
  if (n_rows >= 32 * active)
    return gemm_bm<64>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16, x16,
                       y, s, mark, mark_ctx, names);
  return gemm_bm<16>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16, x16, y,
                     s, mark, mark_ctx, names);
}

}  // namespace moe
