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
#include <type_traits>

#include "gemv_core.h"
#include "lds_dma.h"

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
// (16-row gate/up of the decoded formats: at least 3 waves per SIMD, which
// the two-stage A schedule otherwise exceeds by one register)
__global__ __launch_bounds__(kGemmThreads, BM == 16 && FMT != MOE_FMT_MXFP4 && MODE == kModeGateUp ? 3 : 1) void k_gemm(GemmArgs p) {
  constexpr int MB = BM / 16;  // MFMA row blocks
  constexpr int NB = col_blocks<FMT>();
  constexpr int kPA = 4;       // A stages in flight (one group)
  constexpr bool kGroupB = FMT != MOE_FMT_BF16;
  // A stage buffers: four, two stages written per barrier into the two
  // buffers the previous two stages read (one barrier per two stages: decode
  // b16 down 70 -> 66 us, gate/up 94 -> 91 us); MXFP4 gate/up keeps two and
  // a barrier per stage (its wider raw groups leave no registers for it)
  constexpr int kAB = MODE == kModeDown || FMT != MOE_FMT_MXFP4 ? 4 : 2;
  __shared__ uint32_t s_a[kAB][BM * kLdsRowW];
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  // XCD-aware block order (block_tile)
  int ti, bx;
  if (!block_tile(p.weight_major, p.tiles[0], &ti, &bx)) return;
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
  // stages past the end re-read the last one (never used; keeps the loads unconditional)
#pragma unroll
  for (int u = 0; u < kAB / 2; u++) {
    sa[u].store(&s_a[u][arow * kLdsRowW + acol / 2]);
    sa[u].load(ra, a_off, a_kb(min(kPA + u, nk - 1)), acol);
  }
  __syncthreads();  // the first A stages and the codebook

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
      const uint32_t *A = s_a[it & (kAB - 1)];
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
      // A: the next kAB / 2 stages into their buffers (after every stage, or
      // every second one), their register slots refilled kPA stages on
      if (kAB == 2 || (S & 1)) {
#pragma unroll
        for (int u = 1; u <= kAB / 2; u++) {
          const int an = (S + u) & 3;
          sa[an].store(&s_a[(it + u) & (kAB - 1)][arow * kLdsRowW + acol / 2]);
          sa[an].load(ra, a_off, a_kb(min(it + u + kPA, nk - 1)), acol);
        }
        __syncthreads();
      }
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
// Tiles of 64 or 128 bucket rows: the same block shape on the 32 x 32 x 16
// matrix instructions, which run this chip's fp16 / bf16 products about 1.6
// times faster than the 16 x 16 x 32 ones (measured with the matrix-core
// probe).  Operand layout (v_mfma_f32_32x32x16_{f16,bf16}): lane l holds 8
// consecutive reduction slots 8 (l / 32) + [0, 8) of A row l % 32 and of B
// column l % 32; result register i of lane l is row 8 (i / 4) + 4 (l / 32) +
// i % 4, column l % 32.
//
// Reduction slots: lane half h = l / 32 covers, over a 256-group's 4 stages,
// the contiguous run 128 h + [0, 128) of its weight row, 32 per stage, 8 per
// instruction; the A stage in LDS holds, in column c, k = 256 G + 128 (c /
// 32) + 32 S + c % 32, so that lane (row, h) reads columns 32 h + 8 t of its
// row for instruction t.  Q2K weights keep the swap12 pairing within each
// group of 4 (the A operand is stored in that order where it is produced).
// ---------------------------------------------------------------------------
typedef float f32x16v_t __attribute__((ext_vector_type(16)));

template <int OP>
__device__ __forceinline__ f32x16v_t mfma32(uint4 a, uint4 b, f32x16v_t c) {
  if constexpr (OP == kOpBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// one lane's run of 128 weights of a row in a 256-group: raw bits -> 16
// operand pairs per stage (stage S: the run's weights 32 S .. 32 S + 31)
template <int FMT, int OP>
struct BRun {
  uint32_t q[FMT == MOE_FMT_MXFP4 ? 16 : 8];
  uint32_t s0, s1, s2;  // VQ2: scale; Q2K: 8 scale/min bytes, d|dmin; MXFP4: 4 E8M0 bytes

  // k0: first column of the run (256 G + 128 h)
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k0) {
    const uint32_t db = (uint32_t)expert_data_bytes(FMT, w.N, w.K);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(w.data + (size_t)e * db, db);
    if constexpr (FMT == MOE_FMT_VQ2) {
      const uint32_t sb = (uint32_t)expert_scale_bytes(FMT, w.N, w.K);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
      const uint32_t vo = (uint32_t)row * (uint32_t)(w.K / 4) + (uint32_t)k0 / 4;
      const u32x4_t a = buf_u128(r, vo, 0), b = buf_u128(r, vo + 16, 0);
      q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w, q[4] = b.x, q[5] = b.y, q[6] = b.z, q[7] = b.w;
      s0 = buf_u16(rs, ((uint32_t)row * (uint32_t)(w.K / 256) + (uint32_t)k0 / 256) * 2u, 0);
    } else if constexpr (FMT == MOE_FMT_Q2K) {
      const uint32_t blk = ((uint32_t)row * (uint32_t)(w.K / 256) + (uint32_t)k0 / 256) * kQ2KBytes;
      const uint32_t j = (k0 % 256) / 16;  // first of the 8 sub-blocks
#pragma unroll
      for (int i = 0; i < 8; i++) q[i] = buf_u32(r, blk + 16 + 4 * (j + i), 0);
      s0 = buf_u32(r, blk + j, 0);
      s1 = buf_u32(r, blk + j + 4, 0);
      s2 = buf_u32(r, blk + 80, 0);
    } else {  // MXFP4
      const uint32_t sb = (uint32_t)expert_scale_bytes(FMT, w.N, w.K);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.scales + (size_t)e * sb, sb);
      const uint32_t vo = (uint32_t)row * (uint32_t)(w.K / 2) + (uint32_t)k0 / 2;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const u32x4_t a = buf_u128(r, vo + 16 * i, 0);
        q[4 * i] = a.x, q[4 * i + 1] = a.y, q[4 * i + 2] = a.z, q[4 * i + 3] = a.w;
      }
      s0 = buf_u32(rs, (uint32_t)row * (uint32_t)(w.K / 32) + (uint32_t)k0 / 32, 0);
    }
  }

  __device__ __forceinline__ void decode(int S, uint32_t (&out)[16], const uint2 *cb) const {
    if constexpr (FMT == MOE_FMT_VQ2) {
      const f16x2_t d2 = {__builtin_bit_cast(_Float16, (uint16_t)s0),
                          __builtin_bit_cast(_Float16, (uint16_t)s0)};
      // cb: the table, entry e and copy c at byte 256 e + 8 c (32 copies);
      // lane l reads copy l % 32 at (code byte << 8) | 8 (l % 32), one v_perm_b32
      const uint32_t lane_off = (threadIdx.x & 31u) << 3;
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const uint32_t off = __builtin_amdgcn_perm(q[2 * S + c / 4], lane_off,
                                                   0x0C0C0000u | ((4u + (c % 4)) << 8));
        const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(cb) + off);
        out[2 * c] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.x) * d2);
        out[2 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.y) * d2);
      }
    } else if constexpr (FMT == MOE_FMT_Q2K) {
      const float d = f16_bits_to_f32(s2 & 0xFFFFu), dmin = f16_bits_to_f32(s2 >> 16);
#pragma unroll
      for (int sb = 0; sb < 2; sb++) {
        const int sub = 2 * S + sb;  // sub-block of the run: scale byte `sub`
        const uint32_t scm = ((sub < 4 ? s0 : s1) >> (8 * (sub % 4))) & 255u;
        const float ds = d * (float)(scm & 15u), ms = dmin * (float)(scm >> 4);
        const f16x2_t ds2 = {(_Float16)ds, (_Float16)ds};
        const f16x2_t nms2 = {(_Float16)(-ms), (_Float16)(-ms)};
        const uint32_t x = q[sub];
        const uint32_t nl = x & 0x33333333u, nh = (x >> 2) & 0x33333333u;
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const f16x2_t p0 = __builtin_bit_cast(f16x2_t, q2_pair(nl, b));
          const f16x2_t p1 = __builtin_bit_cast(f16x2_t, q2_pair(nh, b));
          out[8 * sb + 2 * b] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(p0, ds2, nms2));
          out[8 * sb + 2 * b + 1] =
              __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(p1, ds2, nms2));
        }
      }
    } else {  // MXFP4: one E8M0 scale per stage (32 weights)
      const float sc = e8m0_to_f32((s0 >> (8 * S)) & 255u);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t v = q[4 * S + j];
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

// bf16 weights: one stage's 32 weights of the run (64 bytes)
template <int OP>
struct BStageBf16x32 {
  uint32_t q[16];
  __device__ __forceinline__ void load(const WView &w, int e, int row, int k) {
    const uint32_t db = (uint32_t)expert_data_bytes(MOE_FMT_BF16, w.N, w.K);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(w.data + (size_t)e * db, db);
    const uint32_t vo = ((uint32_t)row * (uint32_t)w.K + (uint32_t)k) * 2u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4_t a = buf_u128(r, vo + 16 * i, 0);
      q[4 * i] = a.x, q[4 * i + 1] = a.y, q[4 * i + 2] = a.z, q[4 * i + 3] = a.w;
    }
  }
  __device__ __forceinline__ void decode(uint32_t (&out)[16]) const {
#pragma unroll
    for (int i = 0; i < 16; i++) out[i] = OP == kOpF16 ? bf16x2_to_f16x2(q[i]) : q[i];
  }
};

// A stage for the 32-wide layout: thread t stages row t / (256 / BM), LDS
// columns acol .. acol + 64 / (256 / BM) - 1, in runs of 16: LDS column c is
// k = kb + 128 (c / 32) + c % 32 with kb = 256 G + 32 S
template <int BM>
struct AStage32 {
  static constexpr int kCPT = 64 / (kGemmThreads / BM);  // 16 (BM 64) or 32 (BM 128)
  uint32_t raw[kCPT / 2];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t row_off, int kb, int acol) {
#pragma unroll
    for (int j = 0; j < kCPT / 16; j++) {
      const int c = acol + 16 * j;
      const uint32_t vo = row_off + (uint32_t)(kb + 128 * (c / 32) + c % 32) * 2u;
      const u32x4_t a = buf_u128(r, vo, 0), b = buf_u128(r, vo + 16, 0);
      raw[8 * j] = a.x, raw[8 * j + 1] = a.y, raw[8 * j + 2] = a.z, raw[8 * j + 3] = a.w;
      raw[8 * j + 4] = b.x, raw[8 * j + 5] = b.y, raw[8 * j + 6] = b.z, raw[8 * j + 7] = b.w;
    }
  }
  __device__ __forceinline__ void store(uint32_t *dst) const {
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int i = 0; i < kCPT / 8; i++)
      d4[i] = make_uint4(raw[4 * i], raw[4 * i + 1], raw[4 * i + 2], raw[4 * i + 3]);
  }
  // into an unpadded 128-byte row whose 16-byte chunks are XOR-swizzled by
  // sw: chunk c of the row sits at chunk c ^ sw
  __device__ __forceinline__ void store_sw(uint32_t *row, int c0, int sw) const {
#pragma unroll
    for (int i = 0; i < kCPT / 8; i++)
      *reinterpret_cast<uint4 *>(row + 4 * ((c0 + i) ^ sw)) =
          make_uint4(raw[4 * i], raw[4 * i + 1], raw[4 * i + 2], raw[4 * i + 3]);
  }
};

// 64-row tiles: two waves per SIMD (the registers capped at 256); 128-row
// tiles hold 128 accumulators and run one
template <int MODE, int FMT, int OP, int BM>
__global__ __launch_bounds__(kGemmThreads, BM == 64 ? 2 : 1) void k_gemm32(GemmArgs p) {
  static_assert(BM == 64 || BM == 128, "32-row blocks");
  constexpr int MB = BM / 32;  // MFMA row blocks
  constexpr int NB = 2;        // 32-column blocks per wave (64 weight rows)
  // A stages in flight in registers: four (one group) for 64-row tiles; two
  // for 128-row tiles, whose 16-register stages would otherwise leave no room
  // to hold more than one A fragment at a time (every fragment read then waits
  // out the LDS latency before its matrix instructions)
  constexpr int kPA = BM == 128 ? 2 : 4;
  constexpr bool kGroupB = FMT != MOE_FMT_BF16;
  // A stages in LDS.  VQ2: two unpadded 128-byte rows per stage buffer, 16-byte
  // chunks XOR-swizzled by (row / 2) % 8 (a 16-lane group of operand reads
  // then covers all 64 banks), so that the 64 KB codebook of 32 copies fits
  // beside them in two blocks per CU; one barrier per stage.  Other formats:
  // a ring of four padded buffers, each stage written two stages before it
  // is read, one barrier per two stages.
  constexpr bool kSw = FMT == MOE_FMT_VQ2;
  constexpr int kNBuf = kSw ? 2 : 4;
  constexpr int kLead = kNBuf / 2;  // stages between an A stage's store and its read
  constexpr int kAW = kSw ? kBKs / 2 : kLdsRowW;  // dwords per staged row
  constexpr int kCbCopies = 32;
  __shared__ uint32_t s_a[kNBuf][BM * kAW];
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kCbCopies : 1];
  // XCD-aware block order (block_tile)
  int ti, bx;
  if (!block_tile(p.weight_major, p.tiles[0], &ti, &bx)) return;
  const int e = __builtin_amdgcn_readfirstlane(p.tiles[1 + 3 * ti]);
  const int r0 = __builtin_amdgcn_readfirstlane(p.tiles[2 + 3 * ti]);
  const int r1 = __builtin_amdgcn_readfirstlane(p.tiles[3 + 3 * ti]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;  // MFMA row / column within a block; k half
  const int n0 = bx * block_cols<MODE, FMT>();

  if constexpr (FMT == MOE_FMT_VQ2) {  // codebook as exact fp16 integers, kCbCopies copies
    const uint32_t cw = reinterpret_cast<const uint32_t *>(p.w0.codebook)[tid];
    uint32_t hv[2];
#pragma unroll
    for (int j = 0; j < 2; j++)
      hv[j] = pack_h2((float)(int)(int8_t)((cw >> (16 * j)) & 255u),
                      (float)(int)(int8_t)((cw >> (16 * j + 8)) & 255u));
#pragma unroll
    for (int j = 0; j < kCbCopies; j++)
      s_cb[tid * kCbCopies + ((j + tid) & (kCbCopies - 1))] = make_uint2(hv[0], hv[1]);
  }

  constexpr int kTPR = kGemmThreads / BM;
  constexpr int kCPT = kBKs / kTPR;
  const int arow = tid / kTPR, acol = (tid % kTPR) * kCPT;
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)p.K * 2u;
  uint32_t a_off = a_bytes;  // past the end: zeros
  if (r0 + arow < r1) {
    const int src = (MODE == kModeGateUp && p.row_token) ? p.row_token[r0 + arow] : r0 + arow;
    a_off = (uint32_t)src * (uint32_t)p.K * 2u;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(MODE == kModeGateUp ? p.x : p.a16, a_bytes);
  const int nk = p.K / kBKs;
  const int ng = nk / 4;
  auto a_kb = [&](int it) { return 256 * (it >> 2) + 32 * (it & 3); };

  // this lane's weight rows: gate/up: block 0 the gate rows, block 1 the up
  // rows of the same a columns; down: two blocks of 32 outputs
  constexpr int kWaveCols = MODE == kModeGateUp ? 32 : 64;
  int wrow[NB];
  const WView *wv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    if constexpr (MODE == kModeGateUp) {
      wrow[nb] = n0 + kWaveCols * wave + l32;
      wv[nb] = nb == 0 ? &p.w0 : &p.w1;
    } else {
      wrow[nb] = n0 + kWaveCols * wave + 32 * nb + l32;
      wv[nb] = &p.w0;
    }
  }

  AStage32<BM> sa[kPA];
  BRun<FMT, OP> gb0[NB], gb1[NB];
  BStageBf16x32<OP> sb16[2][NB];
  auto b16_k = [&](int it) { return 256 * (it >> 2) + 128 * h + 32 * (it & 3); };
#pragma unroll
  for (int u = 0; u < kPA; u++) sa[u].load(ra, a_off, a_kb(min(u, nk - 1)), acol);
  if constexpr (kGroupB) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) gb0[nb].load(*wv[nb], e, wrow[nb], 128 * h);
  } else {
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int nb = 0; nb < NB; nb++) sb16[u][nb].load(*wv[nb], e, wrow[nb], b16_k(min(u, nk - 1)));
  }
  auto a_store = [&](const AStage32<BM> &st, int buf) {
    if constexpr (kSw)
      st.store_sw(&s_a[buf][arow * kAW], acol / 8, (arow >> 1) & 7);
    else
      st.store(&s_a[buf][arow * kAW + acol / 2]);
  };
#pragma unroll
  for (int u = 0; u < kLead; u++) {
    a_store(sa[u], u);
    sa[u].load(ra, a_off, a_kb(min(kPA + u, nk - 1)), acol);
  }
  __syncthreads();  // the first A stages and the codebook

  const int m_active = (r1 - r0 + 31) >> 5;  // row blocks holding bucket rows
  f32x16v_t acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[m][nb][i] = 0.0f;
  const uint2 *cb = s_cb;

  // B operands: VQ2 and Q2K decode one stage ahead into the other buffer of
  // bp (their decode is long enough to be worth overlapping); MXFP4 and bf16
  // weights convert in a few instructions, so they decode each stage just
  // before its matrix instructions into one buffer, which keeps the 64-row
  // tiles within 256 registers
  constexpr bool kJit = FMT == MOE_FMT_MXFP4 || FMT == MOE_FMT_BF16;
  uint32_t bp[kJit ? 1 : 2][NB][16];
  if constexpr (kGroupB && !kJit) {
#pragma unroll
    for (int nb = 0; nb < NB; nb++) gb0[nb].decode(0, bp[0][nb], cb);
  }

  // MA: row blocks that hold bucket rows, a compile-time constant of the loop
  // below (a per-block test inside it would cut the loop into branches that
  // the compiler schedules one by one, each waiting for every LDS read)
  auto kloop = [&](auto ma_c) {
  constexpr int MA = decltype(ma_c)::value;
  auto group = [&](int G, BRun<FMT, OP>(&cur)[NB], BRun<FMT, OP>(&nxt)[NB]) {
    if constexpr (kGroupB) {
      const int gn = min(G + 1, ng - 1);
#pragma unroll
      for (int nb = 0; nb < NB; nb++) nxt[nb].load(*wv[nb], e, wrow[nb], 256 * gn + 128 * h);
    }
#pragma unroll
    for (int S = 0; S < 4; S++) {
      const int it = 4 * G + S;
      const uint32_t *A = s_a[it % kNBuf];
      const int kCur = kJit ? 0 : (S & 1);  // bp buffer this stage reads
      if constexpr (kGroupB && kJit) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) cur[nb].decode(S, bp[0][nb], cb);
      } else if constexpr (kGroupB) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          if (S < 3)
            cur[nb].decode(S + 1, bp[(S + 1) & 1][nb], cb);
          else
            nxt[nb].decode(0, bp[(S + 1) & 1][nb], cb);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) sb16[S & 1][nb].decode(bp[0][nb]);
        const int st = min(it + 2, nk - 1);
#pragma unroll
        for (int nb = 0; nb < NB; nb++) sb16[S & 1][nb].load(*wv[nb], e, wrow[nb], b16_k(st));
      }
      auto a_frag = [&](int m, int t) {
        if constexpr (kSw)
          return *reinterpret_cast<const uint4 *>(
              &A[(32 * m + l32) * kAW + 4 * ((4 * h + t) ^ ((l32 >> 1) & 7))]);
        else
          return *reinterpret_cast<const uint4 *>(&A[(32 * m + l32) * kAW + (32 * h + 8 * t) / 2]);
      };
      // bf16 weights (the dense shared expert, 128-row tiles at one wave per
      // SIMD): instruction t + 1's A fragments are read before instruction
      // t's MFMAs (the compiler otherwise reuses one register tuple and waits
      // out each read); the scheduling barrier keeps LDS reads and MFMAs in
      // that order and lets everything else move.  The decoded formats keep
      // the compiler's order (measured: Q2K down 2.5% slower, MXFP4 no gain)
      constexpr bool kPipeA = FMT == MOE_FMT_BF16;
      uint4 afn[MA];
      if constexpr (kPipeA) {
#pragma unroll
        for (int m = 0; m < MA; m++) afn[m] = a_frag(m, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        uint4 af[MA];
#pragma unroll
        for (int m = 0; m < MA; m++) {
          if constexpr (kPipeA) {
            af[m] = afn[m];
            if (t < 3) afn[m] = a_frag(m, t + 1);
          } else {
            af[m] = a_frag(m, t);
          }
        }
        if constexpr (kPipeA) __builtin_amdgcn_sched_barrier(0x276);
#pragma unroll
        for (int m = 0; m < MA; m++) {
#pragma unroll
          for (int nb = 0; nb < NB; nb++) {
            const uint32_t *b = bp[kCur][nb];
            const uint4 bf = make_uint4(b[4 * t], b[4 * t + 1], b[4 * t + 2], b[4 * t + 3]);
            acc[m][nb] = mfma32<OP>(af[m], bf, acc[m][nb]);
          }
        }
      }
      // stage it + kLead into the buffer that stage it - kLead read (every
      // wave left it before the last barrier); stage it + kLead + kPA into
      // its registers
      const int an = (S + kLead) % kPA;
      a_store(sa[an], (it + kLead) % kNBuf);
      sa[an].load(ra, a_off, a_kb(min(it + kLead + kPA, nk - 1)), acol);
      if (S % kLead == kLead - 1) __syncthreads();
    }
  };
  for (int G = 0; G < ng; G += 2) {
    group(G, gb0, gb1);
    if (G + 1 < ng) group(G + 1, gb1, gb0);
  }
  };
  // 64-row tiles: one or both 32-row blocks; 128-row tiles (one dense expert,
  // all tiles full but the last) always all four
  if constexpr (MB == 2) {
    if (m_active >= 2)
      kloop(std::integral_constant<int, 2>{});
    else
      kloop(std::integral_constant<int, 1>{});
  } else {
    kloop(std::integral_constant<int, MB>{});
  }

  // result register i of the lane: row 8 (i / 4) + 4 h + i % 4 of the block, column l32
#pragma unroll
  for (int m = 0; m < MB; m++) {
    if (m >= m_active) continue;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = r0 + 32 * m + 8 * (i / 4) + 4 * h + (i % 4);
      if (r >= r1) continue;
      if constexpr (MODE == kModeGateUp) {
        const float a = silu_mul(acc[m][0][i], acc[m][1][i]);
        const int col = n0 + kWaveCols * wave + l32;
        p.a_out[(size_t)r * p.N + (p.a_swap ? swap12(col) : col)] =
            __builtin_bit_cast(uint16_t, (_Float16)a);
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
          p.y_out[(size_t)r * p.N + n0 + kWaveCols * wave + 32 * nb + l32] = acc[m][nb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The grouped GEMM with the token tile moved into LDS by direct loads
// (buffer_load_dwordx4 ... lds), for the decoded formats.  One block of 8
// waves per CU (two per SIMD): the waves share the codebook (32 copies, no
// bank conflicts) and the A tile, and with no register holding a staged A
// tile a block takes up to 128 rows (four 32-row MFMA blocks), so that most
// expert buckets are one tile and their weights are decoded once.
// Wave w covers output columns 32 w + [0, 32) of gate and up (gate/up, 256
// a columns per block) or outputs 64 w + [0, 64) (down, 512 per block); the
// B side (a lane's weight run, decoded into operand registers) is the one of
// k_gemm32.
//
// A ring of 2 kSync stages in LDS.  Stage `it` holds, for every tile row, the
// 64 k of k_gemm32's stage order (k = 256 G + 32 S + 128 (c / 32) + c % 32
// for column c) in an unpadded 128-byte row whose 16-byte chunks are swizzled
// by (row / 2) % 8.  A wave's load instruction fills 1 KB = 8 rows (lane i
// writes slot i, so it fetches the global chunk that belongs at that slot);
// wave w fills rows 8 w + [0, 8), and rows 64 + 8 w + [0, 8) where the tile
// has them (96 rows: waves 0..3; 128 rows: all).  Rows past the bucket read past the end of the buffer
// and land as zeros.  Every kSync stages: wait for all of this wave's loads
// (the kSync stages about to be read were issued kSync stages earlier, and
// nothing newer is in flight), one barrier (every wave's loads are visible,
// and every wave has left the previous kSync stages), then the loads of the
// next kSync stages into the buffers those read.  With a barrier every
// stage, the two waves of a SIMD (one block) waited on each other far more
// often: the spacing is the measured best per format (dma_sync).  Past the
// last stage the last one is loaded again (harmless, and simpler).
// ---------------------------------------------------------------------------
constexpr int kDmaThreads = 512;

// stages per barrier (measured, same-box pairs): VQ2 / Q2K 96-row tiles two
// (prefill 2048: gate/up 790 -> 715-740 us, down 542 -> 482-492 us against
// k_gemm32's 64-row tiles; one barrier per stage: no gain, one per four:
// gate/up 805-830 us); MXFP4 64-row tiles four (prefill 4096: 2775 -> 2660 us
// per step; two per barrier: 2930 us)
#ifndef MOE_DMA_SYNC
#define MOE_DMA_SYNC 0
#endif
template <int FMT, int BM>
constexpr int dma_sync() {
  if (MOE_DMA_SYNC) return MOE_DMA_SYNC;
  return FMT == MOE_FMT_MXFP4 ? 4 : 2;
}

template <int MODE>
constexpr int dma_block_cols() { return MODE == kModeGateUp ? 256 : 512; }

template <int FMT, int BM>
struct DmaCfg {
  static constexpr int kCb = FMT == MOE_FMT_VQ2 ? 32 : 0;  // codebook copies
  static constexpr int kStage = BM * 128;                   // bytes per A stage
  // four stages: stage 4 G + S sits in buffer S, an address the compiler
  // knows (a ring of another length costs an address add per operand read)
  static constexpr int kSync = dma_sync<FMT, BM>();
  static constexpr int kNA = 2 * kSync;
  static constexpr int kRuns = BM / 8;  // 1 KB runs per stage
  static_assert(8 * 256 * kCb + kNA * kStage <= 163840, "LDS");
};

template <int MODE, int FMT, int OP, int BM>
__global__ __launch_bounds__(kDmaThreads, 1) void k_gemm_dma(GemmArgs p) {
  static_assert(BM == 64 || BM == 96 || BM == 128, "two to four 32-row blocks");
  using Cfg = DmaCfg<FMT, BM>;
  constexpr int MB = BM / 32;
  constexpr int NB = 2;
  constexpr int kNA = Cfg::kNA, kCb = Cfg::kCb, kRuns = Cfg::kRuns, kSync = Cfg::kSync;
  __shared__ __attribute__((aligned(16))) uint32_t s_a[kNA][BM * 32];
  __shared__ uint2 s_cb[kCb ? 256 * kCb : 1];
  int ti, bx;
  if (!block_tile(p.weight_major, p.tiles[0], &ti, &bx)) return;
  const int e = __builtin_amdgcn_readfirstlane(p.tiles[1 + 3 * ti]);
  const int r0 = __builtin_amdgcn_readfirstlane(p.tiles[2 + 3 * ti]);
  const int r1 = __builtin_amdgcn_readfirstlane(p.tiles[3 + 3 * ti]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int n0 = bx * dma_block_cols<MODE>();

  if constexpr (FMT == MOE_FMT_VQ2) {  // codebook as exact fp16 integers, 32 copies
    const int ent = tid & 255, half = tid >> 8;
    const uint32_t cw = reinterpret_cast<const uint32_t *>(p.w0.codebook)[ent];
    uint32_t hv[2];
#pragma unroll
    for (int j = 0; j < 2; j++)
      hv[j] = pack_h2((float)(int)(int8_t)((cw >> (16 * j)) & 255u),
                      (float)(int)(int8_t)((cw >> (16 * j + 8)) & 255u));
#pragma unroll
    for (int j = 0; j < kCb / 2; j++) {
      const int c = kCb / 2 * half + j;
      s_cb[ent * kCb + ((c + ent) & (kCb - 1))] = make_uint2(hv[0], hv[1]);
    }
  }

  // this wave's A runs: run w, and run 8 + w where the tile has it
  constexpr int kCh = (kRuns + 7) / 8;
  const int n_ch = wave + 8 < kRuns ? 2 : 1;
  const uint32_t a_bytes = (uint32_t)p.a_rows * (uint32_t)p.K * 2u;
  const i32x4r_t ra = rsrc_words(MODE == kModeGateUp ? p.x : p.a16, a_bytes);
  uint32_t a_vo[kCh];  // row offset + this lane's chunk offset within a stage
#pragma unroll
  for (int j = 0; j < kCh; j++) {
    const int r = 8 * (8 * j + wave) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);  // the global chunk for this slot
    uint32_t vo = a_bytes;                       // past the end: zeros
    if (r < BM && r0 + r < r1) {
      const int src = (MODE == kModeGateUp && p.row_token) ? p.row_token[r0 + r] : r0 + r;
      vo = (uint32_t)src * (uint32_t)p.K * 2u + 2u * (uint32_t)(128 * (c >> 2) + 8 * (c & 3));
    }
    a_vo[j] = vo;
  }
  const int nk = p.K / kBKs;
  const int ng = nk / 4;
  auto a_issue = [&](int it) {
    const int st = min(it, nk - 1);
    const uint32_t kb2 = 2u * (uint32_t)(256 * (st >> 2) + 32 * (st & 3));
    const uint32_t base = lds_offset(&s_a[it & (kNA - 1)][0]);
#pragma unroll
    for (int j = 0; j < kCh; j++) {
      if (j < n_ch) {
        // rows past the bucket keep an offset past the end
        const uint32_t vo = a_vo[j] >= a_bytes ? a_bytes : a_vo[j] + kb2;
        lds_load16(ra, base + 1024u * (uint32_t)(8 * j + wave), vo);
      }
    }
  };

  constexpr int kWaveCols = MODE == kModeGateUp ? 32 : 64;
  int wrow[NB];
  const WView *wv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    if constexpr (MODE == kModeGateUp) {
      wrow[nb] = n0 + kWaveCols * wave + l32;
      wv[nb] = nb == 0 ? &p.w0 : &p.w1;
    } else {
      wrow[nb] = n0 + kWaveCols * wave + 32 * nb + l32;
      wv[nb] = &p.w0;
    }
  }

  BRun<FMT, OP> gb0[NB], gb1[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) gb0[nb].load(*wv[nb], e, wrow[nb], 128 * h);
#pragma unroll
  for (int u = 0; u < kSync; u++) a_issue(u);

  const int m_active = (r1 - r0 + 31) >> 5;
  f32x16v_t acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; m++)
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[m][nb][i] = 0.0f;
  const uint2 *cb = s_cb;

  // B: VQ2 and Q2K decode one stage ahead into the other buffer of bp; MXFP4
  // converts just before use
  constexpr bool kJit = FMT == MOE_FMT_MXFP4;
  uint32_t bp[kJit ? 1 : 2][NB][16];

  auto kloop = [&](auto ma_c) {
    constexpr int MA = decltype(ma_c)::value;
    auto group = [&](int G, BRun<FMT, OP>(&cur)[NB], BRun<FMT, OP>(&nxt)[NB], auto par_c) {
      constexpr int kPar = decltype(par_c)::value;
#pragma unroll
      for (int S = 0; S < 4; S++) {
        const int it = 4 * G + S;
        if (S % kSync == 0) {
          // stages it .. it + kSync - 1 were loaded kSync stages ago and
          // nothing newer is in flight
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
          __syncthreads();
          if (S == 0) {
            const int gn = min(G + 1, ng - 1);
#pragma unroll
            for (int nb = 0; nb < NB; nb++) nxt[nb].load(*wv[nb], e, wrow[nb], 256 * gn + 128 * h);
          }
#pragma unroll
          for (int u = 0; u < kSync; u++) a_issue(it + kSync + u);
        }
        const uint32_t *A = s_a[kNA == 8 ? 4 * kPar + S : S];  // stage it's buffer, it % kNA
        const int kCur = kJit ? 0 : (S & 1);
        if constexpr (kJit) {
#pragma unroll
          for (int nb = 0; nb < NB; nb++) cur[nb].decode(S, bp[0][nb], cb);
        } else {
          if (it == 0) {  // the codebook is in LDS after the first barrier
#pragma unroll
            for (int nb = 0; nb < NB; nb++) cur[nb].decode(0, bp[0][nb], cb);
          }
#pragma unroll
          for (int nb = 0; nb < NB; nb++) {
            if (S < 3)
              cur[nb].decode(S + 1, bp[(S + 1) & 1][nb], cb);
            else
              nxt[nb].decode(0, bp[(S + 1) & 1][nb], cb);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; t++) {
          uint4 af[MA];
#pragma unroll
          for (int m = 0; m < MA; m++)
            af[m] = *reinterpret_cast<const uint4 *>(
                &A[(32 * m + l32) * 32 + 4 * ((4 * h + t) ^ ((l32 >> 1) & 7))]);
#pragma unroll
          for (int m = 0; m < MA; m++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
              const uint32_t *b = bp[kCur][nb];
              const uint4 bf = make_uint4(b[4 * t], b[4 * t + 1], b[4 * t + 2], b[4 * t + 3]);
              acc[m][nb] = mfma32<OP>(af[m], bf, acc[m][nb]);
            }
        }
      }
    };
    for (int G = 0; G < ng; G += 2) {
      group(G, gb0, gb1, std::integral_constant<int, 0>{});
      if (G + 1 < ng) group(G + 1, gb1, gb0, std::integral_constant<int, 1>{});
    }
  };
  if constexpr (MB == 2) {
    if (m_active >= 2)
      kloop(std::integral_constant<int, 2>{});
    else
      kloop(std::integral_constant<int, 1>{});
  } else if constexpr (MB == 3) {
    if (m_active >= 3)
      kloop(std::integral_constant<int, 3>{});
    else if (m_active == 2)
      kloop(std::integral_constant<int, 2>{});
    else
      kloop(std::integral_constant<int, 1>{});
  } else {
    if (m_active >= 4)
      kloop(std::integral_constant<int, 4>{});
    else if (m_active == 3)
      kloop(std::integral_constant<int, 3>{});
    else if (m_active == 2)
      kloop(std::integral_constant<int, 2>{});
    else
      kloop(std::integral_constant<int, 1>{});
  }
  // no load into LDS may be left in flight when the block ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

#pragma unroll
  for (int m = 0; m < MB; m++) {
    if (m >= m_active) continue;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = r0 + 32 * m + 8 * (i / 4) + 4 * h + (i % 4);
      if (r >= r1) continue;
      if constexpr (MODE == kModeGateUp) {
        const float a = silu_mul(acc[m][0][i], acc[m][1][i]);
        const int col = n0 + kWaveCols * wave + l32;
        p.a_out[(size_t)r * p.N + (p.a_swap ? swap12(col) : col)] =
            __builtin_bit_cast(uint16_t, (_Float16)a);
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
          p.y_out[(size_t)r * p.N + n0 + kWaveCols * wave + 32 * nb + l32] = acc[m][nb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One dense bf16 expert over all T rows (the shared expert from 96 tokens),
// with both operands staged in LDS by direct loads.  A block computes 128
// rows against 256 weight rows: gate/up takes 128 gate and the 128 up rows of
// the same SwiGLU columns (column group c = w % 4: columns 32 c + [0, 32) of
// both), down 256 outputs (group c: outputs 64 c + [0, 64)); wave w covers
// rows 64 (w / 4) + [0, 64) of its group (2 x 2 accumulators of 32 x 32).
// Eight waves, two per SIMD: with four (each all 128 rows, one per SIMD)
// gate/up took 81-83 us at 2048 rows against 69-71 us.  buffer_load_dwordx4
// ... lds moves 16 bytes per lane from global memory into LDS (lane i of a
// wave's load writes slot i of a 1 KB run, from whatever global address the
// lane names), three K stages of 64 deep, so no register holds a staged tile
// and the matrix instructions have a whole stage of loads ahead of them.
// LDS rows are 128 bytes, unpadded, 16-byte chunks XOR-swizzled by
// (row / 2) % 8 (a 16-lane group of operand reads covers all 64 banks).
// Reduction slots: instruction t of a stage takes chunks 2t (lane half 0)
// and 2t + 1 (half 1) of every row, for A and B alike.  Gate/up multiplies
// bf16 tokens by bf16 weights and writes the fp16 SwiGLU output; down
// multiplies that fp16 output by the weights converted to fp16 as they leave
// LDS (exact in the binary16 range) and writes fp32.
// ---------------------------------------------------------------------------
constexpr int kDnRows = 128;   // rows per block
constexpr int kDnB = 256;      // weight rows per block
constexpr int kDnK = 64;       // K per stage
constexpr int kDnStages = 3;   // stages in LDS
constexpr int kDnThreads = 512;  // 8 waves: 2 row halves x 4 column groups

template <int MODE>
constexpr int dense_cols() { return MODE == kModeGateUp ? kDnB / 2 : kDnB; }

struct DenseArgs {
  int T, K, N;             // rows, reduction length, output columns
  const uint16_t *a;       // gate/up: bf16 tokens [T][K]; down: fp16 SwiGLU output [T][K]
  const uint16_t *w0, *w1;  // bf16 [N][K]: gate and up, or down (w1 unused)
  uint16_t *a_out;         // gate/up: fp16 [T][N]
  float *y_out;            // down: fp32 [T][N]
  int a_swap;              // gate/up: a_out in Q2K slot order
};

template <int MODE>
__global__ __launch_bounds__(kDnThreads, 1) void k_dense(DenseArgs p) {
  constexpr int kRowU = kDnK / 2;  // dwords per staged row
  constexpr int OP = MODE == kModeGateUp ? kOpBF16 : kOpF16;
  __shared__ __attribute__((aligned(16))) uint32_t s_a[kDnStages][kDnRows * kRowU];
  __shared__ __attribute__((aligned(16))) uint32_t s_b[kDnStages][kDnB * kRowU];
  // weights-first block order, XCD-aware (as the grouped GEMM's dense case)
  const uint32_t nbx = gridDim.x, nby = gridDim.y;
  const uint32_t bid = blockIdx.y * nbx + blockIdx.x;
  const uint32_t jx = bid >> 3;
  const int ti = (int)(jx % nby), bx = (int)((jx / nby) * 8 + (bid & 7));
  const int row0 = ti * kDnRows, n0 = bx * dense_cols<MODE>();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave & 3, rh = wave >> 2;  // column group, row half
  const int l32 = lane & 31, h = lane >> 5;
  const int nk = p.K / kDnK;

  // this lane's slot in each of the wave's direct loads: run j of a stage
  // holds rows 8 j .. 8 j + 7; lane i writes slot i: row 8 j + i / 8, physical
  // chunk i % 8, which holds logical chunk (i % 8) ^ ((row / 2) % 8)
  const i32x4r_t ra = rsrc_words(p.a, (uint32_t)p.T * (uint32_t)p.K * 2u);
  const uint32_t wb = (uint32_t)p.N * (uint32_t)p.K * 2u;
  const i32x4r_t r0 = rsrc_words(p.w0, wb), r1 = rsrc_words(MODE == kModeGateUp ? p.w1 : p.w0, wb);
  constexpr int kARuns = kDnRows / 8 / 8;  // A runs per wave and stage: 2
  constexpr int kBRuns = kDnB / 8 / 8;     // B runs per wave and stage: 4
  uint32_t avo[kARuns], bvo[kBRuns];
#pragma unroll
  for (int u = 0; u < kARuns; u++) {
    const int j = kARuns * wave + u, row = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const int gr = min(row0 + row, p.T - 1);  // rows past T repeat row T - 1 (not stored)
    avo[u] = ((uint32_t)gr * (uint32_t)p.K + 8u * (uint32_t)c) * 2u;
  }
#pragma unroll
  for (int u = 0; u < kBRuns; u++) {
    const int j = kBRuns * wave + u, row = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    // gate/up: rows below 128 are gate rows n0 + row, the rest up rows
    const int wr = n0 + (MODE == kModeGateUp ? (row & (kDnB / 2 - 1)) : row);
    bvo[u] = ((uint32_t)wr * (uint32_t)p.K + 8u * (uint32_t)c) * 2u;
  }
  auto issue = [&](int it) {
    const int buf = it % kDnStages;
    const uint32_t ko = (uint32_t)it * kDnK * 2u;
#pragma unroll
    for (int u = 0; u < kARuns; u++)
      lds_load16(ra, lds_offset(&s_a[buf][(kARuns * wave + u) * 256]), avo[u] + ko);
#pragma unroll
    for (int u = 0; u < kBRuns; u++) {
      const int j = kBRuns * wave + u;
      lds_load16(MODE == kModeGateUp && j >= kDnB / 16 ? r1 : r0, lds_offset(&s_b[buf][j * 256]),
                 bvo[u] + ko);
    }
  };

  f32x16v_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[m][nb][i] = 0.0f;

  issue(0);
  if (nk > 1) issue(1);
  // stage 0 in LDS for every wave (this wave's stage-1 loads may still fly)
  if (nk > 1)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kARuns + kBRuns));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  for (int it = 0; it < nk; it++) {
    if (it + 2 < nk) issue(it + 2);
    const uint32_t *A = s_a[it % kDnStages];
    const uint32_t *B = s_b[it % kDnStages];
    auto a_frag = [&](int m, int t) {
      const int row = 64 * rh + 32 * m + l32;
      return *reinterpret_cast<const uint4 *>(&A[row * kRowU + 4 * ((2 * t + h) ^ ((row >> 1) & 7))]);
    };
    auto b_frag = [&](int nb, int t) {
      const int row = MODE == kModeGateUp ? (kDnB / 2) * nb + 32 * wc + l32 : 64 * wc + 32 * nb + l32;
      const uint4 v =
          *reinterpret_cast<const uint4 *>(&B[row * kRowU + 4 * ((2 * t + h) ^ ((row >> 1) & 7))]);
      if constexpr (MODE == kModeGateUp)
        return v;
      else
        return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
                          bf16x2_to_f16x2(v.w));
    };
#pragma unroll
    for (int t = 0; t < 4; t++) {
      uint4 bf[2];
#pragma unroll
      for (int nb = 0; nb < 2; nb++) bf[nb] = b_frag(nb, t);
#pragma unroll
      for (int m = 0; m < 2; m++) {
        const uint4 af = a_frag(m, t);
#pragma unroll
        for (int nb = 0; nb < 2; nb++) acc[m][nb] = mfma32<OP>(af, bf[nb], acc[m][nb]);
      }
    }
    if (it + 1 < nk) {
      // stage it + 1 complete for this wave (stage it + 2's loads may fly),
      // then for every wave; the barrier also ends this stage's reads of the
      // buffer that stage it + 3 overwrites
      if (it + 2 < nk)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kARuns + kBRuns));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __syncthreads();
    }
  }

  // result register i: row 8 (i / 4) + 4 h + i % 4 of row block m, column l32
#pragma unroll
  for (int m = 0; m < 2; m++) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = row0 + 64 * rh + 32 * m + 8 * (i / 4) + 4 * h + (i % 4);
      if (r >= p.T) continue;
      if constexpr (MODE == kModeGateUp) {
        const float a = silu_mul(acc[m][0][i], acc[m][1][i]);
        const int col = n0 + 32 * wc + l32;
        p.a_out[(size_t)r * p.N + (p.a_swap ? swap12(col) : col)] =
            __builtin_bit_cast(uint16_t, (_Float16)a);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; nb++) p.y_out[(size_t)r * p.N + n0 + 64 * wc + 32 * nb + l32] = acc[m][nb][i];
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

// grid.x: the layer's output columns over the block's; grid.y: tiles.  Tiles
// of 64 and 128 rows run the 32 x 32 x 16 instructions, 16-row tiles the
// 16 x 16 x 32 ones
// the direct-load kernel's formats and shapes
bool dma_ok(int H, int I, int fmt_gate, int fmt_down) {
  auto dec = [](int f) { return f == MOE_FMT_VQ2 || f == MOE_FMT_Q2K || f == MOE_FMT_MXFP4; };
  return dec(fmt_gate) && dec(fmt_down) && I % dma_block_cols<kModeGateUp>() == 0 &&
         H % dma_block_cols<kModeDown>() == 0;
}
// 96- and 128-row tiles always take it; 64-row tiles only for MXFP4 (VQ2
// and Q2K: k_gemm32 is as fast or faster there, prefill 4096 from 64-row
// tiles 2645 vs 2660-2690 us)
template <int BM>
bool use_dma(int fmt) {
  return BM == 96 || BM == 128 || (BM == 64 && fmt == MOE_FMT_MXFP4);
}

template <int MODE, int BM>
hipError_t gemm_dma_fmt(const GemmArgs &a, int fmt, int op, int tiles, hipStream_t s) {
#define MOE_DMA_CASE(F, O)                                                                    \
  if (fmt == F && op == O)                                                                    \
    return launch(k_gemm_dma<MODE, F, O, BM>, dim3(a.N / dma_block_cols<MODE>(), tiles),       \
                  dim3(kDmaThreads), s, a);
  MOE_DMA_CASE(MOE_FMT_VQ2, kOpF16)
  MOE_DMA_CASE(MOE_FMT_Q2K, kOpF16)
  MOE_DMA_CASE(MOE_FMT_MXFP4, kOpBF16)
  MOE_DMA_CASE(MOE_FMT_MXFP4, kOpF16)
#undef MOE_DMA_CASE
  return hipErrorInvalidValue;
}

template <int MODE, int BM>
hipError_t gemm_fmt(const GemmArgs &a, int fmt, int op, int tiles, hipStream_t s, bool dma) {
  if constexpr (BM == 64 || BM == 96 || BM == 128) {
    if (dma && use_dma<BM>(fmt)) return gemm_dma_fmt<MODE, BM>(a, fmt, op, tiles, s);
  }
  if constexpr (BM == 96) {
    return hipErrorInvalidValue;
  } else {
#define MOE_GEMM_CASE(F, O)                                                                  \
  if (fmt == F && op == O) {                                                                 \
    if constexpr (BM >= 64)                                                                  \
      return launch(k_gemm32<MODE, F, O, BM>, dim3(a.N / block_cols<MODE, F>(), tiles),      \
                    dim3(kGemmThreads), s, a);                                               \
    else                                                                                     \
      return launch(k_gemm<MODE, F, O, BM>, dim3(a.N / block_cols<MODE, F>(), tiles),        \
                    dim3(kGemmThreads), s, a);                                               \
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
  const bool dma = (BM == 64 || BM == 96 || BM == 128) && offsets && dma_ok(H, I, gate.fmt, down.fmt);
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
  // one dense bf16 expert from 128-row tiles: both operands staged in LDS by
  // direct loads (the column blocks a multiple of 8 for the block order)
  const bool dense = BM == 128 && !offsets && gate.fmt == MOE_FMT_BF16 &&
                     down.fmt == MOE_FMT_BF16 && H % kDnK == 0 && I % kDnK == 0 &&
                     I % (8 * dense_cols<kModeGateUp>()) == 0 &&
                     H % (8 * dense_cols<kModeDown>()) == 0;
  if (dense) {
    DenseArgs da{T, H, I, x, reinterpret_cast<const uint16_t *>(gate.data),
                 reinterpret_cast<const uint16_t *>(up.data), a16, nullptr, g.a_swap};
    err = launch(k_dense<kModeGateUp>, dim3(I / dense_cols<kModeGateUp>(), (T + kDnRows - 1) / kDnRows),
                 dim3(kDnThreads), s, da);
  } else {
    err = gemm_fmt<kModeGateUp, BM>(g, gate.fmt, gateup_op(gate.fmt), max_tiles, s, dma);
  }
  if (err != hipSuccess) return err;

  GemmArgs d{};
  d.K = I, d.N = H, d.w0 = down, d.w1 = down, d.a16 = a16, d.a_rows = n_rows, d.tiles = tiles;
  d.weight_major = !offsets && (H / block_cols<kModeDown, MOE_FMT_BF16>()) % 8 == 0 && max_tiles >= 16;
  d.y_out = y;
  if (mark) mark(mark_ctx, names[2]);
  if (dense) {
    DenseArgs dd{n_rows, I, H, a16, reinterpret_cast<const uint16_t *>(down.data), nullptr,
                 nullptr, y, 0};
    return launch(k_dense<kModeDown>, dim3(H / dense_cols<kModeDown>(), (n_rows + kDnRows - 1) / kDnRows),
                  dim3(kDnThreads), s, dd);
  }
  return gemm_fmt<kModeDown, BM>(d, down.fmt, kOpF16, max_tiles, s, dma);
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
  // rows per tile: 128 for one dense expert of 96 rows or more (k_dense);
  // for grouped experts in a decoded format (k_gemm_dma, two waves per SIMD,
  // the token tile in LDS only), 128 above 96 rows per active expert and 96
  // from 49 (most buckets one tile, each expert's weights decoded about once
  // instead of 1.5 or 2.5 times: prefill 2048, 64 rows per expert, 1486 ->
  // 1375 us per step; prefill 4096, 128 rows, 2651 -> 2492 us); otherwise 64
  // from 32 rows per active expert (k_gemm32), else 16
  const int active = offsets ? (gate.E < n_rows ? gate.E : n_rows) : 1;
  if (!offsets && n_rows >= 96)
    return gemm_bm<128>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16,
                        x16, y, s, mark, mark_ctx, names);
  if (offsets && dma_ok(H, I, gate.fmt, down.fmt) && n_rows > 96 * active)
    return gemm_bm<128>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16, x16,
                        y, s, mark, mark_ctx, names);
  if (offsets && dma_ok(H, I, gate.fmt, down.fmt) && n_rows > 48 * active)
    return gemm_bm<96>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16, x16,
                       y, s, mark, mark_ctx, names);
  if (n_rows >= 32 * active)
    return gemm_bm<64>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16, x16,
                       y, s, mark, mark_ctx, names);
  return gemm_bm<16>(gate, up, down, H, I, T, x, offsets, sorted_token, n_rows, tiles, a16, x16, y,
                     s, mark, mark_ctx, names);
}

}  // namespace moe
