// decode.hip -- one token through the whole MoE layer in three launches.
//
// Batch-1 decode streams ~109 MB of weights for ~0.5 GFLOP, so it is bound by
// HBM bandwidth and by the fixed cost of each kernel boundary.  The layer's
// dependency chain (router -> selection -> routed gate/up -> routed down) is
// cut into three launches, and the shared expert -- independent of routing
// (the pages keep it at full precision and add it to the routed sum:
// dibi8.com ds4 guide "Key innovations" item 1) -- fills the same launches:
//   p1: router logits (fp64, one wave per expert)  +  shared gate/up + SwiGLU
//   p2: top-k selection, recomputed by every routed block from the logits
//       (no separate launch), then routed gate/up + SwiGLU  +  shared down
//   p3: routed down of the k experts (one expert per wave) + weighted sum +
//       shared output, reduced in a fixed order (deterministic, no atomics)
// Blocks are 8 waves; within each launch, block ranges select the role.
#include "select.h"

namespace moe {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kP3Rows = 8;

// ---------------------------------------------------------------------------
// p1: router + shared gate/up.  Block b: router rows e = b, b + nb, ... (each
// row split over the 8 waves, 512 weights per wave, fp64 partials reduced in
// LDS in wave order) and shared rows i = b*8 + wave (+ nb*8 ...), one gate/up
// row pair per wave.
// ---------------------------------------------------------------------------
template <int SSPL>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_p1(DecodeArgs p) {
  __shared__ double s_part[kDecWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = gridDim.x;
  if (p.Is) {
    for (int i0 = blockIdx.x * kDecWaves; i0 < p.Is; i0 += nb * kDecWaves)
      gateup_rows<MOE_FMT_BF16, SSPL, 64, 1, 1>(p.sg, p.su, p.H, p.Is, p.x, 0, 0, 1, nullptr, 0,
                                                 nullptr, i0 + wave, nullptr, kASplit, p.a_sh_hi,
                                                 p.a_sh_lo);
  }
  if (p.logits_in) return;
  for (int e = blockIdx.x; e < p.E; e += nb) {
    const uint16_t *wrow = p.w_router + (size_t)e * p.H;
    double acc = 0.0;
    for (int h = (wave * 64 + lane) * 8; h < p.H; h += kDecThreads * 8) {
      const uint4 xv = *reinterpret_cast<const uint4 *>(p.x + h);
      const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + h);
      acc = fma((double)bf16_lo(xv.x), (double)bf16_lo(wv.x), acc);
      acc = fma((double)bf16_hi(xv.x), (double)bf16_hi(wv.x), acc);
      acc = fma((double)bf16_lo(xv.y), (double)bf16_lo(wv.y), acc);
      acc = fma((double)bf16_hi(xv.y), (double)bf16_hi(wv.y), acc);
      acc = fma((double)bf16_lo(xv.z), (double)bf16_lo(wv.z), acc);
      acc = fma((double)bf16_hi(xv.z), (double)bf16_hi(wv.z), acc);
      acc = fma((double)bf16_lo(xv.w), (double)bf16_lo(wv.w), acc);
      acc = fma((double)bf16_hi(xv.w), (double)bf16_hi(wv.w), acc);
    }
    acc = group_sum_f64<64>(acc);
    if (lane == 0) s_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
      for (int w = 0; w < kDecWaves; w++) t += s_part[w];
      p.logits[e] = (float)t;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// p2: block b does shared-down rows n = b*8 + wave (+ nb*8 ...) and routed
// gate/up tile b (expert slot b / tiles, 8 waves x ST rows).  The shared-down
// loads are issued first, so they are in flight while wave 0 selects the
// experts from the logits.
// ---------------------------------------------------------------------------
template <int RFMT, int RSPL, int DSPL>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_p2(DecodeArgs p) {
  __shared__ uint2 s_cb[RFMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  __shared__ int s_e[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = gridDim.x;
  // shared down: first row of this wave, loads in flight during selection
  const int n_first = blockIdx.x * kDecWaves + wave;
  Chunk<MOE_FMT_BF16, DSPL, 64> cd;
  ADown<MOE_FMT_BF16, DSPL, 64> ad[1];
  const bool do_sd = p.Is && n_first < p.H;
  if (do_sd) {
    cd.load(p.sd, 0, n_first, lane);
    ad[0].load_split(p.a_sh_hi, p.a_sh_lo, lane);
  }
  const bool do_routed = (int)blockIdx.x < p.nb_routed;
  if (do_routed) {
    if constexpr (RFMT == MOE_FMT_VQ2) fill_codebook(p.gate.codebook, s_cb);
    if (wave == 0) {
      int e;
      float w;
      select_wave(p.mode, p.E, p.k, p.logits_in ? p.logits_in : p.logits, p.tid ? p.tid[0] : 0,
                  &e, &w);
      if (lane < p.k) {
        s_e[lane] = e;
        if (blockIdx.x == 0) {
          p.topk_idx[lane] = e;
          p.topk_w[lane] = w;
        }
      }
    }
  }
  if (do_sd) {
    float y[1];
    cd.template dot_a<1>(ad, nullptr, y);
    y[0] = wave_sum_f(y[0]);
    if (lane == 0) p.shared_y[n_first] = y[0];
    for (int n = n_first + nb * kDecWaves; n < p.H; n += nb * kDecWaves) {
      cd.load(p.sd, 0, n, lane);
      cd.template dot_a<1>(ad, nullptr, y);
      y[0] = wave_sum_f(y[0]);
      if (lane == 0) p.shared_y[n] = y[0];
    }
  }
  if (!do_routed) return;
  __syncthreads();
  constexpr int ST = steps_for<RFMT, RSPL>();
  const int j = blockIdx.x / p.tiles_per_expert, tile = blockIdx.x % p.tiles_per_expert;
  const int row_base = (tile * kDecWaves + wave) * ST;
  const int e_sel = __builtin_amdgcn_readfirstlane(s_e[j]);
  gateup_rows<RFMT, RSPL, 64, ST, 1>(p.gate, p.up, p.H, p.I, p.x, e_sel, j, j + 1, nullptr, 0,
                                     p.a, row_base, s_cb + (lane % kNCopy), p.a_mode, p.a_hi,
                                     p.a_lo);
}

// ---------------------------------------------------------------------------
// p3: routed down (one expert per wave, kP3Rows rows in two halves, the
// second half's loads issued before the first half is computed) + weighted
// sum over experts in wave order + shared output.
// ---------------------------------------------------------------------------
template <int DFMT, int DSPL>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_p3(DecodeArgs p) {
  __shared__ uint2 s_cb[DFMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  __shared__ float s_part[kDecWaves][kP3Rows];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (DFMT == MOE_FMT_VQ2) {
    fill_codebook(p.down.codebook, s_cb);
    __syncthreads();
  }
  constexpr int PF = 2;  // rows whose loads are in flight per wave
  const uint2 *cb = s_cb + (lane % kNCopy);
  const int row0 = blockIdx.x * kP3Rows;
  float acc[kP3Rows];
#pragma unroll
  for (int r = 0; r < kP3Rows; r++) acc[r] = 0.0f;
  for (int j = wave; j < p.k; j += kDecWaves) {
    const int e = __builtin_amdgcn_readfirstlane(p.topk_idx[j]);
    const float wj = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p.topk_w[j])));
    Chunk<DFMT, DSPL, 64> c[PF];
#pragma unroll
    for (int r = 0; r < PF; r++) c[r].load(p.down, e, min(row0 + r, p.H - 1), lane);
    ADown<DFMT, DSPL, 64> av[1];
    if constexpr (DFMT == MOE_FMT_Q2K || DFMT == MOE_FMT_BF16)
      av[0].load_split(p.a_hi + (size_t)j * p.I, p.a_lo + (size_t)j * p.I, lane);
    else
      av[0].load(p.a + (size_t)j * p.I, lane);
#pragma unroll
    for (int r = 0; r < kP3Rows; r++) {
      float y[1];
      c[r % PF].template dot_a<1>(av, cb, y);
      if (r + PF < kP3Rows) c[r % PF].load(p.down, e, min(row0 + r + PF, p.H - 1), lane);
      __builtin_amdgcn_sched_barrier(0);
      acc[r] = fmaf(wj, y[0], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kP3Rows; r++) {
    const float v = wave_sum_f(acc[r]);
    if (lane == 0) s_part[wave][r] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < kP3Rows) {
    const int r = threadIdx.x, row = row0 + r;
    if (row < p.H) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; w++) v += s_part[w][r];
      if (p.shared_y) v += p.shared_y[row];
      p.out[row] = v;
      if (p.out_bf16) p.out_bf16[row] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

int spl_of(int K) {
  int spl, lpr;
  if (!gemv_geometry(K, &spl, &lpr) || lpr != 64) return 0;
  return spl;
}

template <int RFMT, int RSPL, int DSPL>
hipError_t p2_launch(const DecodeArgs &a, hipStream_t s) {
  launch(k_dec_p2<RFMT, RSPL, DSPL>, dim3(max(a.nb_routed, a.nb_shared_down)), dim3(kDecThreads), s, a);
  return hipGetLastError();
}

template <int RFMT>
hipError_t p2_fmt(const DecodeArgs &a, int rspl, int dspl, hipStream_t s) {
  if (rspl == 4 && dspl == 2) return p2_launch<RFMT, 4, 2>(a, s);
  if (rspl == 4 && dspl == 4) return p2_launch<RFMT, 4, 4>(a, s);
  if (rspl == 2 && dspl == 2) return p2_launch<RFMT, 2, 2>(a, s);
  if (rspl == 2 && dspl == 4) return p2_launch<RFMT, 2, 4>(a, s);
  return hipErrorInvalidValue;
}

template <int DFMT>
hipError_t p3_fmt(const DecodeArgs &a, int dspl, hipStream_t s) {
  const int grid = (a.H + kP3Rows - 1) / kP3Rows;
  if (dspl == 2)
    launch(k_dec_p3<DFMT, 2>, dim3(grid), dim3(kDecThreads), s, a);
  else if (dspl == 4)
    launch(k_dec_p3<DFMT, 4>, dim3(grid), dim3(kDecThreads), s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int rows_per_block(int fmt, int spl) {
  int st = 1;
  switch (fmt) {
    case MOE_FMT_BF16: st = spl == 2 ? steps_for<MOE_FMT_BF16, 2>() : steps_for<MOE_FMT_BF16, 4>(); break;
    case MOE_FMT_Q2K: st = spl == 2 ? steps_for<MOE_FMT_Q2K, 2>() : steps_for<MOE_FMT_Q2K, 4>(); break;
    case MOE_FMT_VQ2: st = spl == 2 ? steps_for<MOE_FMT_VQ2, 2>() : steps_for<MOE_FMT_VQ2, 4>(); break;
    case MOE_FMT_MXFP4: st = spl == 2 ? steps_for<MOE_FMT_MXFP4, 2>() : steps_for<MOE_FMT_MXFP4, 4>(); break;
  }
  return kDecWaves * st;
}

}  // namespace

bool decode1_supported(int H, int I, int Is, int k) {
  const int sh = spl_of(H), si = spl_of(I);
  const bool shared_ok = Is == 0 || spl_of(Is) == 2 || spl_of(Is) == 4;
  return (sh == 2 || sh == 4) && (si == 2 || si == 4) && shared_ok && k <= 16 && H % 512 == 0;
}

hipError_t launch_decode1(DecodeArgs a, hipStream_t s, void (*mark)(void *, const char *),
                          void *mark_ctx) {
  const int hs = spl_of(a.H), is = spl_of(a.I), ss = a.Is ? spl_of(a.Is) : 2;
  // p1: one router row per block and one shared gate/up row pair per wave
  a.nb_router = a.logits_in ? 0 : a.E;
  a.nb_shared_gu = a.Is ? (a.Is + kDecWaves - 1) / kDecWaves : 0;
  const int rpb = rows_per_block(a.gate.fmt, hs);
  a.tiles_per_expert = (a.I + rpb - 1) / rpb;
  a.nb_routed = a.k * a.tiles_per_expert;
  // p2: shared-down rows are spread one per wave over the routed blocks
  a.nb_shared_down = a.Is ? min((a.H + kDecWaves - 1) / kDecWaves, max(a.nb_routed, 1)) : 0;
  if (!a.Is) a.shared_y = nullptr;
  a.a_mode = a.down.fmt == MOE_FMT_Q2K ? kASplitQ2K : a.down.fmt == MOE_FMT_BF16 ? kASplit : kAF32;
  hipError_t e;
  if (a.nb_router + a.nb_shared_gu > 0) {
    mark(mark_ctx, "decode_p1");
    const int g1 = max(a.nb_router, a.nb_shared_gu);
    if (hs == 4)
      launch(k_dec_p1<4>, dim3(g1), dim3(kDecThreads), s, a);
    else
      launch(k_dec_p1<2>, dim3(g1), dim3(kDecThreads), s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark(mark_ctx, "decode_p2");
  switch (a.gate.fmt) {
    case MOE_FMT_BF16: e = p2_fmt<MOE_FMT_BF16>(a, hs, ss, s); break;
    case MOE_FMT_Q2K: e = p2_fmt<MOE_FMT_Q2K>(a, hs, ss, s); break;
    case MOE_FMT_VQ2: e = p2_fmt<MOE_FMT_VQ2>(a, hs, ss, s); break;
    default: e = p2_fmt<MOE_FMT_MXFP4>(a, hs, ss, s); break;
  }
  if (e != hipSuccess) return e;
  mark(mark_ctx, "decode_p3");
  switch (a.down.fmt) {
    case MOE_FMT_BF16: e = p3_fmt<MOE_FMT_BF16>(a, is, s); break;
    case MOE_FMT_Q2K: e = p3_fmt<MOE_FMT_Q2K>(a, is, s); break;
    case MOE_FMT_VQ2: e = p3_fmt<MOE_FMT_VQ2>(a, is, s); break;
    default: e = p3_fmt<MOE_FMT_MXFP4>(a, is, s); break;
  }
  return e;
}

}  // namespace moe
