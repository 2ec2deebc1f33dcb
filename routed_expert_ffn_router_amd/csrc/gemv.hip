// gemv.hip -- decode path: dequant-fused GEMVs over the experts' weights.
//
// Decode reads every selected expert's weights once per token batch, so it is
// bound by HBM bandwidth (the ds4 pages: routed experts dominate the model's
// size and generation pays for fetching them -- hysenlabs.com, "SSD
// streaming"; baiwuji.top, "SSD streaming").  These kernels stream the
// quantized bytes once, decode them in registers and reduce with wavefront
// DPP; no matrix cores.  Blocks are 4 waves; grid.y walks the active experts
// of a plan (or one dense expert), grid.x the row tiles.
#include "gemv_core.h"

namespace moe {

struct GateUpArgs {
  WView gate, up;
  int H, I;
  const uint16_t *x;
  const int32_t *plan;  // null: dense expert 0 over rows [0, n_dense)
  int n_dense;
  const int32_t *row_token;
  float *a;
};

struct DownArgs {
  WView down;
  int H, I;
  const float *a;
  const int32_t *plan;
  int n_dense;
  float *y;
};

__device__ __forceinline__ bool block_bucket(const int32_t *plan, int n_dense, int *e, int *r0,
                                             int *r1) {
  if (plan) {
    const int a = blockIdx.y;
    if (a >= plan[0]) return false;
    *e = plan[1 + 3 * a];
    *r0 = plan[2 + 3 * a];
    *r1 = plan[3 + 3 * a];
  } else {
    *e = 0;
    *r0 = 0;
    *r1 = n_dense;
  }
  return true;
}

template <int FMT, int SPL, int LPR, int STEPS, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup(GateUpArgs p) {
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  int e, r0, r1;
  if (!block_bucket(p.plan, p.n_dense, &e, &r0, &r1)) return;
  if constexpr (FMT == MOE_FMT_VQ2) {
    fill_codebook(p.gate.codebook, s_cb);
    __syncthreads();
  }
  constexpr int RPS = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_base = (blockIdx.x * 4 + wave) * STEPS * RPS + lane / LPR;
  gateup_rows<FMT, SPL, LPR, STEPS, NT>(p.gate, p.up, p.H, p.I, p.x, e, r0, r1, p.row_token, -1,
                                        p.a, row_base, s_cb + (lane % kNCopy));
}

template <int FMT, int SPL, int LPR, int STEPS, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_down(DownArgs p) {
  __shared__ uint2 s_cb[FMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  int e, r0, r1;
  if (!block_bucket(p.plan, p.n_dense, &e, &r0, &r1)) return;
  if constexpr (FMT == MOE_FMT_VQ2) {
    fill_codebook(p.down.codebook, s_cb);
    __syncthreads();
  }
  constexpr int RPS = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_base = (blockIdx.x * 4 + wave) * STEPS * RPS + lane / LPR;
  down_rows<FMT, SPL, LPR, STEPS, NT>(p.down, p.H, p.I, p.a, e, r0, r1, p.y, row_base,
                                      s_cb + (lane % kNCopy));
}

// --------------------------------------------------------------------------
// host dispatch over formats and K
// --------------------------------------------------------------------------

namespace {

template <int FMT, int SPL, int LPR>
hipError_t gateup_inst(const GateUpArgs &a, int max_active, int ntok_hint, hipStream_t s) {
  constexpr int ST = steps_for<FMT, SPL>();
  constexpr int RPB = 4 * ST * (64 / LPR);
  dim3 grid((a.I + RPB - 1) / RPB, a.plan ? max_active : 1);
  if (ntok_hint >= 4)
    return launch(k_gateup<FMT, SPL, LPR, ST, 4>, dim3(grid), dim3(256), s, a);
  return launch(k_gateup<FMT, SPL, LPR, ST, 1>, dim3(grid), dim3(256), s, a);
}

template <int FMT, int SPL, int LPR>
hipError_t down_inst(const DownArgs &a, int max_active, int ntok_hint, hipStream_t s) {
  constexpr int ST = steps_for<FMT, SPL>();
  constexpr int RPB = 4 * ST * (64 / LPR);
  dim3 grid((a.H + RPB - 1) / RPB, a.plan ? max_active : 1);
  if (ntok_hint >= 4)
    return launch(k_down<FMT, SPL, LPR, ST, 4>, dim3(grid), dim3(256), s, a);
  return launch(k_down<FMT, SPL, LPR, ST, 1>, dim3(grid), dim3(256), s, a);
}

template <int FMT>
hipError_t gateup_fmt(const GateUpArgs &a, int max_active, int nh, hipStream_t s) {
  int spl, lpr;
  if (!gemv_geometry(a.H, &spl, &lpr)) return hipErrorInvalidValue;
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
  if (!gemv_geometry(a.I, &spl, &lpr)) return hipErrorInvalidValue;
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

}  // namespace

bool gemv_supported_k(int K) {
  int spl, lpr;
  return gemv_geometry(K, &spl, &lpr);
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

}  // namespace moe
