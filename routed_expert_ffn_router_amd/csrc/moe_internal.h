// moe_internal.h -- host-side launchers shared between the libmoe sources.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "moe.h"

namespace moe {

// Measurement: a mark arms a pair of events that the next launch records at
// its own start and end (HIP's extended launch); an unarmed launch records
// nothing.  The arming is per host thread and consumed by that launch.
void timer_arm(hipEvent_t start, hipEvent_t stop);
// sets the calling thread's moe_last_error() text; returns code
int set_error(int code, const char *fmt, ...);
void timer_take(hipEvent_t *start, hipEvent_t *stop);

template <typename... P, size_t... I>
inline void kernel_arg_ptrs(std::tuple<P...> &t, void **out, std::index_sequence<I...>) {
  ((out[I] = static_cast<void *>(&std::get<I>(t))), ...);
}

// every libmoe kernel is launched through here; returns the launch's error,
// else any error the thread had pending
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A &&...a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> args{static_cast<P>(a)...};
  void *ptrs[sizeof...(P) + 1];
  kernel_arg_ptrs(args, ptrs, std::index_sequence_for<P...>{});
  hipEvent_t ts, te;
  timer_take(&ts, &te);
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block,
                                          ptrs, 0, s, ts, te, 0);
  const hipError_t pending = hipGetLastError();  // also clears the thread's error state
  return e != hipSuccess ? e : pending;
}

// A projection as the kernels see it.
struct WView {
  int fmt, E, N, K;
  const uint8_t *data;
  const uint8_t *scales;
  const int8_t *codebook;
};

inline WView view_of(const moe_weights &w) {
  return WView{w.fmt, w.n_experts, w.rows, w.cols, static_cast<const uint8_t *>(w.data),
               static_cast<const uint8_t *>(w.scales), w.codebook};
}

// Byte offset of expert e's data / scales in a projection.
__host__ __device__ inline size_t expert_data_bytes(int fmt, int N, int K) {
  size_t n = (size_t)N * K;
  switch (fmt) {
    case MOE_FMT_BF16: return n * 2;
    case MOE_FMT_Q2K: return n / 256 * 84;
    case MOE_FMT_VQ2: return n / 4;
    case MOE_FMT_MXFP4: return n / 2;
  }
  return 0;
}
__host__ __device__ inline size_t expert_scale_bytes(int fmt, int N, int K) {
  size_t n = (size_t)N * K;
  switch (fmt) {
    case MOE_FMT_VQ2: return n / 256 * 2;
    case MOE_FMT_MXFP4: return n / 32;
  }
  return 0;
}

// Compact plan of the experts that received tokens (decode path):
//   plan[0] = n_active; for a < n_active: plan[1+3a] = expert,
//   plan[2+3a] = first bucket row, plan[3+3a] = one past the last.
inline size_t plan_ints(int max_active) { return 1 + 3 * (size_t)max_active; }

// routing ------------------------------------------------------------------
hipError_t launch_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *wr,
                                float *logits, hipStream_t s);
// Logits for the selection only: exact (as above) for the experts that can
// reach the top k, -inf for the others; wn2: E floats of scratch.  Needs
// router_screen_supported(H, E).
bool router_screen_supported(int H, int E);
hipError_t launch_router_screened(int mode, int T, int H, int E, int k, const uint16_t *x,
                                  const uint16_t *wr, const int64_t *tids, float *logits,
                                  float *wn2, hipStream_t s);
// selection; when `plan` is non-null (T*k <= kSmallSlots) it also buckets
// the slots: sorted_token/sorted_slot/slot_pos/row_w [T*k], offsets [E+1]
// (optional) and the compact plan.
constexpr int kSmallSlots = 1024;
hipError_t launch_select(int mode, int T, int E, int k, const float *logits,
                         const int64_t *token_ids, int32_t *idx, float *w, int32_t *offsets,
                         int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos,
                         float *row_w, int32_t *plan, hipStream_t s);

// dispatch -----------------------------------------------------------------
size_t dispatch_ws_bytes(int T, int E, int k);
hipError_t launch_dispatch(int T, int E, int k, const int32_t *idx, int32_t *offsets,
                           int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos,
                           void *ws, hipStream_t s, void (*mark)(void *, const char *) = nullptr,
                           void *mark_ctx = nullptr);
// compact plan from expert offsets (E+1 ints)
hipError_t launch_plan_from_offsets(int E, const int32_t *offsets, int32_t *plan, hipStream_t s);

// dequantize ---------------------------------------------------------------
hipError_t launch_dequant(const WView &w, int expert, int64_t w0, int64_t count, float *out,
                          hipStream_t s);

// decode GEMVs ---------------------------------------------------------------
// a[r][i] = silu(gate_e[i] . x[tok[r]]) * (up_e[i] . x[tok[r]]) for the plan's rows
hipError_t launch_gateup_gemv(const WView &gate, const WView &up, int H, int I,
                              const uint16_t *x, const int32_t *plan, int max_active,
                              const int32_t *row_token, float *a, hipStream_t s);
// y[r][n] = down_e[n] . a[r] for the plan's rows
hipError_t launch_down_gemv(const WView &down, int H, int I, const float *a,
                            const int32_t *plan, int max_active, float *y, hipStream_t s);

// prefill grouped GEMMs (gemm.hip) --------------------------------------------
// Whole expert FFN on the matrix cores: y[r] = down_e . SwiGLU(gate_e, up_e; x[tok[r]])
// for every bucket row r (offsets null: one dense expert over rows [0, n_rows = T)).
// tiles: gemm_tile_ints(n_rows, offsets ? E : 0) ints; a16: fp16 [n_rows][I];
// x16: fp16 [T][H], the tokens converted for fp16 gate/up operands (VQ2, Q2K
// gate), may be null otherwise.  names: tile list, gate/up, down, conversion.
bool gemm_supported(int H, int I, int fmt_gate, int fmt_down);
size_t gemm_tile_ints(int n_rows, int E);
hipError_t launch_gemm_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                           int T, const uint16_t *x, const int32_t *offsets, const int32_t *sorted_token,
                           int n_rows, int32_t *tiles, uint16_t *a16, uint16_t *x16, float *y,
                           hipStream_t s, void (*mark)(void *, const char *), void *mark_ctx,
                           const char *const names[4]);

// tile list of the grouped GEMMs: tiles of bm rows over the buckets
// (offsets [E+1]), or over rows [0, n_dense) of one dense expert (offsets null)
hipError_t launch_tile_list(int E, int n_dense, int bm, const int32_t *offsets, int32_t *tiles,
                            hipStream_t s);

// MXFP4 experts with MX-FP8 activations on the FP4 matrix instructions
// (gemm_fp4.hip): ws of a8_ws_bytes(T, H, I, n_rows) holds the quantized
// tokens and SwiGLU output; a_trace (optional, fp32 [n_rows][I]) gets the
// SwiGLU output before its quantization; names: tile list, gate/up, down,
// quantization
bool a8_supported(int H, int I, const WView &gate, const WView &up, const WView &down);
size_t a8_ws_bytes(int T, int H, int I, int n_rows);
// byte offsets, inside that region, of the SwiGLU output's E4M3 codes and scales
void a8_layout(int T, int H, int I, int n_rows, size_t *codes_off, size_t *scales_off);
hipError_t launch_a8_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                         int T, const uint16_t *x, const int32_t *offsets,
                         const int32_t *sorted_token, int n_rows, int32_t *tiles, void *ws,
                         float *a_trace, float *y, hipStream_t s,
                         void (*mark)(void *, const char *), void *mark_ctx,
                         const char *const names[4]);
hipError_t launch_mx8_quant(int rows, int K, const uint16_t *x, uint8_t *q, uint8_t *sc,
                            hipStream_t s);

// dense one-expert FFN of T <= 64 rows with bf16 weights (a small batch's
// shared expert): a16 fp16 [T][I], y fp32 [T][H]
bool skinny_supported(int H, int I, int T, const WView &gate, const WView &down);
hipError_t launch_skinny_ffn(const WView &gate, const WView &up, const WView &down, int H, int I,
                             int T, const uint16_t *x, uint16_t *a16, float *y, hipStream_t s,
                             void (*mark)(void *, const char *), void *mark_ctx,
                             const char *const names[4]);

// fused batch-1 decode (decode.hip) ------------------------------------------
struct DecodeArgs {
  int H, I, E, k, Is, mode;
  const uint16_t *x;         // [H] bf16
  const uint16_t *w_router;  // [E][H] bf16
  const float *logits_in;    // optional [E]
  const int64_t *tid;        // [1], hash routing
  WView gate, up, down;      // routed experts
  WView sg, su, sd;          // shared expert (bf16), when Is > 0
  float *logits;             // [E]
  float *a_sh;               // [Is] (also holds a_sh_hi / a_sh_lo)
  uint16_t *a_sh_hi, *a_sh_lo;  // [Is] bf16 split of the shared SwiGLU output
  float *a;                  // [k][I] (also holds a_hi / a_lo)
  uint16_t *a_hi, *a_lo;     // [k][I] bf16 split of the routed SwiGLU output
  int a_mode;                // how a is stored (set by launch_decode1)
  int32_t *topk_idx;         // [k]
  float *topk_w;             // [k]
  float *shared_y;           // [H] shared expert output (written by p2)
  float *out;                // [H]
  uint16_t *out_bf16;        // optional [H]
  const float *steer_dir;    // optional [H]: out += steer_alpha * steer_dir
  float steer_alpha;
  const int32_t *slot_idx;   // optional [k]: weight index of choice j (expert cache slots);
                             // p2 then takes it instead of selecting
  int nb_router, nb_shared_gu, nb_routed, tiles_per_expert;
};

bool decode1_supported(int H, int I, int Is, int k);
struct CacheStep;
// p1, then (with a cache) the cache's plan and fill, then p2 and p3
hipError_t launch_decode1(DecodeArgs a, hipStream_t s, void (*mark)(void *, const char *),
                          void *mark_ctx, const CacheStep *cache = nullptr);

// routed-expert residency cache (cache.hip) ----------------------------------
struct CacheStep {
  int mode, E, C, k;
  const float *logits;
  const int64_t *tid;
  int32_t *state;       // cache_state_ints(E, C) ints
  int32_t *topk_idx;    // [k]
  float *topk_w;        // [k]
  int n_planes;         // byte planes of an expert: gate/up/down data and scales
  const uint8_t *src[6];  // host planes of all E experts (device-accessible pointers)
  uint8_t *dst[6];        // slot planes of the C slots
  size_t per_bytes[6];    // bytes of one expert in each plane (multiples of 16)
};
size_t cache_state_ints(int E, int C);
int cache_slot_idx_offset(int E, int C);
hipError_t launch_cache_reset(int E, int C, int32_t *state, hipStream_t s);
hipError_t launch_cache_step(const CacheStep &c, hipStream_t s,
                             void (*mark)(void *, const char *), void *mark_ctx);

// combine -----------------------------------------------------------------
hipError_t launch_combine(int T, int H, int k, const float *y_rows, const int32_t *slot_pos,
                          const float *w, const float *shared_y, const float *steer_dir,
                          float steer_alpha, float *out, uint16_t *out_bf16, hipStream_t s);

}  // namespace moe
