// select.h -- expert selection for one token by one wavefront.
//
// Softmax top-k: the k largest logits in descending order, equal logits
// going to the lower expert index, NaN ranking as -inf; hash routing (the
// grapeot.me ds4 post lists hash MoE routing among V4 Flash's features):
// expert j = ((splitmix64(token_id) + j) mod 2^64) mod E.  Weights are the
// softmax over the k selected logits.
#pragma once
#include "gemv_core.h"

namespace moe {

constexpr int kMaxE = 1024;

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014, finaliser Mix13 by
// Stafford): increment by the golden gamma, then mix.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float order_val(float v) { return v != v ? -INFINITY : v; }

// Lane j < k returns choice j in (*e_out, *w_out); other lanes get e = -1.
// E <= kMaxE; every lane of the wave must call this.
__device__ __forceinline__ void select_wave(int mode, int E, int k, const float *__restrict__ l,
                                            int64_t tid, int *e_out, float *w_out) {
  const int lane = threadIdx.x & 63;
  int my_e = -1;
  float my_l = -INFINITY;
  if (mode == MOE_ROUTE_HASH) {
    const uint64_t z = splitmix64((uint64_t)tid);
    if (lane < k) {
      my_e = (int)((z + (uint64_t)lane) % (uint64_t)E);
      my_l = l[my_e];
    }
  } else {
    constexpr int NC = kMaxE / 64;
    float v[NC];
    uint32_t taken = 0;  // bit i: candidate lane + 64 i is taken or absent
#pragma unroll
    for (int i = 0; i < NC; i++) {
      const int e = lane + 64 * i;
      v[i] = e < E ? order_val(l[e]) : -INFINITY;
      if (e >= E) taken |= 1u << i;
    }
    for (int j = 0; j < k; j++) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < NC; i++) {
        const bool free_ = !((taken >> i) & 1u);
        if (free_ && (bi == 0x7FFFFFFF || v[i] > bv)) {
          bv = v[i];
          bi = lane + 64 * i;
        }
      }
      const float m = wave_max_f(bv);
      const int e = wave_min_i((bi != 0x7FFFFFFF && bv == m) ? bi : 0x7FFFFFFF);
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
      if (lane == j) {
        my_e = e;
        my_l = l[e];
      }
    }
  }
  const float mine = lane < k ? order_val(my_l) : -INFINITY;
  const float m = wave_max_f(mine);
  const float ex = lane < k ? expf(mine - m) : 0.0f;
  const float den = wave_sum_f(ex);
  *e_out = my_e;
  *w_out = ex / den;
}

}  // namespace moe
