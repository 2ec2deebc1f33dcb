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
// a signed integer with the order of the (non-NaN) float, and back; -0 and +0
// get different keys, so callers pass +0 for both
__device__ __forceinline__ int float_key(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float key_float(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }

// The logits a wave needs for one token, loaded up front so that the selection
// costs one memory round trip: candidate e = lane + 64 i sits in v[i].
template <int NC>
struct Logits {
  float v[NC];
  // candidates past E read entry E - 1 (no branch around the loads); the
  // selection never takes them
  __device__ __forceinline__ void load(int E, const float *__restrict__ l) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NC; i++) v[i] = l[min(lane + 64 * i, E - 1)];
  }
};

// Lane j < k returns choice j in (*e_out, *w_out); other lanes get e = -1.
// E <= 64 * NC; every lane of the wave must call this.  Softmax top-k reads
// only the preloaded logits (lg); hash routing takes the k selected ones from
// lg too when E <= 64 * NC (from memory otherwise), so lg is loaded in both
// modes.
template <int NC>
__device__ __forceinline__ void select_wave(int mode, int E, int k, const Logits<NC> &lg,
                                            const float *__restrict__ l, int64_t tid, int *e_out,
                                            float *w_out) {
  const int lane = threadIdx.x & 63;
  int my_e = -1;
  float my_l = -INFINITY;
  if (mode == MOE_ROUTE_HASH) {
    const uint64_t z = splitmix64((uint64_t)tid);
    const int e = (int)((z + (uint64_t)lane) % (uint64_t)E);
    float r;
    if (E <= 64 * NC) {
      // its logit from the preloaded ones: slot e / 64 of lane e % 64
      r = 0.0f;
#pragma unroll
      for (int i = 0; i < NC; i++) {
        const float t = __shfl(lg.v[i], e & 63, 64);
        if (i == (e >> 6)) r = t;
      }
    } else {
      r = l[e];
    }
    if (lane < k) {
      my_e = e;
      my_l = r;
    }
  } else if constexpr (NC == 4) {
    // each lane sorts its four candidates once (value descending, index
    // ascending on ties; NaN and absent candidates as -inf, absent ones after
    // every present one by their index); a round then compares only the
    // lanes' heads and the winner's lane pops its head.  Values are compared
    // as integer keys with the order of the floats (-0 made +0 first, so
    // that it ties with +0), which the DPP maximum takes without the float
    // maximum's NaN handling.
    int v[4];
    int id[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      id[i] = lane + 64 * i;
      v[i] = float_key(id[i] < E ? order_val(lg.v[i]) + 0.0f : -INFINITY);
    }
    auto order = [&](int a, int b) {  // afterwards a comes before b
      const bool sw = v[b] > v[a] || (v[b] == v[a] && id[b] < id[a]);
      const int tv = v[a];
      const int ti = id[a];
      v[a] = sw ? v[b] : v[a];
      id[a] = sw ? id[b] : id[a];
      v[b] = sw ? tv : v[b];
      id[b] = sw ? ti : id[b];
    };
    order(0, 1);
    order(2, 3);
    order(0, 2);
    order(1, 3);
    order(1, 2);
    const int absent = float_key(-INFINITY);
    int my_key = absent;
    for (int j = 0; j < k; j++) {
      // the largest head, then the lowest index among heads equal to it,
      // both reduced in VALU registers (no round trips through scalars)
      const int m = wave_max_all(v[0]);
      const int e = wave_min_all(v[0] == m ? id[0] : 0x7FFFFFFF);
      const bool pop = lane == (e & 63);
      v[0] = pop ? v[1] : v[0];
      id[0] = pop ? id[1] : id[0];
      v[1] = pop ? v[2] : v[1];
      id[1] = pop ? id[2] : id[1];
      v[2] = pop ? v[3] : v[2];
      id[2] = pop ? id[3] : id[2];
      v[3] = pop ? absent : v[3];
      id[3] = pop ? 0x7FFFFFFF : id[3];
      if (lane == j) {
        my_e = e;
        my_key = m;
      }
    }
    my_l = key_float(my_key);  // already in selection-order form: NaN reads as -inf
  } else {
    float v[NC];
    uint32_t taken = 0;  // bit i: candidate lane + 64 i is taken or absent
#pragma unroll
    for (int i = 0; i < NC; i++) {
      v[i] = lane + 64 * i < E ? order_val(lg.v[i]) : -INFINITY;
      if (lane + 64 * i >= E) taken |= 1u << i;
    }
    for (int j = 0; j < k; j++) {
      // this lane's best free candidate (ties to its lower slot)
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
      // the lanes holding the maximum; one of them is the rule's choice unless
      // several tie, when the lowest expert index among them wins
      const uint64_t tied = __ballot(bi != 0x7FFFFFFF && bv == m);
      int e;
      if ((tied & (tied - 1)) == 0)
        e = __builtin_amdgcn_readlane(bi, __builtin_ctzll(tied));
      else
        e = wave_min_i((bi != 0x7FFFFFFF && bv == m) ? bi : 0x7FFFFFFF);
      const int owner = e & 63, slot = e >> 6;
      if (owner == lane) taken |= 1u << slot;
      // the raw logit of the winner: m itself unless the maximum is -inf (then
      // it may be a NaN, taken from its owner's register)
      float raw = m;
      if (m == -INFINITY) {
        float r = lg.v[0];
#pragma unroll
        for (int i = 1; i < NC; i++)
          if (i == slot) r = lg.v[i];
        raw = __shfl(r, owner, 64);
      }
      if (lane == j) {
        my_e = e;
        my_l = raw;
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

// convenience: load and select (E <= kMaxE)
__device__ __forceinline__ void select_wave(int mode, int E, int k, const float *__restrict__ l,
                                            int64_t tid, int *e_out, float *w_out) {
  if (E <= 256) {
    Logits<4> lg;
    lg.load(E, l);
    select_wave<4>(mode, E, k, lg, l, tid, e_out, w_out);
  } else {
    Logits<kMaxE / 64> lg;
    lg.load(E, l);
    select_wave<kMaxE / 64>(mode, E, k, lg, l, tid, e_out, w_out);
  }
}

}  // namespace moe
