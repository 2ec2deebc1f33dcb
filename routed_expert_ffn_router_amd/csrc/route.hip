// route.hip -- router logits, expert selection and slot bucketing.
//
// Router (kept at full precision on the ds4 pages: dibi8.com guide "Key
// innovations" item 1, hysenlabs.com "Model support and quantization"):
//   logits[t][e] = sum_h x[t][h] * Wr[e][h]
// Each bf16 x bf16 product is exact in fp64 and, for activations and router
// weights of ordinary range, so is every partial sum, so the fp64 result does
// not depend on the summation order; it is rounded once to fp32.  This makes
// the logits -- and therefore the selected experts -- reproducible bit for bit.
//
// Selection: softmax top-k (ties to the lower expert index) or SplitMix64 hash
// routing (grapeot.me ds4 post: V4 Flash uses hash MoE routing); weights are
// the softmax of the selected logits.
//
// Bucketing: a counting sort of the T*k slots by expert, stable in slot order.
#include "select.h"

namespace moe {

// ----------------------------------------------------------------------------
// router logits
// ----------------------------------------------------------------------------

__device__ __forceinline__ double dot8_bf16_f64(uint4 a, uint4 b) {
  double s = (double)bf16_lo(a.x) * (double)bf16_lo(b.x);
  s = fma((double)bf16_hi(a.x), (double)bf16_hi(b.x), s);
  s = fma((double)bf16_lo(a.y), (double)bf16_lo(b.y), s);
  s = fma((double)bf16_hi(a.y), (double)bf16_hi(b.y), s);
  s = fma((double)bf16_lo(a.z), (double)bf16_lo(b.z), s);
  s = fma((double)bf16_hi(a.z), (double)bf16_hi(b.z), s);
  s = fma((double)bf16_lo(a.w), (double)bf16_lo(b.w), s);
  s = fma((double)bf16_hi(a.w), (double)bf16_hi(b.w), s);
  return s;
}

// one wave per logit; lanes stride over h in 8-element chunks (H % 8 == 0)
__global__ __launch_bounds__(256) void k_router_gemv(int T, int H, int E,
                                                      const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      float *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int o = blockIdx.x * 4 + (threadIdx.x >> 6); o < T * E; o += nw) {
    const int t = o / E, e = o - t * E;
    const uint16_t *xr = x + (size_t)t * H;
    const uint16_t *wrow = wr + (size_t)e * H;
    double acc = 0.0;
    for (int h = lane * 8; h < H; h += 512)
      acc += dot8_bf16_f64(*reinterpret_cast<const uint4 *>(xr + h),
                           *reinterpret_cast<const uint4 *>(wrow + h));
    acc = group_sum_f64<64>(acc);
    if (lane == 0) logits[(size_t)t * E + e] = (float)acc;
  }
}

// tiled fp64 GEMM for many tokens: 32 tokens x 64 experts per block, each
// thread 2 x 4 outputs, K staged through LDS as fp64 in chunks of 16.
__global__ __launch_bounds__(256) void k_router_gemm(int T, int H, int E,
                                                      const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      float *__restrict__ logits) {
  __shared__ double xs[16][33];
  __shared__ double ws[16][65];
  const int t0 = blockIdx.y * 32, e0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  double acc[2][4] = {};
  for (int k0 = 0; k0 < H; k0 += 16) {
    for (int i = tid; i < 32 * 16; i += 256) {
      const int tt = i >> 4, kk = i & 15, t = t0 + tt;
      xs[kk][tt] = (t < T && k0 + kk < H) ? (double)bf16_bits_to_f32(x[(size_t)t * H + k0 + kk]) : 0.0;
    }
    for (int i = tid; i < 64 * 16; i += 256) {
      const int ee = i >> 4, kk = i & 15, e = e0 + ee;
      ws[kk][ee] = (e < E && k0 + kk < H) ? (double)bf16_bits_to_f32(wr[(size_t)e * H + k0 + kk]) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; kk++) {
      const double a0 = xs[kk][ty * 2], a1 = xs[kk][ty * 2 + 1];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const double b = ws[kk][tx * 4 + j];
        acc[0][j] = fma(a0, b, acc[0][j]);
        acc[1][j] = fma(a1, b, acc[1][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int t = t0 + ty * 2 + i, e = e0 + tx * 4 + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = (float)acc[i][j];
    }
}

// fp64 matrix cores for many tokens.  v_mfma_f64_16x16x4f64 takes A[l%16][l/16]
// and B[l/16][l%16] from lane l and leaves D[4r + l/16][l%16] in its result
// register r.  Which h the MFMA's reduction slot of a lane stands for is free
// (the fp64 sum does not depend on the order): lane group g = l/16 feeds
// h = h0 + 8g + s at step s, so each lane reads 8 consecutive bf16 of its row.
// Block: 4 waves = 32 tokens x 64 experts; a wave holds 16 tokens x 32 experts
// as two MFMA tiles, each split over two accumulators (even and odd steps) so
// four independent chains fill the pipe.  H % 32 == 0, E % 64 == 0.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_router_mfma(int T, int H, int E,
                                                      const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ wr,
                                                      float *__restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.y * 32 + 16 * (wave & 1);
  const int e0 = blockIdx.x * 64 + 32 * (wave >> 1);
  const int ta = min(t0 + r, T - 1);  // rows past T repeat the last token and are not stored
  const uint4 *xa = reinterpret_cast<const uint4 *>(x + (size_t)ta * H + 8 * g);
  const uint4 *wb0 = reinterpret_cast<const uint4 *>(wr + (size_t)(e0 + r) * H + 8 * g);
  const uint4 *wb1 = reinterpret_cast<const uint4 *>(wr + (size_t)(e0 + 16 + r) * H + 8 * g);
  f64x4_t c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0}, d0 = {0, 0, 0, 0}, d1 = {0, 0, 0, 0};
  const int n = H / 32;
  // a ring of kP steps in flight: one step of MFMAs alone is far shorter than
  // a memory round trip, and a block holds one wave per SIMD
  constexpr int kP = 4;
  uint4 a[kP], b0[kP], b1[kP];
#pragma unroll
  for (int u = 0; u < kP; u++) {
    const int i = min(u, n - 1);
    a[u] = xa[4 * i], b0[u] = wb0[4 * i], b1[u] = wb1[4 * i];
  }
  for (int i0 = 0; i0 < n; i0 += kP) {
#pragma unroll
    for (int u = 0; u < kP; u++) {
      if (i0 + u < n) {
        const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
        const uint32_t bv0[4] = {b0[u].x, b0[u].y, b0[u].z, b0[u].w};
        const uint32_t bv1[4] = {b1[u].x, b1[u].y, b1[u].z, b1[u].w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const double alo = bf16_lo(av[j]), ahi = bf16_hi(av[j]);
          c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(alo, (double)bf16_lo(bv0[j]), c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(alo, (double)bf16_lo(bv1[j]), c1, 0, 0, 0);
          d0 = __builtin_amdgcn_mfma_f64_16x16x4f64(ahi, (double)bf16_hi(bv0[j]), d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f64_16x16x4f64(ahi, (double)bf16_hi(bv1[j]), d1, 0, 0, 0);
        }
      }
      // refill the slot (past the end: the last step again, never used)
      const int i = min(i0 + u + kP, n - 1);
      a[u] = xa[4 * i], b0[u] = wb0[4 * i], b1[u] = wb1[4 * i];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int t = t0 + 4 * q + g;
    if (t < T) {
      logits[(size_t)t * E + e0 + r] = (float)(c0[q] + d0[q]);
      logits[(size_t)t * E + e0 + 16 + r] = (float)(c1[q] + d1[q]);
    }
  }
}

hipError_t launch_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *wr,
                                float *logits, hipStream_t s) {
  if (T <= 8) {
    const int waves = T * E;
    const int blocks = (waves + 3) / 4;
    return launch(k_router_gemv, dim3(blocks), dim3(256), s, T, H, E, x, wr, logits);
  }
  if (E % 64 == 0 && H % 32 == 0)
    return launch(k_router_mfma, dim3(E / 64, (T + 31) / 32), dim3(256), s, T, H, E, x, wr,
                  logits);
  dim3 grid((E + 63) / 64, (T + 31) / 32);
  return launch(k_router_gemm, dim3(grid), dim3(256), s, T, H, E, x, wr, logits);
}

// ----------------------------------------------------------------------------
// screened router logits (many tokens; for the selection only)
// ----------------------------------------------------------------------------
// The selection needs exact logits only for the experts that can reach the
// top k.  An fp32 approximation L~ from the bf16 matrix cores, with a rigorous
// error bound delta, names the candidates
//   C = { e : L~_e >= L~_(k) - 2 delta }     (L~_(k): the k-th largest L~)
// and only their logits are computed exactly (fp64, as above); the others are
// written as -inf.  An expert outside C has an exact, fp32-rounded logit
// strictly below those of k experts in C, so it is outside the top k of the
// full row whatever the tie rule, and the top k of the full row -- finite or
// +inf, so above -inf -- are all in C: the selection and its softmax weights
// are those of the full row, bit for bit.
//
// The bound.  A product of two bf16 is exact in fp32.  Any summation of H such
// products with a unit roundoff u <= 2^-23 per step (rounded or truncated)
// errs by at most gamma * sum |x_h w_h|, gamma = H u / (1 - H u) <= H 2^-22
// while H u <= 1/2, and sum |x_h w_h| <= |x| |w_e| (Cauchy-Schwarz); flushed
// subnormal products or partial sums add below 2 H 2^-126.  Rounding the exact
// value L to fp32 moves it by at most 2^-24 |L| + 2^-150, and |L| <= max |L~| +
// eps.  delta takes each of these twice.  |w_e|^2 comes from the approximation
// kernel in fp32 (v_dot2, the same kind of bound), |x|^2 is summed in fp64.  A
// row with a non-finite approximation, or one whose logits could leave the fp32
// range, takes every expert as a candidate; in hash mode the candidates are the
// k hashed experts and no approximation is made.

typedef __bf16 bf16x8_rt __attribute__((ext_vector_type(8)));
typedef float f32x16_rt __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_rt mfma_bf16_32(uint4 a, uint4 b, f32x16_rt c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_rt, a),
                                                 __builtin_bit_cast(bf16x8_rt, b), c, 0, 0, 0);
}
__device__ __forceinline__ float sumsq8_bf16(uint4 v, float s) {
  s = dot2_bf16(v.x, v.x, s);
  s = dot2_bf16(v.y, v.y, s);
  s = dot2_bf16(v.z, v.z, s);
  return dot2_bf16(v.w, v.w, s);
}

// Approximate logits: block (bx, by) = tokens 32 by + [0, 32) x experts
// 64 bx + [0, 64); its four waves take a quarter of H each and their partial
// tiles are added in LDS in a fixed order.  v_mfma_f32_32x32x16_bf16 takes
// A[l%32][8(l/32) + i] and B[8(l/32) + i][l%32] (i < 8) from lane l and leaves
// D[8(q/4) + 4(l/32) + q%4][l%32] in its result register q.  The blocks of the
// first token tile also write sum_h w[e][h]^2 for their experts into wn2.
// E % 64 == 0, H % 64 == 0.
__global__ __launch_bounds__(256) void k_router_approx(int T, int H, int E,
                                                        const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wr,
                                                        float *__restrict__ logits,
                                                        float *__restrict__ wn2) {
  __shared__ float red[4][32][64];
  __shared__ float nrm[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.y * 32, e0 = blockIdx.x * 64;
  const int hq = H / 4, h0 = wave * hq + 8 * g;
  const int ta = min(t0 + r, T - 1);  // rows past T repeat the last token and are not stored
  const uint4 *xa = reinterpret_cast<const uint4 *>(x + (size_t)ta * H + h0);
  const uint4 *wb0 = reinterpret_cast<const uint4 *>(wr + (size_t)(e0 + r) * H + h0);
  const uint4 *wb1 = reinterpret_cast<const uint4 *>(wr + (size_t)(e0 + 32 + r) * H + h0);
  const bool norms = blockIdx.y == 0;
  const int n = hq / 16;
  f32x16_rt c0 = {}, c1 = {};
  float s0 = 0.0f, s1 = 0.0f;
  constexpr int kP = 8;  // steps in flight
  uint4 a[kP], b0[kP], b1[kP];
#pragma unroll
  for (int u = 0; u < kP; u++) {
    const int i = min(u, n - 1);
    a[u] = xa[2 * i], b0[u] = wb0[2 * i], b1[u] = wb1[2 * i];
  }
  for (int i0 = 0; i0 < n; i0 += kP) {
#pragma unroll
    for (int u = 0; u < kP; u++) {
      if (i0 + u < n) {
        c0 = mfma_bf16_32(a[u], b0[u], c0);
        c1 = mfma_bf16_32(a[u], b1[u], c1);
        if (norms) {
          s0 = sumsq8_bf16(b0[u], s0);
          s1 = sumsq8_bf16(b1[u], s1);
        }
      }
      const int i = min(i0 + u + kP, n - 1);
      a[u] = xa[2 * i], b0[u] = wb0[2 * i], b1[u] = wb1[2 * i];
    }
  }
#pragma unroll
  for (int q = 0; q < 16; q++) {
    red[wave][q][lane] = c0[q];
    red[wave][16 + q][lane] = c1[q];
  }
  if (norms) {
    s0 += __shfl_xor(s0, 32, 64);
    s1 += __shfl_xor(s1, 32, 64);
    nrm[wave][lane] = lane < 32 ? s0 : s1;  // lane j: expert e0 + j
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; q++) {
    const int reg = 8 * wave + q, i = reg & 15;
    const float v = ((red[0][reg][lane] + red[1][reg][lane]) + red[2][reg][lane]) + red[3][reg][lane];
    const int t = t0 + 8 * (i >> 2) + 4 * g + (i & 3);
    if (t < T) logits[(size_t)t * E + e0 + 32 * (reg >> 4) + r] = v;
  }
  if (norms && wave == 0)
    wn2[e0 + lane] = ((nrm[0][lane] + nrm[1][lane]) + nrm[2][lane]) + nrm[3][lane];
}

__device__ __forceinline__ double dot8_bf16_f64_acc(uint4 a, uint4 b, double s) {
  s = fma((double)bf16_lo(a.x), (double)bf16_lo(b.x), s);
  s = fma((double)bf16_hi(a.x), (double)bf16_hi(b.x), s);
  s = fma((double)bf16_lo(a.y), (double)bf16_lo(b.y), s);
  s = fma((double)bf16_hi(a.y), (double)bf16_hi(b.y), s);
  s = fma((double)bf16_lo(a.z), (double)bf16_lo(b.z), s);
  s = fma((double)bf16_hi(a.z), (double)bf16_hi(b.z), s);
  s = fma((double)bf16_lo(a.w), (double)bf16_lo(b.w), s);
  return fma((double)bf16_hi(a.w), (double)bf16_hi(b.w), s);
}

// One wave per token: the candidates, their exact logits, -inf elsewhere,
// written over the approximate row.  H = 512 NJ (lane l holds h = 8 l +
// 512 j + [0, 8) of x), E % 64 == 0 and E <= 256 (expert lane + 64 i in slot i).
template <int NJ>
__global__ __launch_bounds__(256) void k_router_screen(int mode, int T, int E, int k,
                                                        const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wr,
                                                        const float *__restrict__ wn2,
                                                        const int64_t *__restrict__ tids,
                                                        float *__restrict__ logits) {
  constexpr int H = 512 * NJ;
  constexpr int G = NJ <= 8 ? 4 : 2;  // candidates per pass
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nc = E >> 6;
  float *row = logits + (size_t)t * E;
  uint4 xr[NJ];
  const uint4 *xp = reinterpret_cast<const uint4 *>(x + (size_t)t * H) + lane;
#pragma unroll
  for (int j = 0; j < NJ; j++) xr[j] = xp[64 * j];
  uint32_t cm = 0;  // bit i: expert lane + 64 i is a candidate
  if (mode == MOE_ROUTE_HASH) {
    const uint64_t z = splitmix64((uint64_t)tids[t]);
    for (int j = 0; j < k; j++) {
      const int e = (int)((z + (uint64_t)j) % (uint64_t)E);
      if ((e & 63) == lane) cm |= 1u << (e >> 6);
    }
  } else {
    float v[4];
    bool bad = false;
    float amax = 0.0f, wmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[i] = i < nc ? row[lane + 64 * i] : -INFINITY;
      if (i < nc) {
        bad |= !__builtin_isfinite(v[i]);
        amax = fmaxf(amax, fabsf(v[i]));
        wmax = fmaxf(wmax, wn2[lane + 64 * i]);
      }
    }
    double sx = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; j++) sx = dot8_bf16_f64_acc(xr[j], xr[j], sx);
    sx = group_sum_f64<64>(sx);
    const float M = wave_max_f(amax), W = wave_max_f(wmax);
    const double gam = (double)H * 0x1p-22;
    const double wb = ((double)W + (double)H * 0x1p-125) * (1.0 + 2.0 * gam);
    const double S = sqrt(sx * wb) * (1.0 + 0x1p-40);
    const double eps = gam * S + (double)H * 0x1p-125;
    const double delta = eps + 0x1p-23 * ((double)M + eps) + 0x1p-149;
    // also false for a NaN or infinite delta
    const bool screen = __ballot(bad) == 0 && (double)M + 2.0 * delta < 0x1p127;
    if (!screen) {
      cm = (1u << nc) - 1u;
    } else {
      // the k-th largest approximate logit: each lane sorts its (at most four)
      // values as order-preserving integer keys, then k rounds pop the
      // largest head
      int key[4];
#pragma unroll
      for (int i = 0; i < 4; i++) key[i] = float_key(v[i] + 0.0f);
      auto order = [&](int p, int q) {
        const int hi = max(key[p], key[q]), lo = min(key[p], key[q]);
        key[p] = hi, key[q] = lo;
      };
      order(0, 1);
      order(2, 3);
      order(0, 2);
      order(1, 3);
      order(1, 2);
      int kth = 0;
      for (int j = 0; j < k; j++) {
        kth = wave_max_all(key[0]);
        const uint64_t at = __ballot(key[0] == kth);
        if (lane == __builtin_ctzll(at)) {
          key[0] = key[1], key[1] = key[2], key[2] = key[3];
          key[3] = float_key(-INFINITY);
        }
      }
      const double tau = (double)key_float(kth) - 2.0 * delta;
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (i < nc && (double)v[i] >= tau) cm |= 1u << i;
    }
  }
  // the candidates in expert order, G per pass, from the slot ballots
  uint64_t m0 = __ballot(cm & 1u), m1 = __ballot(cm & 2u), m2 = __ballot(cm & 4u),
           m3 = __ballot(cm & 8u);
  auto next = [&]() -> int {
    if (m0) { const int b = __builtin_ctzll(m0); m0 &= m0 - 1; return b; }
    if (m1) { const int b = __builtin_ctzll(m1); m1 &= m1 - 1; return 64 + b; }
    if (m2) { const int b = __builtin_ctzll(m2); m2 &= m2 - 1; return 128 + b; }
    if (m3) { const int b = __builtin_ctzll(m3); m3 &= m3 - 1; return 192 + b; }
    return -1;
  };
  float ex[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  int e_next = next();
  while (e_next >= 0) {
    int ids[G];
    ids[0] = e_next;
#pragma unroll
    for (int u = 1; u < G; u++) {
      const int e = next();
      ids[u] = e >= 0 ? e : ids[u - 1];  // a repeat past the end: same value again
    }
    e_next = next();
    double acc[G];
#pragma unroll
    for (int u = 0; u < G; u++) acc[u] = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; j++)
#pragma unroll
      for (int u = 0; u < G; u++) {
        const uint4 wv = reinterpret_cast<const uint4 *>(wr + (size_t)ids[u] * H)[lane + 64 * j];
        acc[u] = dot8_bf16_f64_acc(xr[j], wv, acc[u]);
      }
#pragma unroll
    for (int u = 0; u < G; u++) {
      const double s = group_sum_f64<64>(acc[u]);
      if ((ids[u] & 63) == lane) {
        const int sl = ids[u] >> 6;
        const float f = (float)s;
        ex[0] = sl == 0 ? f : ex[0];
        ex[1] = sl == 1 ? f : ex[1];
        ex[2] = sl == 2 ? f : ex[2];
        ex[3] = sl == 3 ? f : ex[3];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (i < nc) row[lane + 64 * i] = ex[i];
}

bool router_screen_supported(int H, int E) {
  return E % 64 == 0 && E <= 256 && H % 512 == 0 && H >= 512 && H <= 8192;
}

template <int NJ>
static hipError_t launch_screen_nj(int mode, int T, int E, int k, const uint16_t *x,
                                   const uint16_t *wr, const float *wn2, const int64_t *tids,
                                   float *logits, hipStream_t s) {
  return launch(k_router_screen<NJ>, dim3((T + 3) / 4), dim3(256), s, mode, T, E, k, x, wr, wn2,
                tids, logits);
}

hipError_t launch_router_screened(int mode, int T, int H, int E, int k, const uint16_t *x,
                                  const uint16_t *wr, const int64_t *tids, float *logits,
                                  float *wn2, hipStream_t s) {
  if (!router_screen_supported(H, E)) return hipErrorInvalidValue;
  if (mode != MOE_ROUTE_HASH) {
    const hipError_t e = launch(k_router_approx, dim3(E / 64, (T + 31) / 32), dim3(256), s, T, H,
                                E, x, wr, logits, wn2);
    if (e != hipSuccess) return e;
  }
  switch (H / 512) {
#define MOE_SCREEN_CASE(n) \
  case n: return launch_screen_nj<n>(mode, T, E, k, x, wr, wn2, tids, logits, s);
    MOE_SCREEN_CASE(1) MOE_SCREEN_CASE(2) MOE_SCREEN_CASE(3) MOE_SCREEN_CASE(4)
    MOE_SCREEN_CASE(5) MOE_SCREEN_CASE(6) MOE_SCREEN_CASE(7) MOE_SCREEN_CASE(8)
    MOE_SCREEN_CASE(9) MOE_SCREEN_CASE(10) MOE_SCREEN_CASE(11) MOE_SCREEN_CASE(12)
    MOE_SCREEN_CASE(13) MOE_SCREEN_CASE(14) MOE_SCREEN_CASE(15) MOE_SCREEN_CASE(16)
#undef MOE_SCREEN_CASE
  }
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// selection
// ----------------------------------------------------------------------------

// selection only: one wave per token
__global__ __launch_bounds__(256) void k_select(int mode, int T, int E, int k,
                                                 const float *__restrict__ logits,
                                                 const int64_t *__restrict__ tids,
                                                 int32_t *__restrict__ idx, float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int e;
  float wt;
  select_wave(mode, E, k, logits + (size_t)t * E, tids ? tids[t] : 0, &e, &wt);
  if (lane < k) {
    idx[(size_t)t * k + lane] = e;
    w[(size_t)t * k + lane] = wt;
  }
}

// exclusive prefix sum over a 1024-thread block; returns the prefix of v,
// *total gets the block sum.  tmp: 16 ints of shared memory.
__device__ int block_excl_scan_1024(int v, int *tmp, int *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int c = tmp[i];
    base += i < wv ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Selection of all T tokens plus bucketing of the n = T*k <= 1024 slots in
// one 1024-thread block (the decode path: no second launch for dispatch).
__global__ __launch_bounds__(1024) void k_select_plan(
    int mode, int T, int E, int k, const float *__restrict__ logits,
    const int64_t *__restrict__ tids, int32_t *__restrict__ idx, float *__restrict__ w,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_token,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_pos, float *__restrict__ row_w,
    int32_t *__restrict__ plan) {
  __shared__ int s_e[kSmallSlots];
  __shared__ float s_w[kSmallSlots];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_off[kMaxE];
  __shared__ int s_tmp[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = T * k;
  for (int t = wv; t < T; t += 16) {
    int e;
    float wt;
    select_wave(mode, E, k, logits + (size_t)t * E, tids ? tids[t] : 0, &e, &wt);
    if (lane < k) {
      s_e[t * k + lane] = e;
      s_w[t * k + lane] = wt;
      idx[(size_t)t * k + lane] = e;
      w[(size_t)t * k + lane] = wt;
    }
  }
  for (int e = threadIdx.x; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  if ((int)threadIdx.x < n) atomicAdd(&s_cnt[s_e[threadIdx.x]], 1);
  __syncthreads();
  const int e = threadIdx.x;
  const int c = e < E ? s_cnt[e] : 0;
  int total, n_active;
  const int off = block_excl_scan_1024(c, s_tmp, &total);
  const int apos = block_excl_scan_1024(c > 0 ? 1 : 0, s_tmp, &n_active);
  if (e < E) {
    s_off[e] = off;
    if (offsets) offsets[e] = off;
    if (c > 0 && plan) {
      plan[1 + 3 * apos] = e;
      plan[2 + 3 * apos] = off;
      plan[3 + 3 * apos] = off + c;
    }
  }
  if (e == 0) {
    if (offsets) offsets[E] = n;
    if (plan) plan[0] = n_active;
  }
  __syncthreads();
  const int f = threadIdx.x;
  if (f < n) {
    const int ef = s_e[f];
    int rank = 0;
    for (int g = 0; g < f; g++) rank += s_e[g] == ef;
    const int r = s_off[ef] + rank;
    sorted_token[r] = f / k;
    if (sorted_slot) sorted_slot[r] = f;
    if (slot_pos) slot_pos[f] = r;
    if (row_w) row_w[r] = s_w[f];
  }
}

hipError_t launch_select(int mode, int T, int E, int k, const float *logits,
                         const int64_t *token_ids, int32_t *idx, float *w, int32_t *offsets,
                         int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos,
                         float *row_w, int32_t *plan, hipStream_t s) {
  if (sorted_token)
    return launch(k_select_plan, dim3(1), dim3(1024), s, mode, T, E, k, logits, token_ids, idx, w,
                  offsets, sorted_token, sorted_slot, slot_pos, row_w, plan);
  return launch(k_select, dim3((T + 3) / 4), dim3(256), s, mode, T, E, k, logits, token_ids, idx,
                w);
}

// ----------------------------------------------------------------------------
// dispatch for any number of slots: per-chunk counts -> scan -> stable scatter
// ----------------------------------------------------------------------------

constexpr int kChunk = 256;

__global__ __launch_bounds__(kChunk) void k_chunk_counts(int n, int E, const int32_t *__restrict__ idx,
                                                          int32_t *__restrict__ counts) {
  __shared__ int s_cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += kChunk) s_cnt[e] = 0;
  __syncthreads();
  const int f = blockIdx.x * kChunk + threadIdx.x;
  if (f < n) atomicAdd(&s_cnt[idx[f]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) counts[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// one 1024-thread block: thread e sums the chunk counts of expert e, a scan
// over experts gives the bucket starts, then thread e rewrites its chunks'
// counts as global starts.  Counts are read kBatch at a time before any
// store, so each pass waits for memory nchunks / kBatch times, not nchunks.
__global__ __launch_bounds__(1024) void k_chunk_scan(int n, int nchunks, int E,
                                                      int32_t *__restrict__ counts,
                                                      int32_t *__restrict__ offsets) {
  constexpr int kBatch = 16;
  __shared__ int s_tmp[16];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E)
    for (int b0 = 0; b0 < nchunks; b0 += kBatch) {
#pragma unroll
      for (int j = 0; j < kBatch; j++)
        tot += b0 + j < nchunks ? counts[(size_t)(b0 + j) * E + e] : 0;
    }
  int total;
  const int off = block_excl_scan_1024(e < E ? tot : 0, s_tmp, &total);
  if (e < E) {
    offsets[e] = off;
    int run = off;
    for (int b0 = 0; b0 < nchunks; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; j++) c[j] = b0 + j < nchunks ? counts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; j++)
        if (b0 + j < nchunks) {
          counts[(size_t)(b0 + j) * E + e] = run;
          run += c[j];
        }
    }
  }
  if (e == 0) offsets[E] = n;
}

__global__ __launch_bounds__(kChunk) void k_chunk_scatter(int n, int E, int k,
                                                           const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ base,
                                                           int32_t *__restrict__ sorted_token,
                                                           int32_t *__restrict__ sorted_slot,
                                                           int32_t *__restrict__ slot_pos) {
  __shared__ int s_e[kChunk];
  const int f0 = blockIdx.x * kChunk;
  const int f = f0 + threadIdx.x;
  s_e[threadIdx.x] = f < n ? idx[f] : -1;
  __syncthreads();
  if (f < n) {
    const int ef = s_e[threadIdx.x];
    int rank = 0;
    for (int g = 0; g < (int)threadIdx.x; g++) rank += s_e[g] == ef;
    const int r = base[(size_t)blockIdx.x * E + ef] + rank;
    sorted_token[r] = f / k;
    if (sorted_slot) sorted_slot[r] = f;
    if (slot_pos) slot_pos[f] = r;
  }
}

size_t dispatch_ws_bytes(int T, int E, int k) {
  const size_t n = (size_t)T * k;
  const size_t nchunks = (n + kChunk - 1) / kChunk;
  return nchunks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_dispatch(int T, int E, int k, const int32_t *idx, int32_t *offsets,
                           int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos,
                           void *ws, hipStream_t s, void (*mark)(void *, const char *),
                           void *mark_ctx) {
  const int n = T * k;
  const int nchunks = (n + kChunk - 1) / kChunk;
  int32_t *counts = static_cast<int32_t *>(ws);
  if (mark) mark(mark_ctx, "dispatch_counts");
  hipError_t err = launch(k_chunk_counts, dim3(nchunks), dim3(kChunk), s, n, E, idx, counts);
  if (err != hipSuccess) return err;
  if (mark) mark(mark_ctx, "dispatch_scan");
  err = launch(k_chunk_scan, dim3(1), dim3(1024), s, n, nchunks, E, counts, offsets);
  if (err != hipSuccess) return err;
  if (mark) mark(mark_ctx, "dispatch_scatter");
  return launch(k_chunk_scatter, dim3(nchunks), dim3(kChunk), s, n, E, k, idx, counts,
                sorted_token, sorted_slot, slot_pos);
}

// compact plan from offsets: one 1024-thread block (E <= 1024)
__global__ __launch_bounds__(1024) void k_plan_from_offsets(int E, const int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ plan) {
  __shared__ int s_tmp[16];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  int n_active;
  const int apos = block_excl_scan_1024(c > 0 ? 1 : 0, s_tmp, &n_active);
  if (c > 0) {
    plan[1 + 3 * apos] = e;
    plan[2 + 3 * apos] = offsets[e];
    plan[3 + 3 * apos] = offsets[e + 1];
  }
  if (e == 0) plan[0] = n_active;
}

hipError_t launch_plan_from_offsets(int E, const int32_t *offsets, int32_t *plan, hipStream_t s) {
  return launch(k_plan_from_offsets, dim3(1), dim3(1024), s, E, offsets, plan);
}

}  // namespace moe
