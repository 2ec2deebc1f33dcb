// probe.hip -- measurement probes (include/moe_probe.h): a streaming HBM
// read and dense matrix-core loops, timed by the caller to give the peaks
// the layer's kernels are compared against.
#include "gemv_core.h"
#include "moe_probe.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // 16-byte loads in flight per thread

// grid-stride: block b reads chunks b, b + grid, ... of 256 threads x 4 x 16 bytes
// (indices past the end re-read the last 16 bytes: no branch around the loads)
__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const u32x4_t *__restrict__ buf,
                                                               size_t n16,
                                                               uint32_t *__restrict__ sink) {
  __shared__ uint32_t s_acc[kProbeThreads / 64];
  const size_t chunk = (size_t)kProbeThreads * kProbeUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * chunk; base < n16; base += (size_t)gridDim.x * chunk) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) {
      const size_t i = base + (size_t)u * kProbeThreads + threadIdx.x;
      v[u] = __builtin_nontemporal_load(buf + (i < n16 ? i : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // fold the block's words: the loads cannot be dropped
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; w++) r ^= s_acc[w];
    sink[blockIdx.x] = r;
  }
}

typedef __bf16 bf16x8p_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8p_t __attribute__((ext_vector_type(8)));
typedef float f32x4p_t __attribute__((ext_vector_type(4)));
typedef int i32x8p_t __attribute__((ext_vector_type(8)));
typedef float f32x16p_t __attribute__((ext_vector_type(16)));

// the 32 x 32 x 16 shapes: 4 independent accumulators of 16 registers per wave
template <int KIND>
__global__ __launch_bounds__(256) void k_probe_mfma32(int iters, float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x16p_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[i][r] = 0.f;
  const uint32_t w0 = 0x3F803F80u ^ (uint32_t)lane;
  uint4 a = make_uint4(w0, w0 + 1, w0 + 2, w0 + 3), b = make_uint4(w0 + 4, w0 + 5, w0 + 6, w0 + 7);
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (KIND == MOE_PROBE_BF16_32)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8p_t, a),
                                                         __builtin_bit_cast(bf16x8p_t, b), acc[i],
                                                         0, 0, 0);
      else
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8p_t, a),
                                                        __builtin_bit_cast(f16x8p_t, b), acc[i],
                                                        0, 0, 0);
    }
  }
  float *out = sink + ((size_t)blockIdx.x * 256 + threadIdx.x) * 32;
#pragma unroll
  for (int r = 0; r < 16; r++) out[r] = acc[0][r] + acc[1][r], out[16 + r] = acc[2][r] + acc[3][r];
}

// 8 independent accumulators per wave; operands from registers (lane-dependent
// values, so nothing folds away)
template <int KIND>
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x4p_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = (f32x4p_t){0.f, 0.f, 0.f, 0.f};
  const uint32_t w0 = 0x3F803F80u ^ (uint32_t)lane;
  uint4 a = make_uint4(w0, w0 + 1, w0 + 2, w0 + 3), b = make_uint4(w0 + 4, w0 + 5, w0 + 6, w0 + 7);
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if constexpr (KIND == MOE_PROBE_BF16)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8p_t, a),
                                                         __builtin_bit_cast(bf16x8p_t, b), acc[i],
                                                         0, 0, 0);
      else if constexpr (KIND == MOE_PROBE_F16)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8p_t, a),
                                                        __builtin_bit_cast(f16x8p_t, b), acc[i],
                                                        0, 0, 0);
      else {
        const i32x8p_t af = {(int)a.x, (int)a.y, (int)a.z, (int)a.w,
                             (int)b.x, (int)b.y, (int)b.z, (int)b.w};
        const i32x8p_t bf = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
        acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf, acc[i], 0, 4, 0, 127,
                                                                  0, 127);
      }
    }
  }
  float *out = sink + ((size_t)blockIdx.x * 256 + threadIdx.x) * 32;
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) out[4 * i + r] = acc[i][r];
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_probe_read_blocks(size_t bytes) {
  const size_t chunk = (size_t)kProbeThreads * kProbeUnroll * 16;
  const size_t need = (bytes + chunk - 1) / chunk;
  // enough workgroups to keep every CU streaming (8 per CU), not more than needed
  return (int)(need < 2048 ? (need ? need : 1) : 2048);
}

int moe_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink) return set_error(MOE_EINVAL, "probe: null buffer or sink");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return set_error(MOE_EINVAL, "probe: bytes must be a positive multiple of 16, buf aligned");
  const int blocks = moe_probe_read_blocks(bytes);
  const hipError_t e = launch(k_probe_read, dim3(blocks), dim3(kProbeThreads),
                              static_cast<hipStream_t>(stream),
                              static_cast<const u32x4_t *>(buf), bytes / 16, sink);
  if (e != hipSuccess) return set_error(MOE_EHIP, "probe read: %s", hipGetErrorString(e));
  return MOE_OK;
}

int moe_probe_mfma(int kind, int blocks, int iters, float *sink, double *flops_out,
                   void *stream) {
  if (blocks < 1 || iters < 1 || !sink) return set_error(MOE_EINVAL, "probe: bad arguments");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  double per;  // flops per instruction
  switch (kind) {
    case MOE_PROBE_BF16:
      e = launch(k_probe_mfma<MOE_PROBE_BF16>, dim3(blocks), dim3(256), s, iters, sink);
      per = 2.0 * 16 * 16 * 32;
      break;
    case MOE_PROBE_F16:
      e = launch(k_probe_mfma<MOE_PROBE_F16>, dim3(blocks), dim3(256), s, iters, sink);
      per = 2.0 * 16 * 16 * 32;
      break;
    case MOE_PROBE_BF16_32:
      e = launch(k_probe_mfma32<MOE_PROBE_BF16_32>, dim3(blocks), dim3(256), s, iters, sink);
      per = 2.0 * 32 * 32 * 16 / 2;  // 4 instructions per round: counted as 8 halves
      break;
    case MOE_PROBE_F16_32:
      e = launch(k_probe_mfma32<MOE_PROBE_F16_32>, dim3(blocks), dim3(256), s, iters, sink);
      per = 2.0 * 32 * 32 * 16 / 2;
      break;
    case MOE_PROBE_F8F4:
      e = launch(k_probe_mfma<MOE_PROBE_F8F4>, dim3(blocks), dim3(256), s, iters, sink);
      per = 2.0 * 16 * 16 * 128;
      break;
    default:
      return set_error(MOE_EINVAL, "probe: unknown kind %d", kind);
  }
  if (e != hipSuccess) return set_error(MOE_EHIP, "probe mfma: %s", hipGetErrorString(e));
  if (flops_out) *flops_out = per * 8.0 * iters * 4.0 * blocks;
  return MOE_OK;
}

}  // extern "C"
