// combine.hip -- weighted sum of the routed experts' outputs plus the shared
// expert, in gather form (one writer per output element, no atomics), and
// the optional activation-steering term (grapeot.me ds4 post, the steering
// paragraphs: a per-layer direction scaled at run time is added to the FFN
// output):
//   out[t][n] = shared_y[t][n] + sum_j w[t][j] * y_rows[slot_pos[t*k+j]][n]
//               + alpha * dir[n]
// accumulated in fp64 in that order -- each fp32 x fp32 product is exact in
// fp64, so every step is one rounded addition -- and rounded once to fp32.
// The kernel is bound by its y_rows reads; the fp64 adds cost nothing
// measurable.  Also moe_dequantize's kernel.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// block: 256 threads x 4 consecutive outputs of one token
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k,
                                                  const float *__restrict__ y_rows,
                                                  const int32_t *__restrict__ slot_pos,
                                                  const float *__restrict__ w,
                                                  const float *__restrict__ shared_y,
                                                  const float *__restrict__ dir, float alpha,
                                                  float *__restrict__ out,
                                                  uint16_t *__restrict__ out_bf16) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (shared_y) {
    const float4 s = *reinterpret_cast<const float4 *>(shared_y + (size_t)t * H + n);
    acc[0] = s.x, acc[1] = s.y, acc[2] = s.z, acc[3] = s.w;
  }
  for (int j = 0; j < k; j++) {
    const double wj = w[(size_t)t * k + j];
    const float4 y = *reinterpret_cast<const float4 *>(
        y_rows + (size_t)slot_pos[(size_t)t * k + j] * H + n);
    acc[0] = fma(wj, (double)y.x, acc[0]);
    acc[1] = fma(wj, (double)y.y, acc[1]);
    acc[2] = fma(wj, (double)y.z, acc[2]);
    acc[3] = fma(wj, (double)y.w, acc[3]);
  }
  if (dir) {
    const double a = alpha;
    const float4 d = *reinterpret_cast<const float4 *>(dir + n);
    acc[0] = fma(a, (double)d.x, acc[0]);
    acc[1] = fma(a, (double)d.y, acc[1]);
    acc[2] = fma(a, (double)d.z, acc[2]);
    acc[3] = fma(a, (double)d.w, acc[3]);
  }
  const float4 r = make_float4((float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]);
  *reinterpret_cast<float4 *>(out + (size_t)t * H + n) = r;
  if (out_bf16) {
    uint2 b;
    b.x = f32_to_bf16_bits(r.x) | (f32_to_bf16_bits(r.y) << 16);
    b.y = f32_to_bf16_bits(r.z) | (f32_to_bf16_bits(r.w) << 16);
    *reinterpret_cast<uint2 *>(out_bf16 + (size_t)t * H + n) = b;
  }
}

hipError_t launch_combine(int T, int H, int k, const float *y_rows, const int32_t *slot_pos,
                          const float *w, const float *shared_y, const float *steer_dir,
                          float steer_alpha, float *out, uint16_t *out_bf16, hipStream_t s) {
  dim3 grid((H / 4 + 255) / 256, T);
  return launch(k_combine, dim3(grid), dim3(256), s, T, H, k, y_rows, slot_pos, w, shared_y,
                steer_dir, steer_alpha, out, out_bf16);
}

// ---------------------------------------------------------------------------
// moe_dequantize: the same decoders as the FFN kernels, one weight per thread
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_dequant(WView w, int e, int64_t w0, int64_t count,
                                                  float *__restrict__ out) {
  const size_t dbytes = expert_data_bytes(w.fmt, w.N, w.K);
  const size_t sbytes = expert_scale_bytes(w.fmt, w.N, w.K);
  const uint8_t *data = w.data + (size_t)e * dbytes;
  const uint8_t *scales = w.scales ? w.scales + (size_t)e * sbytes : nullptr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256) {
    const int64_t f = w0 + i;
    float v;
    switch (w.fmt) {
      case MOE_FMT_BF16:
        v = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(data)[f]);
        break;
      case MOE_FMT_Q2K:
        v = q2k_weight(data + (f / 256) * kQ2KBytes, (int)(f % 256));
        break;
      case MOE_FMT_VQ2: {
        const uint32_t code = data[f / 4];
        const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(scales)[f / 256]);
        v = vq2_weight(code, (int)(f % 4), d, w.codebook);
        break;
      }
      default: {  // MXFP4
        v = mxfp4_weight(data[f / 2], (int)(f & 1), scales[f / 32]);
        break;
      }
    }
    out[i] = v;
  }
}

hipError_t launch_dequant(const WView &w, int expert, int64_t w0, int64_t count, float *out,
                          hipStream_t s) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch(k_dequant, dim3((unsigned)blocks), dim3(256), s, w, expert, w0, count, out);
}

}  // namespace moe
