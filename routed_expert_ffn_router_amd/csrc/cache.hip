// cache.hip -- a residency cache of routed experts in HBM, filled from pinned
// host memory, for one-token decode.
//
// The pages run models larger than memory by streaming the routed experts
// from SSD while generating, since generation reads only the few experts a
// token picks while prefill amortises them over the chunk (hysenlabs.com ds4
// page, "SSD streaming"; baiwuji.top ds4 article, "Core features" item 2).
// Here the slower tier is pinned host memory and the fast tier a pool of C
// expert slots in HBM; everything is decided on the device, between the
// router (p1) and the routed gate/up (p2), with no host round trip:
//   plan (one wave): select the k experts from the router logits (the same
//     selection as p2's), look each up in the expert -> slot table; a miss
//     takes the least recently used slot that no chosen expert holds (ties:
//     the lowest slot); record hits, misses and the copies to make;
//   fill: copy each missed expert's bytes of gate, up and down (data and
//     scale planes) from host memory into its slot, 16-byte loads spread
//     over many workgroups so that the host link streams;
// then p2 and p3 read the slot pool at the planned slots.
//
// State (int32, caller's device memory, moe_cache_state_ints(E, C)):
//   [0] clock (steps so far)  [1] copies planned this step
//   [2] hits so far           [3] misses so far
//   [4, 4+E) slot of expert e or -1;  then owner[C] (expert in slot or -1),
//   stamp[C] (clock of last use), fill_e[16], fill_s[16], slot_idx[16].
#include "select.h"

namespace moe {

constexpr int kCacheHdr = 4;
constexpr int kCacheMaxC = 1024;
constexpr int kFillThreads = 256;

struct CacheLayout {
  int E, C;
  __host__ __device__ int slot_of() const { return kCacheHdr; }
  __host__ __device__ int owner() const { return kCacheHdr + E; }
  __host__ __device__ int stamp() const { return kCacheHdr + E + C; }
  __host__ __device__ int fill_e() const { return kCacheHdr + E + 2 * C; }
  __host__ __device__ int fill_s() const { return fill_e() + 16; }
  __host__ __device__ int slot_idx() const { return fill_s() + 16; }
  __host__ __device__ int total() const { return slot_idx() + 16; }
};

size_t cache_state_ints(int E, int C) { return (size_t)CacheLayout{E, C}.total(); }
int cache_slot_idx_offset(int E, int C) { return CacheLayout{E, C}.slot_idx(); }

__global__ __launch_bounds__(256) void k_cache_reset(int E, int C, int32_t *__restrict__ st) {
  const CacheLayout L{E, C};
  for (int i = blockIdx.x * 256 + threadIdx.x; i < L.total(); i += gridDim.x * 256) {
    int v = 0;
    if (i >= L.slot_of() && i < L.stamp()) v = -1;  // slot_of and owner empty
    st[i] = v;
  }
}

// one wave: selection, lookups, LRU victims (in LDS), table updates
__global__ __launch_bounds__(64) void k_cache_plan(int mode, int E, int C, int k,
                                                    const float *__restrict__ logits,
                                                    const int64_t *__restrict__ tid,
                                                    int32_t *__restrict__ st,
                                                    int32_t *__restrict__ topk_idx,
                                                    float *__restrict__ topk_w) {
  __shared__ int s_owner[kCacheMaxC];
  __shared__ int s_stamp[kCacheMaxC];
  const CacheLayout L{E, C};
  const int lane = threadIdx.x;
  for (int c = lane; c < C; c += 64) {
    s_owner[c] = st[L.owner() + c];
    s_stamp[c] = st[L.stamp() + c];
  }
  int e;
  float w;
  select_wave(mode, E, k, logits, tid ? tid[0] : 0, &e, &w);
  if (lane < k) {
    topk_idx[lane] = e;
    topk_w[lane] = w;
  }
  const int clock = st[0] + 1;
  int s = -1;
  if (lane < k) s = st[L.slot_of() + min(max(e, 0), E - 1)];
  __syncthreads();
  if (lane < k && s >= 0) s_stamp[s] = clock;  // hits: used now, never a victim this step
  __syncthreads();
  int nfill = 0, nhit = 0;
  for (int j = 0; j < k; j++) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    const int sj = __builtin_amdgcn_readlane(s, j);
    if (sj >= 0) {
      if (lane == 0) st[L.slot_idx() + j] = sj;
      nhit++;
      continue;
    }
    // the least recently used slot (lowest index on ties)
    uint64_t best = ~0ull;
    for (int c = lane; c < C; c += 64) {
      const uint64_t key = ((uint64_t)(uint32_t)s_stamp[c] << 32) | (uint32_t)c;
      best = key < best ? key : best;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t other = __shfl_xor(best, o, 64);
      best = other < best ? other : best;
    }
    const int v = (int)(uint32_t)best;
    if (lane == 0) {
      const int old = s_owner[v];
      if (old >= 0) st[L.slot_of() + old] = -1;
      st[L.slot_of() + ej] = v;
      s_owner[v] = ej;
      s_stamp[v] = clock;
      st[L.fill_e() + nfill] = ej;
      st[L.fill_s() + nfill] = v;
      st[L.slot_idx() + j] = v;
    }
    nfill++;
    __syncthreads();
  }
  for (int c = lane; c < C; c += 64) {
    st[L.owner() + c] = s_owner[c];
    st[L.stamp() + c] = s_stamp[c];
  }
  if (lane == 0) {
    st[0] = clock;
    st[1] = nfill;
    st[2] += nhit;
    st[3] += nfill;
  }
}

// the byte planes of one expert: src = host base + e * per, dst = slot base + s * per
struct FillPlanes {
  int n;
  const uint8_t *src[6];
  uint8_t *dst[6];
  uint32_t per16[6];  // 16-byte units per expert of each plane
};

// blockIdx.y: planned copy j (exits past the step's count); blockIdx.x: a
// 1/gridDim.x share of the expert's 16-byte units of every plane
__global__ __launch_bounds__(kFillThreads) void k_cache_fill(int E, int C, const int32_t *__restrict__ st,
                                                             FillPlanes fp) {
  const CacheLayout L{E, C};
  const int j = blockIdx.y;
  if (j >= st[1]) return;
  const int e = st[L.fill_e() + j], s = st[L.fill_s() + j];
  for (int p = 0; p < fp.n; p++) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(fp.src[p]) + (size_t)e * fp.per16[p];
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(fp.dst[p]) + (size_t)s * fp.per16[p];
    const uint32_t n = fp.per16[p];
    const uint32_t step = gridDim.x * kFillThreads;
    uint32_t i = blockIdx.x * kFillThreads + threadIdx.x;
    // four 16-byte loads in flight per thread over the host link
    for (; i + 3 * step < n; i += 4 * step) {
      const u32x4_t a = src[i], b = src[i + step], c = src[i + 2 * step], d = src[i + 3 * step];
      dst[i] = a, dst[i + step] = b, dst[i + 2 * step] = c, dst[i + 3 * step] = d;
    }
    for (; i < n; i += step) dst[i] = src[i];
  }
}

hipError_t launch_cache_reset(int E, int C, int32_t *state, hipStream_t s) {
  const int n = CacheLayout{E, C}.total();
  return launch(k_cache_reset, dim3((n + 255) / 256), dim3(256), s, E, C, state);
}

hipError_t launch_cache_step(const CacheStep &c, hipStream_t s, void (*mark)(void *, const char *),
                             void *mark_ctx) {
  if (mark) mark(mark_ctx, "cache_plan");
  hipError_t err = launch(k_cache_plan, dim3(1), dim3(64), s, c.mode, c.E, c.C, c.k, c.logits,
                          c.tid, c.state, c.topk_idx, c.topk_w);
  if (err != hipSuccess) return err;
  FillPlanes fp{};
  fp.n = c.n_planes;
  uint32_t most = 0;
  for (int p = 0; p < c.n_planes; p++) {
    fp.src[p] = c.src[p];
    fp.dst[p] = c.dst[p];
    fp.per16[p] = (uint32_t)(c.per_bytes[p] / 16);
    most = fp.per16[p] > most ? fp.per16[p] : most;
  }
  // enough workgroups per copy that k copies keep every CU loading
  const uint32_t bx = (most + kFillThreads * 4 - 1) / (kFillThreads * 4);
  if (mark) mark(mark_ctx, "cache_fill");
  return launch(k_cache_fill, dim3(bx < 256 ? bx : 256, c.k), dim3(kFillThreads), s, c.E, c.C,
                (const int32_t *)c.state, fp);
}

}  // namespace moe
