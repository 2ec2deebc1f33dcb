// decode.hip -- one token through the whole MoE layer in three launches.
//
// Batch-1 decode streams ~109 MB of weights for ~0.5 GFLOP, so it is bound by
// HBM bandwidth and by the fixed cost of each kernel boundary.  The layer's
// dependency chain (router -> selection -> routed gate/up -> routed down) is
// cut into three launches, and the shared expert -- independent of routing
// (the pages keep it at full precision and add it to the routed sum:
// dibi8.com ds4 guide "Key innovations" item 1) -- fills the same launches:
//   p1: shared gate/up + SwiGLU (8 waves per block, a row pair each) and the
//       router logits (a ninth wave per block, one expert row, fp64)
//   p2: top-k selection, recomputed by every block from the logits (no
//       separate launch), then routed gate/up + SwiGLU for its tile; every
//       wave first requests one row of the shared down, which streams while
//       the selection leaves the routed weights waiting
//   p3: routed down of the k experts (one expert per wave) + weighted sum
//       with the shared down, reduced in a fixed order (deterministic, no
//       atomics)
#include "select.h"

namespace moe {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kP1Threads = kDecThreads + 64;  // + the router wave
// output rows per p3 block: 8 (two blocks per CU: four waves per SIMD keep
// the VALU busy while rows arrive; with 16 rows and one block p3 took
// 0.45 us longer), 16 for VQ2, whose blocks each fill the codebook
template <int DFMT>
constexpr int p3_rows() { return DFMT == MOE_FMT_VQ2 ? 16 : 8; }
constexpr int kP3Threads = kDecThreads;
constexpr int kRouterChunks = 8;              // H <= 64 lanes x 8 bf16 x 8

// ---------------------------------------------------------------------------
// p1: block b, waves 0..7: shared gate/up row pairs i = b*8 + wave (+ nb*8 ...);
// wave 8: router rows e = b (+ nb ...), a whole row per wave, each lane
// summing its eight-element chunks in fp64 (every product of two bf16 is exact
// in fp64 and, for values of ordinary range, so is the sum: the result does
// not depend on the order), then one rounding to fp32.
// ---------------------------------------------------------------------------
template <int SSPL>
__global__ __launch_bounds__(kP1Threads) void k_dec_p1(DecodeArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = gridDim.x;
  const int nc = p.H / 512;  // router chunks of 8 per lane
  uint4 wv[kRouterChunks], xv[kRouterChunks];
  auto router_loads = [&](int e) {
    const uint16_t *wrow = p.w_router + (size_t)e * p.H;
#pragma unroll
    for (int c = 0; c < kRouterChunks; c++)
      if (c < nc) {
        wv[c] = *reinterpret_cast<const uint4 *>(wrow + lane * 8 + 512 * c);
        xv[c] = *reinterpret_cast<const uint4 *>(p.x + lane * 8 + 512 * c);
      }
  };
  const bool router = wave == kDecWaves && !p.logits_in && (int)blockIdx.x < p.E;
  if (router) router_loads(blockIdx.x);
  // the router row's loads go out before the shared weight stream, which they
  // would otherwise queue behind
  __syncthreads();
  if (wave == kDecWaves) {
    if (!router) return;
    for (int e = blockIdx.x; e < p.E; e += nb) {
      if (e != (int)blockIdx.x) router_loads(e);
      double acc = 0.0;
#pragma unroll
      for (int c = 0; c < kRouterChunks; c++)
        if (c < nc) {
          const uint32_t xa[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
          const uint32_t wa[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
          for (int q = 0; q < 4; q++) {
            acc = fma((double)bf16_lo(xa[q]), (double)bf16_lo(wa[q]), acc);
            acc = fma((double)bf16_hi(xa[q]), (double)bf16_hi(wa[q]), acc);
          }
        }
      acc = group_sum_f64<64>(acc);
      if (lane == 0) p.logits[e] = (float)acc;
    }
    return;
  }
  if (p.Is) {
    for (int i0 = blockIdx.x * kDecWaves; i0 < p.Is; i0 += nb * kDecWaves)
      gateup_rows<MOE_FMT_BF16, SSPL, 64, 1, 1>(p.sg, p.su, p.H, p.Is, p.x, 0, 0, 1, nullptr, 0,
                                                 nullptr, i0 + wave, nullptr, kASplit, p.a_sh_hi,
                                                 p.a_sh_lo);
  }
}

// ---------------------------------------------------------------------------
// p2: block b: routed gate/up tile b (expert slot b / tiles, 8 waves x ST
// rows).  The selection's inputs are fetched first, then each wave's shared
// down row; wave 0 selects while the others fill the codebook, and after the
// block barrier each wave finishes its shared row before its routed rows.
// ---------------------------------------------------------------------------
template <int RFMT, int RSPL, int SSPL>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_p2(DecodeArgs p) {
  // the VQ2 codebook in 32 copies (64 KB; two blocks still fit a CU): each
  // lane of a half-wave reads its own copy (with 16, lanes l and l + 16 share
  // one and the lookups took bank conflicts)
  constexpr int kCopies = 32;
  __shared__ uint2 s_cb[RFMT == MOE_FMT_VQ2 ? 256 * kCopies : 1];
  __shared__ int s_e[16];
  __shared__ int s_ready;  // waves whose LDS outputs (selection, codebook) are written
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x == 0) s_ready = 0;
  __syncthreads();  // (nothing is in flight yet)
  const float *lsrc = p.logits_in ? p.logits_in : p.logits;
  const bool small_e = p.E <= 256;
  // unconditional loads (a branch around them would make the compiler wait
  // for every later load before their first use): the first 256 logits, the
  // token id (any 8 bytes in softmax mode) and this thread's codebook entry
  Logits<4> lg;
  lg.load(p.E, lsrc);
  const int64_t tid0 = *(p.tid ? p.tid : reinterpret_cast<const int64_t *>(p.x));
  uint32_t cbw = 0;
  if constexpr (RFMT == MOE_FMT_VQ2) cbw = codebook_entry_load(p.gate.codebook);
  // then the shared down rows of waves 1..7 and p1's SwiGLU output: the
  // block's rows 8 b + w (+ 8 nb ...) go to wave w, row 8 b + 0 to wave 1
  // too, so that wave 0 only selects; they stream and are reduced while the
  // selection runs
  const int rb0 = blockIdx.x * kDecWaves;
  Chunk<MOE_FMT_BF16, SSPL, 64> csh[2];
  ADown<MOE_FMT_BF16, SSPL, 64> ash[1];
  if (p.Is && wave > 0) {
    csh[0].load(p.sd, 0, min(rb0 + wave, p.H - 1), lane);
    if (wave == 1) csh[1].load(p.sd, 0, min(rb0, p.H - 1), lane);
    ash[0].load_split(p.a_sh_hi, p.a_sh_lo, lane);
  }
  asm volatile("" ::"v"(cbw), "v"(lg.v[0]), "v"(lg.v[1]), "v"(lg.v[2]), "v"(lg.v[3]),
               "v"((uint32_t)tid0), "v"((uint32_t)(tid0 >> 32)));
  // the codebook copies are written by waves 4-7 alone, so that wave 0
  // goes straight to the selection
  if constexpr (RFMT == MOE_FMT_VQ2)
    if (wave >= 4) {
      codebook_entry_store_all<kCopies>(cbw, s_cb);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) atomicAdd(&s_ready, 1);
    }
  if (wave == 0 && p.slot_idx) {
    // the expert cache planned the choices and their slots
    if (lane < p.k) s_e[lane] = p.slot_idx[lane];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) atomicAdd(&s_ready, 1);
  } else if (wave == 0) {
    // the selection is the block's critical path: its wave issues first
    __builtin_amdgcn_s_setprio(3);
    int e;
    float w;
    if (small_e || p.mode == MOE_ROUTE_HASH)
      select_wave<4>(p.mode, p.E, p.k, lg, lsrc, tid0, &e, &w);
    else
      select_wave(p.mode, p.E, p.k, lsrc, 0, &e, &w);
    __builtin_amdgcn_s_setprio(0);
    if (lane < p.k) {
      s_e[lane] = e;
      if (blockIdx.x == 0) {
        p.topk_idx[lane] = e;
        p.topk_w[lane] = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) atomicAdd(&s_ready, 1);
  } else if (p.Is) {
    const int step = gridDim.x * kDecWaves;
    for (int base = rb0; base < p.H; base += step) {
      if (base != rb0) {
        csh[0].load(p.sd, 0, min(base + wave, p.H - 1), lane);
        if (wave == 1) csh[1].load(p.sd, 0, base, lane);
      }
      float y[1];
      if (base + wave < p.H) {
        csh[0].template dot_a<1>(ash, nullptr, y);
        y[0] = wave_sum_f(y[0]);
        if (lane == 0) p.shared_y[base + wave] = y[0];
      }
      if (wave == 1) {
        csh[1].template dot_a<1>(ash, nullptr, y);
        y[0] = wave_sum_f(y[0]);
        if (lane == 0) p.shared_y[base] = y[0];
      }
    }
  }
  // each wave goes on as soon as the selection and the codebook are written,
  // without waiting for the other waves' shared rows (a bounded wait on an
  // LDS counter that waves of this block always complete; were the bound
  // ever reached, the expert index is still clamped into [0, E), so every
  // load stays inside the weights)
  {
    const int need = RFMT == MOE_FMT_VQ2 ? 5 : 1;
    for (int it = 0; it < (1 << 22); it++) {
      if (__hip_atomic_load(&s_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= need) break;
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
  constexpr int ST = steps_for<RFMT, RSPL>();
  const int j = blockIdx.x / p.tiles_per_expert, tile = blockIdx.x % p.tiles_per_expert;
  const int row_base = (tile * kDecWaves + wave) * ST;
  const int e_sel = min(max(__builtin_amdgcn_readfirstlane(s_e[j]), 0), p.gate.E - 1);
  // every routed row pair's loads go out at once (MXFP4's larger chunks: two)
  constexpr int kRPF = RFMT == MOE_FMT_MXFP4 ? 2 : ST;
  gateup_rows<RFMT, RSPL, 64, ST, 1, kRPF, kCopies>(p.gate, p.up, p.H, p.I, p.x, e_sel, j, j + 1,
                                                    nullptr, 0, p.a, row_base, s_cb, p.a_mode,
                                                    p.a_hi, p.a_lo);
}

// ---------------------------------------------------------------------------
// p3: block b owns output rows [R b, R b + R), R = p3_rows.  Wave w: routed
// down of expert j = w (+ 8 ...) over those rows, weighted by w_j.  Thread
// r < R
// then adds the eight routed partial sums in wave order and p2's shared down.
// ---------------------------------------------------------------------------
template <int DFMT, int DSPL>
__global__ __launch_bounds__(kP3Threads) void k_dec_p3(DecodeArgs p) {
  constexpr int kP3Rows = p3_rows<DFMT>();
  __shared__ uint2 s_cb[DFMT == MOE_FMT_VQ2 ? 256 * kNCopy : 1];
  __shared__ float s_part[kDecWaves][kP3Rows];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = blockIdx.x * kP3Rows;
  if constexpr (DFMT == MOE_FMT_VQ2) {
    fill_codebook(p.down.codebook, s_cb);
    __syncthreads();
  }
  {
    // rows whose loads are in flight per wave: all of the block's rows when
    // their raw bits fit in about 96 registers (the 2-bit formats), else four
    constexpr int kDw = DFMT == MOE_FMT_BF16 ? 8 * DSPL : DFMT == MOE_FMT_VQ2 ? 2 * DSPL : 3 * DSPL;
    constexpr int PF = DFMT != MOE_FMT_MXFP4 && 96 / kDw >= kP3Rows ? kP3Rows : 4;
    const uint2 *cb = s_cb + (lane % kNCopy);
    float acc[kP3Rows];
#pragma unroll
    for (int r = 0; r < kP3Rows; r++) acc[r] = 0.0f;
    // the slot's activations do not depend on the choice: with the 2-bit
    // formats they are requested first and travel alongside the expert index;
    // MXFP4's wider rows go first instead
    constexpr bool kAFirst = DFMT != MOE_FMT_MXFP4;
    // Q2K and MXFP4: p2 leaves a as fp16 (kAF16Q2K, kAF16)
    using AV = std::conditional_t<
        DFMT == MOE_FMT_Q2K, ADownQ2K16<DSPL, 64>,
        std::conditional_t<DFMT == MOE_FMT_MXFP4, ADownF16<DSPL, 64>, ADown<DFMT, DSPL, 64>>>;
    for (int j = wave; j < p.k; j += kDecWaves) {
      AV av[1];
      auto load_a = [&]() {
        if constexpr (DFMT == MOE_FMT_Q2K || DFMT == MOE_FMT_MXFP4)
          av[0].load(p.a_hi + (size_t)j * p.I, lane);
        else if constexpr (DFMT == MOE_FMT_BF16)
          av[0].load_split(p.a_hi + (size_t)j * p.I, p.a_lo + (size_t)j * p.I, lane);
        else
          av[0].load(p.a + (size_t)j * p.I, lane);
      };
      if constexpr (kAFirst) load_a();
      const int32_t *eidx = p.slot_idx ? p.slot_idx : p.topk_idx;  // expert, or its cache slot
      const int e = __builtin_amdgcn_readfirstlane(eidx[j]);
      const float wj = __builtin_bit_cast(
          float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p.topk_w[j])));
      Chunk<DFMT, DSPL, 64> c[PF];
#pragma unroll
      for (int r = 0; r < PF; r++) c[r].load(p.down, e, min(row0 + r, p.H - 1), lane);
      if constexpr (!kAFirst) load_a();
      if constexpr (DFMT == MOE_FMT_Q2K) av[0].sums();  // while the weights are in flight
#pragma unroll
      for (int r = 0; r < kP3Rows; r++) {
        float y[1];
        if constexpr (DFMT == MOE_FMT_Q2K || DFMT == MOE_FMT_MXFP4)
          y[0] = c[r % PF].dot_a16(av[0]);
        else
          c[r % PF].template dot_a<1>(av, cb, y);
        if (r + PF < kP3Rows) c[r % PF].load(p.down, e, min(row0 + r + PF, p.H - 1), lane);
        __builtin_amdgcn_sched_barrier(0);
        acc[r] = fmaf(wj, y[0], acc[r]);
      }
    }
    const float v = rows_reduce<kP3Rows>(acc);
    if ((lane & (64 / kP3Rows - 1)) == 0) s_part[wave][lane / (64 / kP3Rows)] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < kP3Rows) {
    const int r = threadIdx.x, row = row0 + r;
    if (row < p.H) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; w++) v += s_part[w][r];
      if (p.Is) v += p.shared_y[row];
      if (p.steer_dir) v = fmaf(p.steer_alpha, p.steer_dir[row], v);
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

template <int RFMT, int RSPL>
hipError_t p2_shared(const DecodeArgs &a, int sspl, hipStream_t s) {
  if (sspl == 4) return launch(k_dec_p2<RFMT, RSPL, 4>, dim3(a.nb_routed), dim3(kDecThreads), s, a);
  if (sspl == 2) return launch(k_dec_p2<RFMT, RSPL, 2>, dim3(a.nb_routed), dim3(kDecThreads), s, a);
  return hipErrorInvalidValue;
}

template <int RFMT>
hipError_t p2_fmt(const DecodeArgs &a, int rspl, int sspl, hipStream_t s) {
  if (rspl == 4) return p2_shared<RFMT, 4>(a, sspl, s);
  if (rspl == 2) return p2_shared<RFMT, 2>(a, sspl, s);
  return hipErrorInvalidValue;
}

template <int DFMT>
hipError_t p3_fmt(const DecodeArgs &a, int dspl, hipStream_t s) {
  const dim3 grid((a.H + p3_rows<DFMT>() - 1) / p3_rows<DFMT>());
  if (dspl == 2) return launch(k_dec_p3<DFMT, 2>, grid, dim3(kP3Threads), s, a);
  if (dspl == 4) return launch(k_dec_p3<DFMT, 4>, grid, dim3(kP3Threads), s, a);
  return hipErrorInvalidValue;
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

// H in {2048, 4096} (router chunks, lane geometry), I and Is in {2048, 4096}
bool decode1_supported(int H, int I, int Is, int k) {
  const int sh = spl_of(H), si = spl_of(I);
  const bool shared_ok = Is == 0 || spl_of(Is) == 2 || spl_of(Is) == 4;
  return (sh == 2 || sh == 4) && (si == 2 || si == 4) && shared_ok && k <= 16 &&
         H % 512 == 0 && H <= 512 * kRouterChunks;
}

hipError_t launch_decode1(DecodeArgs a, hipStream_t s, void (*mark)(void *, const char *),
                          void *mark_ctx, const CacheStep *cache) {
  const int hs = spl_of(a.H), is = spl_of(a.I), ss = a.Is ? spl_of(a.Is) : 2;
  // p1: one router row per block and one shared gate/up row pair per wave
  a.nb_router = a.logits_in ? 0 : a.E;
  a.nb_shared_gu = a.Is ? (a.Is + kDecWaves - 1) / kDecWaves : 0;
  const int rpb = rows_per_block(a.gate.fmt, hs);
  a.tiles_per_expert = (a.I + rpb - 1) / rpb;
  a.nb_routed = a.k * a.tiles_per_expert;
  a.a_mode = a.down.fmt == MOE_FMT_Q2K     ? kAF16Q2K
             : a.down.fmt == MOE_FMT_MXFP4 ? kAF16
             : a.down.fmt == MOE_FMT_BF16  ? kASplit
                                           : kAF32;
  hipError_t e;
  if (a.nb_router + a.nb_shared_gu > 0) {
    mark(mark_ctx, "decode_p1");
    const int g1 = max(a.nb_router, a.nb_shared_gu);
    e = hs == 4 ? launch(k_dec_p1<4>, dim3(g1), dim3(kP1Threads), s, a)
                : launch(k_dec_p1<2>, dim3(g1), dim3(kP1Threads), s, a);
    if (e != hipSuccess) return e;
  }
  if (cache) {
    e = launch_cache_step(*cache, s, mark, mark_ctx);
    if (e != hipSuccess) return e;
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
