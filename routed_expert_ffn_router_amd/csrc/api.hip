// api.hip -- the C ABI of libmoe (include/moe.h): argument validation,
// workspace carving and kernel sequencing.  Host code only.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"

namespace moe {
bool gemv_supported_k(int K);
}

using namespace moe;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

}  // namespace

// the thread's error text, for the other translation units (probe.hip)
int moe::set_error(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

namespace {

int hip_check(hipError_t e, const char *where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

#define MOE_TRY(expr)             \
  do {                            \
    int rc_ = (expr);             \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sequential carving of the caller's workspace (base == nullptr: sizing only).
struct Carver {
  uint8_t *base;
  size_t off = 0, last = 0;  // last: offset of the latest piece
  explicit Carver(void *b) : base(static_cast<uint8_t *>(b)) {}
  template <class T>
  T *take(size_t n) {
    off = (off + 255) & ~size_t(255);
    last = off;
    T *r = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += n * sizeof(T);
    return r;
  }
  size_t size() const { return (off + 255) & ~size_t(255); }
};

int check_weights(const moe_weights *w, const char *name, int E, int N, int K) {
  if (!w) return fail(MOE_EINVAL, "%s: null weights", name);
  if (w->fmt < MOE_FMT_BF16 || w->fmt > MOE_FMT_MXFP4)
    return fail(MOE_EUNSUPPORTED, "%s: unknown format %d", name, w->fmt);
  if (w->n_experts != E || w->rows != N || w->cols != K)
    return fail(MOE_EINVAL, "%s: shape [%d][%d][%d], expected [%d][%d][%d]", name, w->n_experts,
                w->rows, w->cols, E, N, K);
  if (!w->data) return fail(MOE_EINVAL, "%s: null data", name);
  if (!aligned(w->data, 16)) return fail(MOE_EINVAL, "%s: data not 16-byte aligned", name);
  const long long n = (long long)N * K;
  switch (w->fmt) {
    case MOE_FMT_BF16:
      if (K % 8) return fail(MOE_EINVAL, "%s: bf16 needs cols %% 8 == 0", name);
      break;
    case MOE_FMT_Q2K:
      if (n % 256) return fail(MOE_EINVAL, "%s: q2k needs rows*cols %% 256 == 0", name);
      break;
    case MOE_FMT_VQ2:
      if (K % 256) return fail(MOE_EINVAL, "%s: vq2 needs cols %% 256 == 0", name);
      if (!w->scales || !w->codebook)
        return fail(MOE_EINVAL, "%s: vq2 needs scales and codebook", name);
      if (!aligned(w->scales, 2) || !aligned(w->codebook, 4))
        return fail(MOE_EINVAL, "%s: vq2 scales/codebook misaligned", name);
      break;
    case MOE_FMT_MXFP4:
      if (K % 32) return fail(MOE_EINVAL, "%s: mxfp4 needs cols %% 32 == 0", name);
      if (!w->scales) return fail(MOE_EINVAL, "%s: mxfp4 needs scales", name);
      break;
  }
  return MOE_OK;
}

int check_route_args(int mode, int T, int E, int k) {
  if (mode != MOE_ROUTE_SOFTMAX_TOPK && mode != MOE_ROUTE_HASH)
    return fail(MOE_EINVAL, "unknown routing mode %d", mode);
  if (T < 0) return fail(MOE_EINVAL, "T = %d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_EINVAL, "E = %d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 16) return fail(MOE_EINVAL, "k = %d outside [1, min(E, 16)]", k);
  return MOE_OK;
}

int check_ffn_weights(int E, int H, int I, const moe_weights *gate, const moe_weights *up,
                      const moe_weights *down) {
  MOE_TRY(check_weights(gate, "gate", E, I, H));
  MOE_TRY(check_weights(up, "up", E, I, H));
  MOE_TRY(check_weights(down, "down", E, H, I));
  if (gate->fmt != up->fmt) return fail(MOE_EUNSUPPORTED, "gate and up formats differ");
  if (gate->fmt == MOE_FMT_VQ2 && gate->codebook != up->codebook)
    return fail(MOE_EUNSUPPORTED, "vq2 gate and up must share one codebook");
  if (!gemv_supported_k(H) || !gemv_supported_k(I))
    return fail(MOE_EUNSUPPORTED, "H = %d / I = %d: supported sizes are 128, 256, 512 and "
                "multiples 1, 2, 4, 8 of 1024", H, I);
  return MOE_OK;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

thread_local hipEvent_t t_start = nullptr, t_stop = nullptr;

// Optional per-kernel timing (moe_forward_marked): each mark arms the next
// launch to record marks[n].start / marks[n].stop at its own start and end.
struct Marker {
  moe_mark *m = nullptr;
  int max = 0, n = 0;
  void operator()(const char *name) {
    if (m && n < max) {
      timer_arm(static_cast<hipEvent_t>(m[n].start), static_cast<hipEvent_t>(m[n].stop));
      m[n].name = name;
      n++;
    }
  }
  ~Marker() { timer_arm(nullptr, nullptr); }  // nothing stays armed past the call
};

void mark_cb(void *ctx, const char *name) { (*static_cast<Marker *>(ctx))(name); }

// The caller's second stream for the shared expert (moe_side_stream): it
// does not depend on the routing, so moe_forward runs it there, beside the
// router, the selection, the dispatch and the routed FFN, and joins before
// the combine.
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join;
};

WView bf16_view(const uint16_t *p, int N, int K) {
  return WView{MOE_FMT_BF16, 1, N, K, reinterpret_cast<const uint8_t *>(p), nullptr, nullptr};
}

// ---------------------------------------------------------------------------
// expert FFN workspace and sequence (shared by moe_expert_ffn and moe_forward)
// ---------------------------------------------------------------------------

const char *const kRoutedGemmNames[4] = {"tile_list", "gemm_gateup", "gemm_down",
                                         "tokens_f16"};
const char *const kSharedGemmNames[4] = {"shared_tile_list", "shared_gemm_gateup",
                                         "shared_gemm_down", "shared_tokens_f16"};
const char *const kA8Names[4] = {"tile_list", "a8_gemm_gateup", "a8_gemm_down", "act_quant"};

struct FfnBufs {
  int32_t *plan;
  float *a;        // fp32 SwiGLU output of the GEMV path; fp16 on the GEMM path
  int32_t *tiles;  // GEMM tile list
  uint16_t *x16;   // GEMM path: the tokens as fp16 operands
  void *a8;        // MX-FP8 tokens and SwiGLU output (MOE_ACT_MXFP8)
};

FfnBufs carve_ffn(Carver &c, int T, int n_rows, int E, int H, int I, bool dense, int act) {
  FfnBufs b{};
  b.plan = dense ? nullptr : c.take<int32_t>(plan_ints(std::min(E, std::max(n_rows, 1))));
  b.a = c.take<float>((size_t)std::max(n_rows, 1) * I);
  b.tiles = c.take<int32_t>(gemm_tile_ints(std::max(n_rows, 1), dense ? 0 : E));
  b.x16 = c.take<uint16_t>((size_t)std::max(T, 1) * H);
  if ((act & ~MOE_ACT_TRACE) == MOE_ACT_MXFP8)
    b.a8 = c.take<uint8_t>(a8_ws_bytes(T, H, I, std::max(n_rows, 1)));
  return b;
}

// 32-bit buffer offsets of the GEMM kernels: every operand below 2 GiB
bool gemm_fits(int T, int H, int I, int n_rows) {
  const size_t lim = (size_t)1 << 31;
  return (size_t)T * H * 2 < lim && (size_t)n_rows * I * 2 < lim;
}

// The matrix-core path streams each expert's weights once for all its rows;
// from a handful of tokens on it beats the per-token GEMV (one choice for
// moe_expert_ffn and moe_forward alike, so the two compose exactly)
bool use_gemm(int T, int H, int I, int E, int n_rows, bool dense, int fmt_gate, int fmt_down) {
  (void)E;
  if (!gemm_supported(H, I, fmt_gate, fmt_down) || !gemm_fits(T, H, I, n_rows)) return false;
  return dense ? n_rows >= 32 : T >= 4;
}

int run_ffn(int T, int H, int I, const uint16_t *x, const WView &g, const WView &u,
            const WView &d, int act, const int32_t *offsets, const int32_t *sorted_token,
            int n_rows, float *y, const FfnBufs &b, hipStream_t s, Marker *mk = nullptr) {
  Marker none;
  Marker &m = mk ? *mk : none;
  if ((act & ~MOE_ACT_TRACE) == MOE_ACT_MXFP8)
    return hip_check(launch_a8_ffn(g, u, d, H, I, T, x, offsets, sorted_token, n_rows, b.tiles,
                                   b.a8, (act & MOE_ACT_TRACE) ? b.a : nullptr, y, s, mark_cb,
                                   &m, kA8Names),
                     "a8 ffn");
  if (!offsets && skinny_supported(H, I, T, g, d))
    return hip_check(launch_skinny_ffn(g, u, d, H, I, T, x, reinterpret_cast<uint16_t *>(b.a), y,
                                       s, mark_cb, &m, kRoutedGemmNames),
                     "skinny ffn");
  if (use_gemm(T, H, I, g.E, n_rows, !offsets, g.fmt, d.fmt))
    return hip_check(launch_gemm_ffn(g, u, d, H, I, T, x, offsets, sorted_token, n_rows, b.tiles,
                                     reinterpret_cast<uint16_t *>(b.a), b.x16, y, s, mark_cb, &m,
                                     kRoutedGemmNames),
                     "gemm ffn");
  if (!offsets) {
    m("gateup_gemv");
    MOE_TRY(hip_check(launch_gateup_gemv(g, u, H, I, x, nullptr, T, nullptr, b.a, s), "gate/up"));
    m("down_gemv");
    return hip_check(launch_down_gemv(d, H, I, b.a, nullptr, T, y, s), "down");
  }
  const int E = g.E;
  const int max_active = std::min(E, n_rows);
  m("plan");
  MOE_TRY(hip_check(launch_plan_from_offsets(E, offsets, b.plan, s), "plan"));
  m("gateup_gemv");
  MOE_TRY(hip_check(launch_gateup_gemv(g, u, H, I, x, b.plan, max_active, sorted_token, b.a, s),
                    "gate/up"));
  m("down_gemv");
  return hip_check(launch_down_gemv(d, H, I, b.a, b.plan, max_active, y, s), "down");
}

// ---------------------------------------------------------------------------
// forward: buffers
// ---------------------------------------------------------------------------

struct FwdBufs {
  bool decode1;
  float *logits;
  int32_t *idx;
  float *w;
  float *a_sh, *shared_y;
  int32_t *tiles_sh;
  // small path
  int32_t *plan, *sorted_token, *slot_pos, *tiles;
  uint16_t *x16;
  void *a8;
  float *row_w, *a, *y_rows;
  // large path
  int32_t *offsets, *sorted_slot;
  void *dispatch_ws;
  float *wn2;
  FfnBufs ffn;
};

bool fwd_small(const moe_layer *L, int T) { return (long long)T * L->k <= kSmallSlots; }

bool has_shared(const moe_layer *L) { return L->I_shared > 0 && L->shared_gate; }

bool fwd_decode1(const moe_layer *L, int T) {
  return T == 1 && L->act_fmt == MOE_ACT_BF16 && decode1_supported(L->H, L->I, has_shared(L) ? L->I_shared : 0, L->k);
}

FwdBufs carve_fwd(Carver &c, const moe_layer *L, int T, bool have_logits, bool have_idx,
                  bool have_w) {
  FwdBufs b{};
  const int E = L->E, k = L->k, H = L->H, I = L->I;
  const size_t n = (size_t)T * k;
  const bool shared = L->I_shared > 0 && L->shared_gate;
  b.logits = have_logits ? nullptr : c.take<float>((size_t)T * E);
  b.idx = have_idx ? nullptr : c.take<int32_t>(n);
  b.w = have_w ? nullptr : c.take<float>(n);
  if (shared) {
    b.a_sh = c.take<float>((size_t)T * L->I_shared);
    b.shared_y = c.take<float>((size_t)T * H);
    b.tiles_sh = c.take<int32_t>(gemm_tile_ints(T, 0));
  }
  if (fwd_decode1(L, T)) {
    b.decode1 = true;
    b.a = c.take<float>(n * I);
  } else if (fwd_small(L, T)) {
    b.plan = c.take<int32_t>(plan_ints(std::min<size_t>(E, n)));
    b.sorted_token = c.take<int32_t>(n);
    b.slot_pos = c.take<int32_t>(n);
    b.row_w = c.take<float>(n);
    b.a = c.take<float>(n * I);
    b.y_rows = c.take<float>(n * H);
    b.offsets = c.take<int32_t>(E + 1);
    b.tiles = c.take<int32_t>(gemm_tile_ints((int)n, E));
    b.x16 = c.take<uint16_t>((size_t)T * H);
    if (L->act_fmt == MOE_ACT_MXFP8) b.a8 = c.take<uint8_t>(a8_ws_bytes(T, H, I, (int)n));
  } else {
    b.offsets = c.take<int32_t>(E + 1);
    b.sorted_token = c.take<int32_t>(n);
    b.sorted_slot = c.take<int32_t>(n);
    b.slot_pos = c.take<int32_t>(n);
    b.dispatch_ws = c.take<uint8_t>(dispatch_ws_bytes(T, E, k));
    b.y_rows = c.take<float>(n * H);
    b.wn2 = c.take<float>(E);
    b.ffn = carve_ffn(c, T, (int)n, E, H, I, false, L->act_fmt);
  }
  return b;
}

int check_act(int act, int H, int I, const moe_weights *g, const moe_weights *u,
              const moe_weights *d, bool trace_ok = false) {
  if (act == MOE_ACT_BF16) return MOE_OK;
  if (act != MOE_ACT_MXFP8 && !(trace_ok && act == (MOE_ACT_MXFP8 | MOE_ACT_TRACE)))
    return fail(MOE_EINVAL, "unknown act_fmt %d", act);
  if (!a8_supported(H, I, view_of(*g), view_of(*u), view_of(*d)))
    return fail(MOE_EUNSUPPORTED, "MX-FP8 activations need MXFP4 weights and H, I %% 512 == 0");
  return MOE_OK;
}

int check_layer(const moe_layer *L) {
  if (!L) return fail(MOE_EINVAL, "null layer");
  MOE_TRY(check_route_args(L->route_mode, 0, L->E, L->k));
  if (L->H < 1 || L->I < 1) return fail(MOE_EINVAL, "bad H = %d / I = %d", L->H, L->I);
  if (!L->w_router) return fail(MOE_EINVAL, "null router");
  if (!aligned(L->w_router, 16) || L->H % 8) return fail(MOE_EINVAL, "router misaligned");
  MOE_TRY(check_ffn_weights(L->E, L->H, L->I, &L->gate, &L->up, &L->down));
  MOE_TRY(check_act(L->act_fmt, L->H, L->I, &L->gate, &L->up, &L->down));
  if (L->I_shared < 0) return fail(MOE_EINVAL, "I_shared < 0");
  if (L->steer_dir && !aligned(L->steer_dir, 16))
    return fail(MOE_EINVAL, "steer_dir misaligned");
  if (L->I_shared > 0 && L->shared_gate) {
    if (!L->shared_up || !L->shared_down) return fail(MOE_EINVAL, "incomplete shared expert");
    if (!aligned(L->shared_gate, 16) || !aligned(L->shared_up, 16) ||
        !aligned(L->shared_down, 16))
      return fail(MOE_EINVAL, "shared expert misaligned");
    if (!gemv_supported_k(L->I_shared))
      return fail(MOE_EUNSUPPORTED, "I_shared = %d unsupported", L->I_shared);
  }
  return MOE_OK;
}

}  // namespace

void moe::timer_arm(hipEvent_t start, hipEvent_t stop) { t_start = start, t_stop = stop; }
void moe::timer_take(hipEvent_t *start, hipEvent_t *stop) {
  *start = t_start, *stop = t_stop;
  t_start = t_stop = nullptr;
}

// =============================================================================
// C ABI
// =============================================================================

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }
int moe_abi_version(void) { return MOE_ABI_VERSION; }

size_t moe_route_workspace(int T, int E) {
  if (T < 0 || E < 1) return 0;
  // the logits, then the screened router's E floats
  return (((size_t)T * E * sizeof(float) + 255) & ~size_t(255)) +
         (((size_t)E * sizeof(float) + 255) & ~size_t(255));
}

int moe_route(int mode, int T, int H, int E, int k, const uint16_t *x, const uint16_t *w_router,
              const float *logits_in, const int64_t *token_ids, int32_t *topk_idx, float *topk_w,
              float *logits_out, void *ws, size_t ws_bytes, void *stream) {
  MOE_TRY(check_route_args(mode, T, E, k));
  if (T == 0) return MOE_OK;
  if (!topk_idx || !topk_w) return fail(MOE_EINVAL, "null topk outputs");
  if (mode == MOE_ROUTE_HASH && !token_ids) return fail(MOE_EINVAL, "hash routing needs token_ids");
  hipStream_t s = as_stream(stream);
  const float *lsrc = logits_in;
  if (!logits_in) {
    if (!x || !w_router) return fail(MOE_EINVAL, "null x or router");
    if (H < 8 || H % 8) return fail(MOE_EINVAL, "H = %d must be a positive multiple of 8", H);
    if (!aligned(x, 16) || !aligned(w_router, 16)) return fail(MOE_EINVAL, "x/router misaligned");
    float *dst = logits_out;
    if (!dst) {
      if (!ws || ws_bytes < moe_route_workspace(T, E))
        return fail(MOE_ENOSPC, "route workspace: %zu bytes < %zu", ws_bytes,
                    moe_route_workspace(T, E));
      dst = static_cast<float *>(ws);
    }
    // logits that stay inside the call, for many tokens: the screened router
    // (exact logits for the experts that can reach the top k, -inf for the
    // others; the selection is the same)
    if (!logits_out && (long long)T * k > kSmallSlots && router_screen_supported(H, E)) {
      float *wn2 = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                             (((size_t)T * E * sizeof(float) + 255) & ~size_t(255)));
      MOE_TRY(hip_check(launch_router_screened(mode, T, H, E, k, x, w_router, token_ids, dst, wn2, s),
                        "router"));
    } else {
      MOE_TRY(hip_check(launch_router_logits(T, H, E, x, w_router, dst, s), "router"));
    }
    lsrc = dst;
  } else if (logits_out) {
    MOE_TRY(hip_check(hipMemcpyAsync(logits_out, logits_in, (size_t)T * E * sizeof(float),
                                     hipMemcpyDeviceToDevice, s),
                      "logits copy"));
  }
  return hip_check(launch_select(mode, T, E, k, lsrc, token_ids, topk_idx, topk_w, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, nullptr, s),
                   "select");
}

size_t moe_dispatch_workspace(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return (dispatch_ws_bytes(T, E, k) + 255) & ~size_t(255);
}

int moe_dispatch(int T, int E, int k, const int32_t *topk_idx, int32_t *expert_offsets,
                 int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos, void *ws,
                 size_t ws_bytes, void *stream) {
  MOE_TRY(check_route_args(MOE_ROUTE_SOFTMAX_TOPK, T, E, k));
  if (T == 0) return MOE_OK;
  if (!topk_idx || !expert_offsets || !sorted_token || !sorted_slot || !slot_pos)
    return fail(MOE_EINVAL, "null dispatch pointer");
  if ((long long)T * k > (1ll << 30)) return fail(MOE_EINVAL, "T*k too large");
  if (!ws || ws_bytes < moe_dispatch_workspace(T, E, k))
    return fail(MOE_ENOSPC, "dispatch workspace: %zu bytes < %zu", ws_bytes,
                moe_dispatch_workspace(T, E, k));
  return hip_check(launch_dispatch(T, E, k, topk_idx, expert_offsets, sorted_token, sorted_slot,
                                   slot_pos, ws, as_stream(stream)),
                   "dispatch");
}

int moe_check_buckets(int T, int E, int k, int n_rows, const int32_t *expert_offsets,
                      const int32_t *sorted_token, const int32_t *slot_pos) {
  if (T < 0 || E < 1 || n_rows < 0)
    return fail(MOE_EINVAL, "bad T = %d, E = %d, n_rows = %d", T, E, n_rows);
  if (!expert_offsets) return fail(MOE_EINVAL, "null expert_offsets");
  if (expert_offsets[0] != 0)
    return fail(MOE_EINVAL, "expert_offsets[0] = %d, not 0", expert_offsets[0]);
  for (int e = 0; e < E; e++)
    if (expert_offsets[e + 1] < expert_offsets[e])
      return fail(MOE_EINVAL, "expert_offsets decreases at %d (%d -> %d)", e,
                  expert_offsets[e], expert_offsets[e + 1]);
  if (expert_offsets[E] != n_rows)
    return fail(MOE_EINVAL, "expert_offsets[E] = %d, not n_rows = %d", expert_offsets[E], n_rows);
  if (sorted_token)
    for (int r = 0; r < n_rows; r++)
      if (sorted_token[r] < 0 || sorted_token[r] >= T)
        return fail(MOE_EINVAL, "sorted_token[%d] = %d outside [0, %d)", r, sorted_token[r], T);
  if (slot_pos) {
    if (k < 1 || (long long)T * k != n_rows)
      return fail(MOE_EINVAL, "slot_pos needs T * k = n_rows (T = %d, k = %d, n_rows = %d)", T,
                  k, n_rows);
    std::vector<char> seen((size_t)n_rows, 0);
    for (int f = 0; f < n_rows; f++) {
      const int r = slot_pos[f];
      if (r < 0 || r >= n_rows)
        return fail(MOE_EINVAL, "slot_pos[%d] = %d outside [0, %d)", f, r, n_rows);
      if (seen[r])
        return fail(MOE_EINVAL, "slot_pos[%d] = %d repeats an earlier slot's row", f, r);
      seen[r] = 1;
    }
  }
  return MOE_OK;
}

#ifdef MOE_DEBUG
// host copies of device index arrays for the MOE_DEBUG checks (synchronous)
static int debug_fetch(std::vector<int32_t> &h, const int32_t *d, size_t n, hipStream_t s) {
  h.resize(n);
  if (n == 0) return MOE_OK;
  if (hipMemcpyAsync(h.data(), d, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(MOE_EHIP, "MOE_DEBUG: copy of index arrays failed");
  return MOE_OK;
}
#endif

size_t moe_expert_ffn_workspace(int T, int n_rows, int E, int H, int I, int fmt_gate,
                                int fmt_down, int act_fmt) {
  (void)fmt_gate, (void)fmt_down;
  if (T < 0 || n_rows < 0 || E < 1 || I < 1 || H < 1) return 0;
  Carver c(nullptr);
  carve_ffn(c, T, n_rows, E, H, I, false, act_fmt);
  return c.size();
}

int moe_expert_ffn_a8_layout(int T, int n_rows, int E, int H, int I, size_t *codes_off,
                             size_t *scales_off, size_t *f32_off) {
  if (T < 1 || n_rows < 1 || E < 1 || I < 32 || H < 1 || I % 32)
    return fail(MOE_EINVAL, "bad sizes T = %d, n_rows = %d, E = %d, H = %d, I = %d", T, n_rows,
                E, H, I);
  if (!codes_off || !scales_off || !f32_off) return fail(MOE_EINVAL, "null output");
  Carver c(nullptr);
  FfnBufs b = carve_ffn(c, T, n_rows, E, H, I, false, MOE_ACT_MXFP8);
  (void)b;
  const size_t a8 = c.last;  // the MX-FP8 region is carved last
  {
    Carver d(reinterpret_cast<void *>(uintptr_t(256)));  // offsets relative to a fake base
    *f32_off = reinterpret_cast<uintptr_t>(
                   carve_ffn(d, T, n_rows, E, H, I, false, MOE_ACT_MXFP8).a) - 256;
  }
  a8_layout(T, H, I, n_rows, codes_off, scales_off);
  *codes_off += a8;
  *scales_off += a8;
  return MOE_OK;
}

int moe_expert_ffn(int T, int H, int I, const uint16_t *x, const moe_weights *gate,
                   const moe_weights *up, const moe_weights *down, int act_fmt,
                   const int32_t *expert_offsets, const int32_t *sorted_token, int n_rows,
                   float *y_rows, void *ws, size_t ws_bytes, void *stream) {
  if (T < 0 || n_rows < 0) return fail(MOE_EINVAL, "negative T or n_rows");
  if (!gate) return fail(MOE_EINVAL, "null gate");
  const int E = gate->n_experts;
  MOE_TRY(check_ffn_weights(E, H, I, gate, up, down));
  MOE_TRY(check_act(act_fmt, H, I, gate, up, down, true));
  if (T == 0 || n_rows == 0) return MOE_OK;
  if (!x || !y_rows) return fail(MOE_EINVAL, "null x or y_rows");
  if (!aligned(x, 16) || !aligned(y_rows, 16)) return fail(MOE_EINVAL, "x/y_rows misaligned");
  const bool dense = expert_offsets == nullptr;
  if (dense && n_rows != T) return fail(MOE_EINVAL, "dense call needs n_rows == T");
  if (!dense && !sorted_token) return fail(MOE_EINVAL, "null sorted_token");
  const size_t need =
      moe_expert_ffn_workspace(T, n_rows, E, H, I, gate->fmt, down->fmt, act_fmt);
  if (!ws || ws_bytes < need)
    return fail(MOE_ENOSPC, "expert_ffn workspace: %zu bytes < %zu", ws_bytes, need);
#ifdef MOE_DEBUG
  if (!dense) {
    std::vector<int32_t> ho, hs;
    MOE_TRY(debug_fetch(ho, expert_offsets, (size_t)E + 1, as_stream(stream)));
    MOE_TRY(debug_fetch(hs, sorted_token, (size_t)n_rows, as_stream(stream)));
    MOE_TRY(moe_check_buckets(T, E, 0, n_rows, ho.data(), hs.data(), nullptr));
  }
#endif
  Carver c(ws);
  FfnBufs b = carve_ffn(c, T, n_rows, E, H, I, dense, act_fmt);
  return run_ffn(T, H, I, x, view_of(*gate), view_of(*up), view_of(*down), act_fmt,
                 expert_offsets, sorted_token, n_rows, y_rows, b, as_stream(stream));
}

int moe_combine(int T, int H, int k, const float *y_rows, const int32_t *slot_pos,
                const float *topk_w, const float *shared_y, const float *steer_dir,
                float steer_alpha, float *out_f32, uint16_t *out_bf16, void *stream) {
  if (T < 0 || H < 1 || k < 1 || k > 16) return fail(MOE_EINVAL, "bad T/H/k");
  if (T == 0) return MOE_OK;
  if (H % 4) return fail(MOE_EINVAL, "H = %d must be a multiple of 4", H);
  if (!y_rows || !slot_pos || !topk_w || !out_f32) return fail(MOE_EINVAL, "null combine pointer");
  if (!aligned(y_rows, 16) || !aligned(out_f32, 16) || (shared_y && !aligned(shared_y, 16)) ||
      (steer_dir && !aligned(steer_dir, 16)) || (out_bf16 && !aligned(out_bf16, 8)))
    return fail(MOE_EINVAL, "combine buffers misaligned");
#ifdef MOE_DEBUG
  {
    std::vector<int32_t> hp;
    const int n = T * k;
    MOE_TRY(debug_fetch(hp, slot_pos, (size_t)n, as_stream(stream)));
    for (int f = 0; f < n; f++)
      if (hp[f] < 0 || hp[f] >= n)
        return fail(MOE_EINVAL, "slot_pos[%d] = %d outside [0, %d)", f, hp[f], n);
  }
#endif
  return hip_check(launch_combine(T, H, k, y_rows, slot_pos, topk_w, shared_y, steer_dir,
                                  steer_alpha, out_f32, out_bf16, as_stream(stream)),
                   "combine");
}

size_t moe_forward_workspace(const moe_layer *L, int T) {
  if (!L || T < 0 || L->E < 1 || L->k < 1) return 0;
  Carver c(nullptr);
  carve_fwd(c, L, T, false, false, false);
  return c.size();
}

static int forward_impl(const moe_layer *L, int T, const uint16_t *x, const float *logits_in,
                        const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                        int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                        const moe_side_stream *side_in, void *stream, Marker &mk) {
  MOE_TRY(check_layer(L));
  if (T < 0) return fail(MOE_EINVAL, "T = %d < 0", T);
  if (T == 0) return MOE_OK;
  if (!x || !out_f32) return fail(MOE_EINVAL, "null x or out");
  if (!aligned(x, 16) || !aligned(out_f32, 16) || (out_bf16 && !aligned(out_bf16, 8)))
    return fail(MOE_EINVAL, "x/out misaligned");
  if (L->route_mode == MOE_ROUTE_HASH && !token_ids)
    return fail(MOE_EINVAL, "hash routing needs token_ids");
  if (side_in && (!side_in->stream || !side_in->fork || !side_in->join))
    return fail(MOE_EINVAL, "side stream: stream, fork and join must all be given");
  if (side_in && side_in->stream == stream)
    return fail(MOE_EINVAL, "side stream: must differ from the call's stream");
  const size_t need = moe_forward_workspace(L, T);
  if (!ws || ws_bytes < need)
    return fail(MOE_ENOSPC, "forward workspace: %zu bytes < %zu", ws_bytes, need);

  hipStream_t s = as_stream(stream);
  const int E = L->E, k = L->k, H = L->H, I = L->I, n = T * k;
  Carver c(ws);
  FwdBufs b = carve_fwd(c, L, T, false, false, false);
  int32_t *idx = topk_idx_out ? topk_idx_out : b.idx;
  float *w = topk_w_out ? topk_w_out : b.w;
  if (b.decode1) {
    DecodeArgs a{};
    a.H = H, a.I = I, a.E = E, a.k = k, a.mode = L->route_mode;
    a.Is = has_shared(L) ? L->I_shared : 0;
    a.x = x, a.w_router = L->w_router, a.logits_in = logits_in, a.tid = token_ids;
    a.gate = view_of(L->gate), a.up = view_of(L->up), a.down = view_of(L->down);
    if (a.Is) {
      a.sg = bf16_view(L->shared_gate, a.Is, H);
      a.su = bf16_view(L->shared_up, a.Is, H);
      a.sd = bf16_view(L->shared_down, H, a.Is);
    }
    a.logits = b.logits, a.a_sh = b.a_sh, a.a = b.a, a.shared_y = b.shared_y;
    // the split forms reuse the fp32 buffers: two uint16 halves per float
    a.a_sh_hi = reinterpret_cast<uint16_t *>(b.a_sh);
    a.a_sh_lo = a.Is ? a.a_sh_hi + a.Is : nullptr;
    a.a_hi = reinterpret_cast<uint16_t *>(b.a);
    a.a_lo = a.a_hi + (size_t)k * I;
    a.topk_idx = idx, a.topk_w = w, a.out = out_f32, a.out_bf16 = out_bf16;
    a.steer_dir = L->steer_dir, a.steer_alpha = L->steer_alpha;
    return hip_check(launch_decode1(a, s, mark_cb, &mk), "decode");
  }
  const bool shared = L->I_shared > 0 && L->shared_gate;
  // the shared expert goes first, on the caller's side stream when one is
  // given (not when each kernel is timed: the marks time one stream)
  SideStream side_v{};
  SideStream *side = nullptr;
  if (shared && !mk.m && side_in) {
    side_v.s = as_stream(side_in->stream);
    side_v.fork = static_cast<hipEvent_t>(side_in->fork);
    side_v.join = static_cast<hipEvent_t>(side_in->join);
    side = &side_v;
  }
  if (side) {
    MOE_TRY(hip_check(hipEventRecord(side->fork, s), "fork"));
    MOE_TRY(hip_check(hipStreamWaitEvent(side->s, side->fork, 0), "fork"));
  }
  int rc_sh = MOE_OK;
  if (shared) {
    const hipStream_t ss = side ? side->s : s;
    const WView sg = bf16_view(L->shared_gate, L->I_shared, H);
    const WView su = bf16_view(L->shared_up, L->I_shared, H);
    const WView sd = bf16_view(L->shared_down, H, L->I_shared);
    if (skinny_supported(H, L->I_shared, T, sg, sd)) {
      rc_sh = hip_check(launch_skinny_ffn(sg, su, sd, H, L->I_shared, T, x,
                                          reinterpret_cast<uint16_t *>(b.a_sh), b.shared_y, ss,
                                          mark_cb, &mk, kSharedGemmNames),
                        "shared skinny");
    } else if (use_gemm(T, H, L->I_shared, 1, T, true, MOE_FMT_BF16, MOE_FMT_BF16)) {
      rc_sh = hip_check(launch_gemm_ffn(sg, su, sd, H, L->I_shared, T, x, nullptr, nullptr, T,
                                        b.tiles_sh, reinterpret_cast<uint16_t *>(b.a_sh), nullptr,
                                        b.shared_y, ss, mark_cb, &mk, kSharedGemmNames),
                        "shared gemm");
    } else {
      mk("shared_gateup");
      rc_sh = hip_check(
          launch_gateup_gemv(sg, su, H, L->I_shared, x, nullptr, T, nullptr, b.a_sh, ss),
          "shared gate/up");
      if (rc_sh == MOE_OK) {
        mk("shared_down");
        rc_sh = hip_check(launch_down_gemv(sd, H, L->I_shared, b.a_sh, nullptr, T, b.shared_y, ss),
                          "shared down");
      }
    }
  }
  if (side) {
    // the caller's stream waits for the side stream only before the combine,
    // but the join is recorded now, so that no path leaves the fork open
    const int rc_j = hip_check(hipEventRecord(side->join, side->s), "join");
    if (rc_sh == MOE_OK) rc_sh = rc_j;
  }
  auto join = [&]() -> int {
    if (side) return hip_check(hipStreamWaitEvent(s, side->join, 0), "join");
    return MOE_OK;
  };
  // the routed part on the caller's stream, up to the combine
  auto routed = [&]() -> int {
    const float *logits = logits_in;
    if (!logits) {
      mk("router");
      // the logits stay inside the call: many tokens take the screened router
      if (!fwd_small(L, T) && router_screen_supported(H, E))
        MOE_TRY(hip_check(launch_router_screened(L->route_mode, T, H, E, k, x, L->w_router,
                                                 token_ids, b.logits, b.wn2, s),
                          "router"));
      else
        MOE_TRY(hip_check(launch_router_logits(T, H, E, x, L->w_router, b.logits, s), "router"));
      logits = b.logits;
    }
    const WView g = view_of(L->gate), u = view_of(L->up), d = view_of(L->down);
    if (fwd_small(L, T)) {
      mk("select_plan");
      MOE_TRY(hip_check(launch_select(L->route_mode, T, E, k, logits, token_ids, idx, w, b.offsets,
                                      b.sorted_token, nullptr, b.slot_pos, b.row_w, b.plan, s),
                        "select"));
      if (L->act_fmt == MOE_ACT_MXFP8)
        return hip_check(launch_a8_ffn(g, u, d, H, I, T, x, b.offsets, b.sorted_token, n, b.tiles,
                                       b.a8, nullptr, b.y_rows, s, mark_cb, &mk, kA8Names),
                         "a8 ffn");
      if (use_gemm(T, H, I, E, n, false, g.fmt, d.fmt))
        // several tokens: every selected expert's weights once, all its rows per load
        return hip_check(launch_gemm_ffn(g, u, d, H, I, T, x, b.offsets, b.sorted_token, n,
                                         b.tiles, reinterpret_cast<uint16_t *>(b.a), b.x16,
                                         b.y_rows, s, mark_cb, &mk, kRoutedGemmNames),
                         "gemm ffn");
      const int max_active = std::min(E, n);
      mk("routed_gateup");
      MOE_TRY(hip_check(
          launch_gateup_gemv(g, u, H, I, x, b.plan, max_active, b.sorted_token, b.a, s),
          "gate/up"));
      mk("routed_down");
      return hip_check(launch_down_gemv(d, H, I, b.a, b.plan, max_active, b.y_rows, s), "down");
    }
    mk("select");
    MOE_TRY(hip_check(launch_select(L->route_mode, T, E, k, logits, token_ids, idx, w, nullptr,
                                    nullptr, nullptr, nullptr, nullptr, nullptr, s),
                      "select"));
    MOE_TRY(hip_check(launch_dispatch(T, E, k, idx, b.offsets, b.sorted_token, b.sorted_slot,
                                      b.slot_pos, b.dispatch_ws, s, mark_cb, &mk),
                      "dispatch"));
    return run_ffn(T, H, I, x, g, u, d, L->act_fmt, b.offsets, b.sorted_token, n, b.y_rows, b.ffn,
                   s, &mk);
  };
  const int rc = rc_sh == MOE_OK ? routed() : rc_sh;
  const int rc_join = join();  // on every path: no fork is left open
  if (rc != MOE_OK) return rc;
  if (rc_join != MOE_OK) return rc_join;
  mk("combine");
  return hip_check(launch_combine(T, H, k, b.y_rows, b.slot_pos, w, b.shared_y, L->steer_dir,
                                  L->steer_alpha, out_f32, out_bf16, s),
                   "combine");
}

int moe_forward(const moe_layer *L, int T, const uint16_t *x, const float *logits_in,
                const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                const moe_side_stream *side, void *stream) {
  Marker none;
  return forward_impl(L, T, x, logits_in, token_ids, out_f32, out_bf16, topk_idx_out, topk_w_out,
                      ws, ws_bytes, side, stream, none);
}

// ---------------------------------------------------------------------------
// moe_forward_static: moe_forward on a scratch buffer the library owns, for
// callers that cannot allocate.  The buffer is a file-scope device array; in
// host code its name is only a stand-in, so its address on each device is
// taken once with hipGetSymbolAddress (with that device current) and kept.
// ---------------------------------------------------------------------------
}  // extern "C"

static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

int static_scratch(void **out) {
  int dev = -1;
  MOE_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MOE_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    MOE_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress"));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_forward_static(const moe_layer *L, int T, const uint16_t *x, const float *logits_in,
                       const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                       int32_t *topk_idx_out, float *topk_w_out, void *stream) {
  MOE_TRY(check_layer(L));
  if (T < 0) return fail(MOE_EINVAL, "T = %d < 0", T);
  if (T == 0) return MOE_OK;
  const size_t need = moe_forward_workspace(L, T);
  if (need > MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_ENOSPC, "moe_forward_static: T = %d needs %zu bytes of scratch, above its "
                "%zu-byte maximum", T, need, (size_t)MOE_STATIC_SCRATCH_BYTES);
  void *ws = nullptr;
  MOE_TRY(static_scratch(&ws));
  Marker none;
  return forward_impl(L, T, x, logits_in, token_ids, out_f32, out_bf16, topk_idx_out, topk_w_out,
                      ws, MOE_STATIC_SCRATCH_BYTES, nullptr, stream, none);
}

// ---------------------------------------------------------------------------
// the routed-expert residency cache
// ---------------------------------------------------------------------------

size_t moe_cache_state_ints(int E, int n_slots) {
  if (E < 1 || n_slots < 1) return 0;
  return cache_state_ints(E, n_slots);
}

static int check_cache(const moe_expert_cache *c, int E, int k) {
  if (!c || !c->state) return fail(MOE_EINVAL, "cache: null cache or state");
  if (c->n_slots < k || c->n_slots > 1024)
    return fail(MOE_EINVAL, "cache: n_slots = %d outside [k = %d, 1024]", c->n_slots, k);
  return MOE_OK;
}

int moe_cache_reset(const moe_expert_cache *c, int E, void *stream) {
  if (E < 1 || E > 1024) return fail(MOE_EINVAL, "E = %d outside [1, 1024]", E);
  MOE_TRY(check_cache(c, E, 1));
  return hip_check(launch_cache_reset(E, c->n_slots, c->state, as_stream(stream)), "cache reset");
}

// the byte planes of a projection, host (all experts) and slots
static int cache_planes(const moe_weights &host, const moe_weights &slot, CacheStep &cs) {
  const size_t pd = expert_data_bytes(host.fmt, host.rows, host.cols);
  const size_t ps = expert_scale_bytes(host.fmt, host.rows, host.cols);
  const void *planes[2] = {host.data, host.scales};
  void *dplanes[2] = {const_cast<void *>(slot.data), const_cast<void *>(slot.scales)};
  const size_t per[2] = {pd, ps};
  for (int i = 0; i < 2; i++) {
    if (!per[i]) continue;
    if (per[i] % 16 || !aligned(planes[i], 16) || !aligned(dplanes[i], 16))
      return fail(MOE_EUNSUPPORTED, "cache: plane bytes per expert (%zu) or bases not 16-byte "
                  "aligned", per[i]);
    void *dev = nullptr;
    MOE_TRY(hip_check(hipHostGetDevicePointer(&dev, const_cast<void *>(planes[i]), 0),
                      "cache: host weights must be pinned, device-mapped host memory"));
    cs.src[cs.n_planes] = static_cast<const uint8_t *>(dev);
    cs.dst[cs.n_planes] = static_cast<uint8_t *>(dplanes[i]);
    cs.per_bytes[cs.n_planes] = per[i];
    cs.n_planes++;
  }
  return MOE_OK;
}

int moe_forward_cached(const moe_layer *L, const moe_expert_cache *c, int T, const uint16_t *x,
                       const float *logits_in, const int64_t *token_ids, float *out_f32,
                       uint16_t *out_bf16, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                       size_t ws_bytes, void *stream) {
  MOE_TRY(check_layer(L));
  MOE_TRY(check_cache(c, L->E, L->k));
  const int C = c->n_slots;
  MOE_TRY(check_ffn_weights(C, L->H, L->I, &c->slot_gate, &c->slot_up, &c->slot_down));
  if (c->slot_gate.fmt != L->gate.fmt || c->slot_down.fmt != L->down.fmt ||
      (c->slot_gate.fmt == MOE_FMT_VQ2 && c->slot_gate.codebook != L->gate.codebook))
    return fail(MOE_EINVAL, "cache: slots differ in format (or codebook) from the layer");
  if (T == 0) return MOE_OK;
  if (T != 1 || !fwd_decode1(L, T))
    return fail(MOE_EUNSUPPORTED, "cache: one-token decode layers only");
  if (!x || !out_f32) return fail(MOE_EINVAL, "null x or out");
  if (!aligned(x, 16) || !aligned(out_f32, 16) || (out_bf16 && !aligned(out_bf16, 8)))
    return fail(MOE_EINVAL, "x/out misaligned");
  if (L->route_mode == MOE_ROUTE_HASH && !token_ids)
    return fail(MOE_EINVAL, "hash routing needs token_ids");
  const size_t need = moe_forward_workspace(L, T);
  if (!ws || ws_bytes < need)
    return fail(MOE_ENOSPC, "forward workspace: %zu bytes < %zu", ws_bytes, need);
  Carver cv(ws);
  FwdBufs b = carve_fwd(cv, L, T, false, false, false);
  CacheStep cs{};
  MOE_TRY(cache_planes(L->gate, c->slot_gate, cs));
  MOE_TRY(cache_planes(L->up, c->slot_up, cs));
  MOE_TRY(cache_planes(L->down, c->slot_down, cs));
  DecodeArgs a{};
  const int H = L->H, I = L->I, E = L->E, k = L->k;
  a.H = H, a.I = I, a.E = E, a.k = k, a.mode = L->route_mode;
  a.Is = has_shared(L) ? L->I_shared : 0;
  a.x = x, a.w_router = L->w_router, a.logits_in = logits_in, a.tid = token_ids;
  a.gate = view_of(c->slot_gate), a.up = view_of(c->slot_up), a.down = view_of(c->slot_down);
  if (a.Is) {
    a.sg = bf16_view(L->shared_gate, a.Is, H);
    a.su = bf16_view(L->shared_up, a.Is, H);
    a.sd = bf16_view(L->shared_down, H, a.Is);
  }
  a.logits = b.logits, a.a_sh = b.a_sh, a.a = b.a, a.shared_y = b.shared_y;
  a.a_sh_hi = reinterpret_cast<uint16_t *>(b.a_sh);
  a.a_sh_lo = a.Is ? a.a_sh_hi + a.Is : nullptr;
  a.a_hi = reinterpret_cast<uint16_t *>(b.a);
  a.a_lo = a.a_hi + (size_t)k * I;
  a.topk_idx = topk_idx_out ? topk_idx_out : b.idx;
  a.topk_w = topk_w_out ? topk_w_out : b.w;
  a.out = out_f32, a.out_bf16 = out_bf16;
  a.steer_dir = L->steer_dir, a.steer_alpha = L->steer_alpha;
  a.slot_idx = c->state + cache_slot_idx_offset(E, C);
  cs.mode = L->route_mode, cs.E = E, cs.C = C, cs.k = k;
  cs.logits = logits_in ? logits_in : b.logits;
  cs.tid = token_ids;
  cs.state = c->state;
  cs.topk_idx = a.topk_idx, cs.topk_w = a.topk_w;
  Marker none;
  return hip_check(launch_decode1(a, as_stream(stream), mark_cb, &none, &cs), "cached decode");
}

int moe_forward_marked(const moe_layer *L, int T, const uint16_t *x, const float *logits_in,
                       const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                       int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                       moe_mark *marks, int max_marks, int *n_marks, void *stream) {
  if (max_marks < 0 || (max_marks > 0 && !marks)) return fail(MOE_EINVAL, "bad marks");
  for (int i = 0; i < max_marks; i++)
    if (!marks[i].start || !marks[i].stop) return fail(MOE_EINVAL, "mark %d lacks an event", i);
  Marker mk;
  mk.m = marks;
  mk.max = max_marks;
  const int rc = forward_impl(L, T, x, logits_in, token_ids, out_f32, out_bf16, topk_idx_out,
                              topk_w_out, ws, ws_bytes, nullptr, stream, mk);
  if (n_marks) *n_marks = mk.n;
  return rc;
}


int moe_mxfp8_quantize(int rows, int K, const uint16_t *x, uint8_t *q, uint8_t *scales,
                       void *stream) {
  if (rows < 0 || K < 32 || K % 32) return fail(MOE_EINVAL, "bad rows = %d / K = %d", rows, K);
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return fail(MOE_EINVAL, "null pointer");
  if (!aligned(x, 16) || !aligned(q, 8)) return fail(MOE_EINVAL, "x/q misaligned");
  return hip_check(launch_mx8_quant(rows, K, x, q, scales, as_stream(stream)), "mxfp8 quantize");
}

int moe_dequantize(const moe_weights *w, int expert, int64_t w0, int64_t count, float *out,
                   void *stream) {
  if (!w) return fail(MOE_EINVAL, "null weights");
  MOE_TRY(check_weights(w, "weights", w->n_experts, w->rows, w->cols));
  if (expert < 0 || expert >= w->n_experts) return fail(MOE_EINVAL, "expert %d out of range", expert);
  const int64_t per = (int64_t)w->rows * w->cols;
  if (w0 < 0 || count < 0 || w0 + count > per) return fail(MOE_EINVAL, "range out of bounds");
  if (count == 0) return MOE_OK;
  if (!out) return fail(MOE_EINVAL, "null out");
  return hip_check(launch_dequant(view_of(*w), expert, w0, count, out, as_stream(stream)),
                   "dequantize");
}

}  // extern "C"
