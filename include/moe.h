/*
 * moe.h -- libmoe: the routed-expert mixture-of-experts FFN layer of a
 * DeepSeek-V4-Flash-class model on one AMD MI355X (gfx950).
 *
 * The layer (ds4 / DwarfStar 4 pages): a full-precision router picks k of E
 * routed experts per token; each routed expert is a SwiGLU FFN whose weights
 * are 2-bit quantized -- an IQ2_XXS-class codebook format for up/gate and
 * Q2_K for down -- or MXFP4; a bf16 shared expert is added to the weighted
 * sum of the routed experts ("DS4 (DwarfStar 4): Chay DeepSeek V4 Flash
 * Local voi Metal & CUDA", dibi8.com, "Cac Doi Moi Kien Truc Chinh" item 1;
 * "DwarfStar: a focused local inference engine for DeepSeek V4 and GLM 5.2",
 * hysenlabs.com, "Model support and quantization"; grapeot.me ds4 post,
 * opening paragraphs, for hash MoE routing).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless stated.  Arrays are row-major and
 *    contiguous.  bf16 and fp16 values are passed as their uint16 bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls validate their arguments on the host, enqueue kernels on
 *    `stream` and return without synchronising; results are ready when the
 *    stream reaches them.  No call allocates or frees memory: scratch space
 *    is the caller's `ws` buffer, sized by the matching *_workspace query.
 *  - Return value: MOE_OK, or a negative MOE_E* code with a message
 *    available from moe_last_error() (thread-local).  Argument errors are
 *    detected before anything is enqueued.  Device-side faults are not
 *    reported by these calls.
 *  - T == 0 (no tokens) is a valid no-op.
 *  - Calls are reentrant; concurrent calls must use distinct ws buffers.
 *    The library creates no HIP objects -- every stream and event it uses is
 *    the caller's -- and holds no mutable state of its own, except the
 *    device scratch of moe_forward_static (below).
 *
 * Value ranges (preconditions the host cannot check without reading device
 * memory; outside them results may be inf/NaN where the CPU reference is
 * finite).  The matrix-core paths (moe_expert_ffn / moe_forward from four
 * tokens on, VQ2 or Q2K gate/up or any down projection) and the one-token
 * down projection of Q2K and MXFP4 experts round the following to IEEE
 * binary16, so each must stay below 65504 in magnitude: the bf16 tokens
 * (VQ2 and Q2K gate/up), the SwiGLU output, each dequantized VQ2 and Q2K
 * weight and the Q2K terms d*scale and dmin*min.  Values below 2^-14 become
 * binary16 subnormals: an absolute error of at most 2^-25 each.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument: null pointer, shape, k, alignment */
  MOE_EUNSUPPORTED = -2, /* valid but unsupported format / shape combination */
  MOE_ENOSPC = -3,       /* workspace smaller than the *_workspace query */
  MOE_EHIP = -4          /* the HIP runtime refused a launch */
};

/* Weight formats.  Blocking is along the row-major flattened [rows, cols]
 * matrix of one expert; experts are stored one after another.
 *  MOE_FMT_BF16  data: uint16 bf16 [E][rows][cols].
 *  MOE_FMT_Q2K   data: 84-byte super-blocks of 256 consecutive weights,
 *                {uint8 sc[16]; uint8 qs[64]; fp16 d; fp16 dmin}:
 *                sub-block s = i/16 has scale sc[s]&15 and min sc[s]>>4,
 *                q_i = (qs[i/4] >> 2*(i%4)) & 3, w_i = d*scale*q_i - dmin*min.
 *                Requires rows*cols % 256 == 0; a block may span rows.
 *  MOE_FMT_VQ2   2.0625-bit codebook format standing for the pages'
 *                IQ2_XXS-class up/gate format: data: uint8 codes
 *                [E][rows][cols/4]; scales: fp16 [E][rows][cols/256];
 *                codebook: int8 [256][4];
 *                w[n][k] = scale[n][k/256] * codebook[code[n][k/4]][k%4].
 *                Requires cols % 256 == 0.
 *  MOE_FMT_MXFP4 OCP MX v1.0 FP4: data: uint8 [E][rows][cols/2] E2M1
 *                nibbles (even k in the low nibble); scales: uint8 E8M0
 *                [E][rows][cols/32]; w = E2M1 * 2^(e-127).
 *                Requires cols % 32 == 0. */
enum { MOE_FMT_BF16 = 0, MOE_FMT_Q2K = 1, MOE_FMT_VQ2 = 2, MOE_FMT_MXFP4 = 3 };

/* Routing modes.
 *  MOE_ROUTE_SOFTMAX_TOPK: the k largest router logits (equal logits go to
 *    the lower expert index; NaN ranks lowest), weights = softmax over the
 *    k selected logits (they sum to 1).
 *  MOE_ROUTE_HASH: expert j of token t is ((splitmix64(token_id[t]) + j)
 *    mod 2^64) mod E, j = 0..k-1, where splitmix64(x) is the first output of
 *    SplitMix64 seeded with x; weights = softmax over those k router logits. */
enum { MOE_ROUTE_SOFTMAX_TOPK = 0, MOE_ROUTE_HASH = 1 };

/* One projection of n_experts experts, each [rows, cols] (out x in). */
typedef struct {
  int32_t fmt, n_experts, rows, cols;
  const void *data;        /* see MOE_FMT_*; 16-byte aligned */
  const void *scales;      /* VQ2: fp16 plane; MXFP4: E8M0 plane; else NULL */
  const int8_t *codebook;  /* VQ2: int8 [256][4]; else NULL */
} moe_weights;

/* Activations entering the routed experts' projections.
 *  MOE_ACT_BF16   the bf16 tokens and an fp32 SwiGLU output, as given.
 *  MOE_ACT_MXFP8  the A8 variant for MXFP4 experts: both are first quantized
 *                 to OCP MX-FP8 -- per 32 consecutive values along K an E8M0
 *                 scale X = 2^(floor(log2 amax) - 8) and E4M3 elements, the
 *                 nearest to v / X (ties to an even mantissa, saturating at
 *                 448; amax == 0 gives scale byte 0 and zero elements) -- and
 *                 multiplied with the raw FP4 weights on the FP4 matrix
 *                 instructions.  MXFP4 gate/up/down only; H, I multiples of
 *                 512.  (hysenlabs.com ds4 page, "Model support and
 *                 quantization": the MXFP4 variant keeps the released FP4
 *                 experts.) */
enum { MOE_ACT_BF16 = 0, MOE_ACT_MXFP8 = 1 };
/* moe_expert_ffn only: MOE_ACT_MXFP8 | MOE_ACT_TRACE also leaves the fp32
 * SwiGLU output, before its MX-FP8 quantization, in the workspace (see
 * moe_expert_ffn_a8_layout), for tests of the quantizer on the values the
 * matrix cores produced. */
#define MOE_ACT_TRACE 0x100

/* One MoE FFN layer.  gate/up are [E][I][H], down is [E][H][I]; the shared
 * expert (optional: NULL pointers or I_shared == 0) is bf16 [I_shared][H],
 * [I_shared][H], [H][I_shared]; the router is bf16 [E][H].  act_fmt: a
 * MOE_ACT_* value for the routed experts (the shared expert is always bf16).
 * steer_dir: optional fp32 [H] direction added to the layer's output with
 * strength steer_alpha (see moe_combine); NULL for none. */
typedef struct {
  int32_t H, I, E, k, I_shared, route_mode;
  const uint16_t *w_router;
  moe_weights gate, up, down;
  const uint16_t *shared_gate, *shared_up, *shared_down;
  int32_t act_fmt;
  const float *steer_dir;
  float steer_alpha;
} moe_layer;

/* A second stream for moe_forward, owned by the caller: `stream` (a
 * hipStream_t, default priority) runs the shared expert beside the routed
 * work; `fork` and `join` are hipEvent_t (timing may be disabled) that the
 * call records -- fork on the caller's stream before anything else, join on
 * `stream` after the shared expert -- and waits on (the caller's stream
 * waits for join before the combine).  Concurrent calls need distinct
 * moe_side_stream objects. */
typedef struct {
  void *stream;
  void *fork;
  void *join;
} moe_side_stream;

/* Text of the last error on the calling thread ("" if none). */
const char *moe_last_error(void);
int moe_abi_version(void);

/* ---------------------------------------------------------------------- */
/* moe_route: router logits + expert selection.
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h], every product exact and
 *   the sum accumulated in fp64, rounded once to fp32 (the router stays at
 *   full precision: dibi8.com ds4 guide, "Cac Doi Moi Kien Truc Chinh" item
 *   1).  Then MOE_ROUTE_SOFTMAX_TOPK or MOE_ROUTE_HASH selection.
 * Exactness domain: the kernels sum in other orders than h = 0, 1, ...; the
 *   result equals the h-order fp64 sum bit for bit whenever that sum is exact
 *   in fp64, in any order -- it is when sum_h |x_h w_h| is below 2^53 times
 *   the last bit of the smallest nonzero product, e.g. when every nonzero x
 *   and router weight has magnitude >= 2^-14 and sum_h |x_h w_h| < 2^11 --
 *   and so the selected experts are reproducible.  Outside it
 *   the fp64 sums may differ in their last bits, which changes the fp32
 *   logit only when it lies within 2^-29 relative of an fp32 rounding
 *   boundary.
 * x: bf16 [T][H]; w_router: bf16 [E][H].
 * logits_in: optional fp32 [T][E]; when given, the router GEMM is skipped
 *   and these logits are used (x and w_router may then be NULL).
 * token_ids: int64 [T], required for MOE_ROUTE_HASH, else ignored.
 * topk_idx: int32 [T][k] out; topk_w: fp32 [T][k] out (softmax weights in
 *   selection order); logits_out: optional fp32 [T][E] out.
 * ws: scratch of moe_route_workspace(T, E) bytes (may be 0 when logits_out
 *   or logits_in is given).  1 <= k <= min(E, 16); E <= 1024.
 * Without logits_in and logits_out, above 1024 (token, choice) slots (E a
 *   multiple of 64 up to 256, H a multiple of 512 up to 8192), the logits
 *   are computed exactly only for the experts whose bf16 matrix-core
 *   approximation, with a rigorous error bound, can reach the top k; the
 *   selected experts and weights are the same bit for bit. */
size_t moe_route_workspace(int T, int E);
int moe_route(int mode, int T, int H, int E, int k, const uint16_t *x, const uint16_t *w_router,
              const float *logits_in, const int64_t *token_ids, int32_t *topk_idx, float *topk_w,
              float *logits_out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* moe_dispatch: bucket the T*k (token, choice) slots by expert, stable in
 * slot order f = t*k + j (a counting sort by prefix sum).  The pages route
 * each token to k routed experts (dibi8.com ds4 guide, "Cac Doi Moi Kien
 * Truc Chinh" item 1; grapeot.me ds4 post, opening paragraphs, for hash
 * routing) but describe no bucketing: this grouping of the slots by expert
 * is the library's own, so that each expert's weights are read once for all
 * of its tokens:
 *   expert_offsets[e] = number of slots routed to experts < e
 *   (expert_offsets[E] = T*k); bucket e is rows [offsets[e], offsets[e+1])
 *   listing its slots in ascending f:
 *   sorted_slot[r] = f, sorted_token[r] = f / k, slot_pos[f] = r.
 * topk_idx: int32 [T][k] with values in [0, E) (not checked on device).
 * Outputs are int32: expert_offsets [E+1], the others [T*k]. */
size_t moe_dispatch_workspace(int T, int E, int k);
int moe_dispatch(int T, int E, int k, const int32_t *topk_idx, int32_t *expert_offsets,
                 int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos, void *ws,
                 size_t ws_bytes, void *stream);

/* moe_check_buckets: validate bucket arrays held in host memory: host
 * copies of moe_dispatch's outputs, or buckets a caller built for
 * moe_expert_ffn and moe_combine.  The bucketing is the library's own, as
 * for moe_dispatch (the pages describe none).
 *   expert_offsets: int32 [E+1]; it must start at 0, never decrease, and
 *     end at n_rows.
 *   sorted_token: int32 [n_rows], each value in [0, T); NULL skips this
 *     check.
 *   slot_pos: int32 [T*k] with T*k == n_rows, a permutation of [0, n_rows),
 *     so that every bucket row is the home of exactly one slot; NULL skips
 *     this check.
 * It reads only these arrays and makes no device call.  Returns MOE_OK, or
 * MOE_EINVAL with a message naming the first index at fault.
 * A library built with MOE_DEBUG defined runs the same checks before any
 * launch, on host copies of its device inputs:
 *   moe_expert_ffn checks expert_offsets and sorted_token;
 *   moe_combine checks that each slot_pos value lies in [0, T*k).
 * The copies synchronize the stream, so such a build cannot be captured
 * in a graph. */
int moe_check_buckets(int T, int E, int k, int n_rows, const int32_t *expert_offsets,
                      const int32_t *sorted_token, const int32_t *slot_pos);

/* ---------------------------------------------------------------------- */
/* moe_expert_ffn: SwiGLU FFN of each expert over its bucket of tokens:
 *   for bucket row r of expert e, token t = sorted_token[r]:
 *   y_rows[r] = Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),
 * with the weights dequantized on the fly (routed experts in 2-bit formats,
 * up/gate IQ2_XXS-class and down Q2_K: dibi8.com ds4 guide, "Cac Doi Moi
 * Kien Truc Chinh" item 1; MXFP4 experts: hysenlabs.com ds4 page, "Model
 * support and quantization"; the SwiGLU form is the library's reading).  x: bf16 [T][H]; gate/up/down
 * as in moe_layer (any of the formats; gate and up of one format).
 * expert_offsets: int32 [E+1] and sorted_token: int32 [n_rows] from
 *   moe_dispatch; expert_offsets == NULL means one dense expert (expert 0
 *   of the weights) applied to all T tokens in order (n_rows == T,
 *   sorted_token ignored) -- the shared expert.
 * act_fmt: MOE_ACT_BF16, or MOE_ACT_MXFP8 (see above; MOE_EUNSUPPORTED
 *   unless every projection is MXFP4 and H, I are multiples of 512).
 * y_rows: fp32 [n_rows][H] out.
 * Accumulation is fp32.  Small buckets (decode) run dequant-fused GEMVs;
 * large ones a grouped GEMM on matrix cores; MOE_ACT_MXFP8 always the
 * FP4 matrix instructions. */
size_t moe_expert_ffn_workspace(int T, int n_rows, int E, int H, int I, int fmt_gate,
                                int fmt_down, int act_fmt);
/* Where a MOE_ACT_MXFP8 call of moe_expert_ffn with these sizes leaves the
 * quantized SwiGLU output in its workspace: byte offsets of the E4M3 codes
 * uint8 [n_rows][I] and of their E8M0 scales uint8 [n_rows][I/32] (bucket
 * order), and, with MOE_ACT_TRACE, of the fp32 values they were quantized
 * from, fp32 [n_rows][I]; valid until the workspace is reused.  For tests
 * that compare the MX-FP8 intermediate with a reference. */
int moe_expert_ffn_a8_layout(int T, int n_rows, int E, int H, int I, size_t *codes_off,
                             size_t *scales_off, size_t *f32_off);
int moe_expert_ffn(int T, int H, int I, const uint16_t *x, const moe_weights *gate,
                   const moe_weights *up, const moe_weights *down, int act_fmt,
                   const int32_t *expert_offsets, const int32_t *sorted_token, int n_rows,
                   float *y_rows, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* moe_combine: the gather form of the weighted scatter-add, then the
 * optional steering term:
 *   out[t][n] = shared_y[t][n] + sum_j topk_w[t][j] * y_rows[slot_pos[t*k+j]][n]
 *               + steer_alpha * steer_dir[n]
 * accumulated in fp64 in that order (each product is exact in fp64) and
 * rounded once to fp32.  The routed experts' weighted sum plus the
 * full-precision shared expert is the layer's output (dibi8.com ds4 guide,
 * "Cac Doi Moi Kien Truc Chinh" item 1).  The steering term is runtime
 * activation steering: a per-layer direction scaled by a strength chosen at
 * run time, added to the FFN output without touching the weights
 * (grapeot.me ds4 post, the activation-steering paragraphs on
 * --dir-steering-ffn); the library adds it to the whole MoE layer output.
 * shared_y: optional fp32 [T][H]; steer_dir: optional fp32 [H].
 * out_f32: fp32 [T][H] out; out_bf16: optional bf16 [T][H] copy (RNE). */
int moe_combine(int T, int H, int k, const float *y_rows, const int32_t *slot_pos,
                const float *topk_w, const float *shared_y, const float *steer_dir,
                float steer_alpha, float *out_f32, uint16_t *out_bf16, void *stream);

/* ---------------------------------------------------------------------- */
/* moe_forward: the whole layer, out = shared(x) + sum_j w_j FFN_{e_j}(x),
 * equal to moe_route -> moe_dispatch -> moe_expert_ffn (routed and shared)
 * -> moe_combine, fused where that pays (few tokens: four kernels with no
 * host round trip).
 * logits_in / token_ids: as in moe_route.  out_f32: fp32 [T][H];
 * out_bf16, topk_idx_out [T][k], topk_w_out [T][k]: optional outputs.
 * side: optional (NULL: everything on `stream`).  Above one token, when
 * given, the shared expert runs on side->stream, forked from `stream` by
 * side->fork before any other work and joined back by side->join before the
 * combine, so the call still orders after earlier work on `stream` and
 * before later work, and can be captured into a HIP graph from `stream`. */
size_t moe_forward_workspace(const moe_layer *layer, int T);
int moe_forward(const moe_layer *layer, int T, const uint16_t *x, const float *logits_in,
                const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                const moe_side_stream *side, void *stream);

/* moe_forward_static: moe_forward for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no ws argument and no allocation of any kind; the workspace
 * is a device array of MOE_STATIC_SCRATCH_BYTES inside the library, one per
 * GPU, held from the first call on that GPU until the process ends.  Layers
 * and token counts whose moe_forward_workspace exceeds it return
 * MOE_ENOSPC (64 MiB: up to 256 tokens of a 4096-hidden, 256-expert top-8
 * layer).  Everything runs on `stream` (no second stream).  Every call on a
 * GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 * Results are identical to moe_forward's. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_static(const moe_layer *layer, int T, const uint16_t *x, const float *logits_in,
                       const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                       int32_t *topk_idx_out, float *topk_w_out, void *stream);

/* ---------------------------------------------------------------------- */
/* A residency cache of routed experts in HBM for one-token decode, filled
 * from pinned host memory: the analogue of the pages' streaming of routed
 * experts from SSD when the model exceeds memory (hysenlabs.com ds4 page,
 * "SSD streaming"; baiwuji.top ds4 article, "Core features" item 2: the few
 * experts a generated token picks are read from the slower tier).
 *   - The layer passed to moe_forward_cached holds all E experts' gate, up
 *     and down in host memory from hipHostMalloc (mapped, so the device can
 *     read it); router and shared expert are in device memory as usual.
 *   - slot_gate/up/down: the same formats for n_slots experts in device
 *     memory: the slots.  n_slots >= k.  Every plane's bytes per expert must
 *     be a multiple of 16 (MOE_EUNSUPPORTED otherwise).
 *   - state: device int32 [moe_cache_state_ints(E, n_slots)], emptied by
 *     moe_cache_reset.  state[2] and state[3] count hits and misses so far;
 *     state[4 + e] is the slot holding expert e, or -1.
 * Each step the device itself selects the k experts (as moe_route does),
 * looks them up, gives each miss the least recently used slot that no
 * expert of this step holds (lowest slot on ties), copies the missed
 * experts' bytes from host memory into their slots, then runs the routed
 * FFN on the slots -- no host round trip, so the call can be captured in a
 * HIP graph.  Results are identical to moe_forward's.  T must be 1 and the
 * layer one that moe_forward runs in its one-token launches
 * (MOE_EUNSUPPORTED otherwise). */
typedef struct {
  int32_t n_slots;
  moe_weights slot_gate, slot_up, slot_down;
  int32_t *state;
} moe_expert_cache;
size_t moe_cache_state_ints(int E, int n_slots);
int moe_cache_reset(const moe_expert_cache *cache, int E, void *stream);
int moe_forward_cached(const moe_layer *layer, const moe_expert_cache *cache, int T,
                       const uint16_t *x, const float *logits_in, const int64_t *token_ids,
                       float *out_f32, uint16_t *out_bf16, int32_t *topk_idx_out,
                       float *topk_w_out, void *ws, size_t ws_bytes, void *stream);

/* moe_forward_marked: moe_forward for measurement tools.  Each kernel the
 * call enqueues (up to max_marks of them) is launched so that it records the
 * caller's events marks[i].start and marks[i].stop (hipEvent_t passed as
 * void*) when it begins and ends on `stream` (HIP's extended launch), and
 * marks[i].name is set to a static string naming that kernel.  *n_marks gets
 * the number of kernels so timed.  Results are identical to moe_forward.
 * Every kernel runs on `stream` (no second stream), so that the timed
 * kernels do not overlap.  Every event must be non-null (MOE_EINVAL
 * otherwise). */
typedef struct {
  void *start;
  void *stop;
  const char *name;
} moe_mark;
int moe_forward_marked(const moe_layer *layer, int T, const uint16_t *x, const float *logits_in,
                       const int64_t *token_ids, float *out_f32, uint16_t *out_bf16,
                       int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                       moe_mark *marks, int max_marks, int *n_marks, void *stream);

/* ---------------------------------------------------------------------- */
/* moe_mxfp8_quantize: the MOE_ACT_MXFP8 quantization of bf16 rows, as the
 * A8 path applies it to the tokens.  x: bf16 [rows][K]; q: E4M3 codes
 * uint8 [rows][K] out; scales: E8M0 uint8 [rows][K/32] out.  K % 32 == 0. */
int moe_mxfp8_quantize(int rows, int K, const uint16_t *x, uint8_t *q, uint8_t *scales,
                       void *stream);

/* moe_dequantize: weights [w0, w0+count) of expert `expert`'s row-major
 * flattened matrix, decoded to fp32 with the same device decoders the FFN
 * kernels use.  out: fp32 [count]. */
int moe_dequantize(const moe_weights *w, int expert, int64_t w0, int64_t count, float *out,
                   void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_MOE_H */
