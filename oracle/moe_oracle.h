/*
 * moe_oracle.h -- CPU reference ("oracle") for the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU library
 * shares no code with it: no headers, no kernels, no tables, no helpers.
 *
 * Plain, slow and obviously correct: every weight is decoded from its
 * definition into fp32, every dot product is accumulated in fp64 in index
 * order, results are rounded once to fp32.
 *
 * Sources (the ds4 / DwarfStar 4 pages):
 *  - "DS4 (DwarfStar 4): Chay DeepSeek V4 Flash Local voi Metal & CUDA"
 *    (dibi8.com), section "Cac Doi Moi Kien Truc Chinh", item 1: only the
 *    routed experts are quantized to 2 bits -- an IQ2_XXS-class format for
 *    up/gate and Q2_K for down -- while the shared expert, projections and
 *    routing layers stay at full precision.
 *  - "DwarfStar: a focused local inference engine for DeepSeek V4 and GLM 5.2"
 *    (hysenlabs.com), section "Model support and quantization": the same
 *    split, plus an MXFP4 variant keeping the released FP4 routed experts.
 *  - The grapeot.me ds4 blog post, opening paragraphs: V4 Flash uses hash MoE
 *    routing and FP4+FP8 mixed-precision weights.
 * The pages name the formats but do not define their bits; the exact field
 * layouts implemented here are this project's readings, stated per function.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FMT_BF16 = 0, ORC_FMT_Q2K = 1, ORC_FMT_VQ2 = 2, ORC_FMT_MXFP4 = 3 };
enum { ORC_ROUTE_SOFTMAX_TOPK = 0, ORC_ROUTE_HASH = 1 };

/* one projection of E experts, each [N rows, K cols], expert-major */
typedef struct {
  int32_t fmt, E, N, K;
  const void *data;       /* bf16 bits | Q2K blocks | VQ2 codes | MXFP4 nibbles */
  const void *scales;     /* VQ2: fp16 [E][N][K/256]; MXFP4: E8M0 [E][N][K/32] */
  const int8_t *codebook; /* VQ2: int8 [256][4] */
} orc_proj;

typedef struct {
  int32_t H, I, E, k, I_shared, route_mode;
  const uint16_t *w_router;    /* bf16 [E][H] */
  orc_proj gate, up, down;     /* [E][I][H], [E][I][H], [E][H][I] */
  const uint16_t *sh_gate, *sh_up, *sh_down; /* bf16 [Is][H], [Is][H], [H][Is]; NULL if none */
  const float *steer_dir;      /* optional fp32 [H]: activation steering direction */
  float steer_alpha;           /* its strength */
} orc_layer;

/* scalar decodes */
float orc_bf16(uint16_t b);
float orc_f16(uint16_t h);
float orc_e2m1(unsigned nibble);
double orc_e8m0(unsigned e);
float orc_e4m3(unsigned code);
uint8_t orc_to_e4m3(double v);
uint64_t orc_splitmix64(uint64_t x);

/* weights [n0, n0+count) of expert e's row-major flattened matrix -> fp32 */
int orc_dequant(const orc_proj *p, int e, int64_t n0, int64_t count, float *out);

/* routing */
void orc_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *w_router,
                       float *logits);
void orc_select_topk(int T, int E, int k, const float *logits, int32_t *idx, float *w);
void orc_select_hash(int T, int E, int k, const int64_t *token_ids, const float *logits,
                     int32_t *idx, float *w);
int orc_route(int mode, int T, int H, int E, int k, const uint16_t *x, const uint16_t *w_router,
              const float *logits_in, const int64_t *token_ids, int32_t *idx, float *w,
              float *logits_out);

/* dispatch: counting sort of the T*k slots by expert, stable in slot order */
void orc_dispatch(int T, int E, int k, const int32_t *idx, int32_t *offsets,
                  int32_t *sorted_token, int32_t *sorted_slot, int32_t *slot_pos);

/* expert FFN over bucketed rows: y_rows[r] = FFN_{e(r)}(x[sorted_token[r]]) */
int orc_expert_ffn(const orc_layer *L, int T, const uint16_t *x, const int32_t *offsets,
                   const int32_t *sorted_token, float *y_rows);
/* shared expert on all T tokens: y[t] = FFN_shared(x[t]) */
int orc_shared_ffn(const orc_layer *L, int T, const uint16_t *x, float *y);
/* combine: out[t] = shared[t] + sum_j w[t,j] * y_rows[slot_pos[t*k+j]]
 *                  + steer_alpha * steer_dir (steer_dir optional) */
void orc_combine(int T, int H, int k, const float *y_rows, const int32_t *slot_pos,
                 const float *w, const float *shared_y, const float *steer_dir,
                 float steer_alpha, float *out);

/* whole layer (route -> dispatch -> expert FFN -> shared -> combine), fp64 inside */
int orc_forward(const orc_layer *L, int T, const uint16_t *x, const float *logits_in,
                const int64_t *token_ids, float *out, int32_t *idx, float *w);
/* brute force: out[t] = shared(x_t) + sum_e G[t,e] FFN_e(x_t) with a dense gate
 * G built from (idx, w); no dispatch, every expert evaluated on every token */
int orc_dense_masked(const orc_layer *L, int T, const uint16_t *x, const int32_t *idx,
                     const float *w, float *out);

/* MX-FP8 (E4M3, E8M0 per 32) quantization of a [rows, K] fp32 matrix */
void orc_mxfp8_quant(int rows, int K, const float *in, uint8_t *codes, uint8_t *scales);
/* the same layer with activations entering each MXFP4 projection quantized
 * to MX-FP8 first (x before gate/up, the SwiGLU output before down) */
int orc_forward_a8(const orc_layer *L, int T, const uint16_t *x, const float *logits_in,
                   const int64_t *token_ids, float *out, int32_t *idx, float *w);

/* its two stages over bucket rows (offsets/sorted_token as for
 * orc_expert_ffn; I % 32 == 0): the MX-FP8 codes [n_rows][I] and E8M0
 * scales [n_rows][I/32] of each row's SwiGLU output, and the down projection
 * of given codes, y_rows [n_rows][H] */
int orc_a8_swiglu_codes(const orc_layer *L, int T, const uint16_t *x, const int32_t *offsets,
                        const int32_t *sorted_token, uint8_t *codes, uint8_t *scales);
int orc_a8_down(const orc_layer *L, const int32_t *offsets, const uint8_t *codes,
                const uint8_t *scales, float *y_rows);

int orc_threads(void);
void orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
