/*
 * moe_oracle.c -- CPU reference for the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).  Plain C99 with optional
 * OpenMP over independent output rows; each output value is still computed
 * by one thread in index order, so results do not depend on the thread count.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* threads of the parallel loops from now on (n >= 1); the results do not
 * depend on it */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* scalar decodes                                                             */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32 */
float orc_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
float orc_f16(uint16_t h) {
  unsigned s = h >> 15, e = (h >> 10) & 31u, m = h & 1023u;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m/1024 * 2^-14 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024u + m), (int)e - 25); /* (1 + m/1024) * 2^(e-15) */
  return (float)(s ? -v : v);
}

/* OCP MX v1.0 FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
 * exponent 0 is subnormal (0 or 0.5).  Magnitudes 0,.5,1,1.5,2,3,4,6. */
float orc_e2m1(unsigned nib) {
  unsigned s = (nib >> 3) & 1u, e = (nib >> 1) & 3u, m = nib & 1u;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return (float)(s ? -v : v);
}

/* OCP MX v1.0 E8M0 shared scale: 2^(e-127); 0xFF is NaN */
double orc_e8m0(unsigned e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* OCP FP8 E4M3 (the "FN" variant of the MX spec): 1 sign, 4 exponent
 * (bias 7), 3 mantissa; exponent 0 subnormal; S.1111.111 is NaN; no inf. */
float orc_e4m3(unsigned c) {
  unsigned s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^-6 */
  else
    v = ldexp(8.0 + m, (int)e - 10); /* (1 + m/8) * 2^(e-7) */
  return (float)(s ? -v : v);
}

/* Nearest E4M3 code to v (ties to the code with an even mantissa),
 * saturating at +-448.  Brute force over all finite codes. */
uint8_t orc_to_e4m3(double v) {
  unsigned sign = (v < 0 || (v == 0 && signbit(v))) ? 0x80u : 0u;
  double a = fabs(v);
  unsigned best = 0;
  double best_err = INFINITY;
  for (unsigned c = 0; c <= 0x7E; c++) {
    double err = fabs((double)orc_e4m3(c) - a);
    if (err < best_err || (err == best_err && (c & 1u) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; finaliser Mix13 of
 * Stafford): advance the state by the golden-gamma increment, then mix.
 * splitmix64(x) is the first output of a generator seeded with x. */
uint64_t orc_splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------------ */
/* weight formats                                                             */
/* ------------------------------------------------------------------------ */

/*
 * Q2_K-style super-block (down projection, 2-bit; dibi8 ds4 page "Key
 * innovations" item 1 and hysenlabs page "Model support and quantization"
 * name the format; the bit layout is this project's reading): 256 weights in
 * 16 sub-blocks of 16, 84 bytes
 *     uint8 sc[16]   low nibble: 4-bit scale of sub-block s, high: 4-bit min
 *     uint8 qs[64]   weight i: (qs[i/4] >> 2*(i%4)) & 3
 *     fp16  d, dmin  (little-endian)
 *   w_i = (d * scale_s) * q_i - dmin * min_s,   s = i / 16.
 * The matrix is its row-major flattened sequence cut into 256-weight blocks.
 */
static float q2k_weight(const uint8_t *blk, unsigned i) {
  unsigned s = i / 16u;
  unsigned sc = blk[s] & 15u, mn = blk[s] >> 4;
  unsigned q = (blk[16 + i / 4u] >> (2u * (i % 4u))) & 3u;
  float d = orc_f16(rd16(blk + 80)), dmin = orc_f16(rd16(blk + 82));
  float scale = d * (float)sc;  /* exact: 11 x 4 significant bits */
  float hi = scale * (float)q;  /* exact: <= 17 bits */
  float lo = dmin * (float)mn;  /* exact: <= 15 bits */
  return hi - lo;               /* the only rounding */
}

/*
 * VQ2: the 2.06-bit codebook format standing for the IQ2_XXS-class up/gate
 * format the pages name.  One 8-bit index per 4 consecutive weights into a
 * 256-entry table of int8 4-vectors, plus an fp16 scale per 256 weights:
 *     w[n][k] = d[n][k/256] * cb[idx[n][k/4]][k%4].
 * Codes and scales are separate planes ([E][N][K/4] and [E][N][K/256]).
 */
static float vq2_weight(const orc_proj *p, int e, int64_t f) {
  const uint8_t *idx = (const uint8_t *)p->data;
  const uint16_t *d = (const uint16_t *)p->scales;
  int64_t per = (int64_t)p->N * p->K;
  int64_t n = f / p->K, k = f % p->K;
  unsigned code = idx[(int64_t)e * (per / 4) + n * (p->K / 4) + k / 4];
  float scale = orc_f16(d[(int64_t)e * (per / 256) + n * (p->K / 256) + k / 256]);
  return scale * (float)p->codebook[code * 4 + (unsigned)(k % 4)];
}

/*
 * MXFP4 (OCP MX v1.0): E2M1 elements sharing an E8M0 scale per 32
 * consecutive weights along K:  w = E2M1(nibble) * 2^(e - 127).
 * Values plane [E][N][K/2] (even k in the low nibble), scales [E][N][K/32].
 */
static float mxfp4_weight(const orc_proj *p, int e, int64_t f) {
  const uint8_t *v = (const uint8_t *)p->data;
  const uint8_t *s = (const uint8_t *)p->scales;
  int64_t per = (int64_t)p->N * p->K;
  uint8_t byte = v[(int64_t)e * (per / 2) + f / 2];
  unsigned nib = (f % 2) ? (byte >> 4) : (byte & 15u);
  int64_t n = f / p->K, k = f % p->K;
  double w = (double)orc_e2m1(nib) * orc_e8m0(s[(int64_t)e * (per / 32) + n * (p->K / 32) + k / 32]);
  return (float)w; /* exact: a 2-bit significand times a power of two */
}

int orc_dequant(const orc_proj *p, int e, int64_t n0, int64_t count, float *out) {
  int64_t per = (int64_t)p->N * p->K;
  if (e < 0 || e >= p->E || n0 < 0 || count < 0 || n0 + count > per) return -1;
  switch (p->fmt) {
    case ORC_FMT_BF16: {
      const uint16_t *w = (const uint16_t *)p->data + (int64_t)e * per;
      for (int64_t f = 0; f < count; f++) out[f] = orc_bf16(w[n0 + f]);
      return 0;
    }
    case ORC_FMT_Q2K: {
      if (per % 256) return -1;
      const uint8_t *base = (const uint8_t *)p->data + (int64_t)e * (per / 256) * 84;
#pragma omp parallel for schedule(static)
      for (int64_t f = 0; f < count; f++) {
        int64_t g = n0 + f;
        out[f] = q2k_weight(base + (g / 256) * 84, (unsigned)(g % 256));
      }
      return 0;
    }
    case ORC_FMT_VQ2:
      if (p->K % 256 || !p->codebook) return -1;
#pragma omp parallel for schedule(static)
      for (int64_t f = 0; f < count; f++) out[f] = vq2_weight(p, e, n0 + f);
      return 0;
    case ORC_FMT_MXFP4:
      if (p->K % 32) return -1;
#pragma omp parallel for schedule(static)
      for (int64_t f = 0; f < count; f++) out[f] = mxfp4_weight(p, e, n0 + f);
      return 0;
    default:
      return -1;
  }
}

static float *dequant_all(const orc_proj *p, int e) {
  int64_t per = (int64_t)p->N * p->K;
  float *w = (float *)malloc((size_t)per * sizeof(float));
  if (w && orc_dequant(p, e, 0, per, w) != 0) {
    free(w);
    return NULL;
  }
  return w;
}

/* ------------------------------------------------------------------------ */
/* routing                                                                    */
/* ------------------------------------------------------------------------ */

/* Router logits, kept at full precision (both ds4 pages on quantization):
 * logits[t][e] = sum_h x[t][h] * Wr[e][h].  Each bf16 product is exact in
 * double; the sum runs in h order in fp64 and is rounded once to fp32. */
void orc_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *wr, float *logits) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) {
      double acc = 0.0;
      for (int h = 0; h < H; h++)
        acc += (double)orc_bf16(x[(int64_t)t * H + h]) * (double)orc_bf16(wr[(int64_t)e * H + h]);
      logits[(int64_t)t * E + e] = (float)acc;
    }
}

static double order_key(float l) { return isnan(l) ? -INFINITY : (double)l; }

/* softmax over the k selected logits: w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max).
 * Equal to the full softmax renormalised over the selection; sums to 1. */
static void softmax_selected(int k, const float *lsel, float *w) {
  double mx = -INFINITY, den = 0.0, ex[64];
  for (int j = 0; j < k; j++) mx = fmax(mx, order_key(lsel[j]));
  for (int j = 0; j < k; j++) {
    ex[j] = exp(order_key(lsel[j]) - mx);
    den += ex[j];
  }
  for (int j = 0; j < k; j++) w[j] = (float)(ex[j] / den);
}

/* Softmax top-k: the k largest logits in descending order, equal logits
 * going to the lower expert index (NaN ranks as -inf). */
void orc_select_topk(int T, int E, int k, const float *logits, int32_t *idx, float *w) {
  char *taken = (char *)malloc((size_t)E);
  float lsel[64];
  for (int t = 0; t < T; t++) {
    const float *l = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || order_key(l[e]) > order_key(l[best])) best = e;
      }
      taken[best] = 1;
      idx[(int64_t)t * k + j] = best;
      lsel[j] = l[best];
    }
    softmax_selected(k, lsel, w + (int64_t)t * k);
  }
  free(taken);
}

/* Hash routing (the grapeot.me blog lists hash MoE routing among V4 Flash's
 * new features; the formula is this project's reading):
 *   idx[t][j] = ((splitmix64(token_id[t]) + j) mod 2^64) mod E,  j = 0..k-1,
 * weights = softmax of the router logits over those k experts. */
void orc_select_hash(int T, int E, int k, const int64_t *tid, const float *logits, int32_t *idx,
                     float *w) {
  float lsel[64];
  for (int t = 0; t < T; t++) {
    uint64_t z = orc_splitmix64((uint64_t)tid[t]);
    for (int j = 0; j < k; j++) {
      int e = (int)((z + (uint64_t)j) % (uint64_t)E);
      idx[(int64_t)t * k + j] = e;
      lsel[j] = logits[(int64_t)t * E + e];
    }
    softmax_selected(k, lsel, w + (int64_t)t * k);
  }
}

int orc_route(int mode, int T, int H, int E, int k, const uint16_t *x, const uint16_t *wr,
              const float *logits_in, const int64_t *tid, int32_t *idx, float *w,
              float *logits_out) {
  if (T < 0 || E < 1 || k < 1 || k > E || k > 64) return -1;
  if (mode == ORC_ROUTE_HASH && !tid) return -1;
  float *l = logits_out ? logits_out : (float *)malloc((size_t)T * E * sizeof(float) + 1);
  if (logits_in)
    memcpy(l, logits_in, (size_t)T * E * sizeof(float));
  else
    orc_router_logits(T, H, E, x, wr, l);
  if (mode == ORC_ROUTE_HASH)
    orc_select_hash(T, E, k, tid, l, idx, w);
  else
    orc_select_topk(T, E, k, l, idx, w);
  if (!logits_out) free(l);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* dispatch                                                                   */
/* ------------------------------------------------------------------------ */

/* Bucket the T*k (token, choice) slots by expert: counts, exclusive prefix
 * sum (offsets[E] = T*k), and each bucket listing its slots f = t*k + j in
 * ascending f.  slot_pos is the inverse map. */
void orc_dispatch(int T, int E, int k, const int32_t *idx, int32_t *offsets, int32_t *sorted_token,
                  int32_t *sorted_slot, int32_t *slot_pos) {
  int64_t n = (int64_t)T * k;
  for (int e = 0; e <= E; e++) offsets[e] = 0;
  for (int64_t f = 0; f < n; f++) offsets[idx[f] + 1]++;
  for (int e = 0; e < E; e++) offsets[e + 1] += offsets[e];
  int32_t *fill = (int32_t *)malloc((size_t)E * sizeof(int32_t) + 1);
  for (int e = 0; e < E; e++) fill[e] = offsets[e];
  for (int64_t f = 0; f < n; f++) {
    int r = fill[idx[f]]++;
    sorted_token[r] = (int32_t)(f / k);
    sorted_slot[r] = (int32_t)f;
    slot_pos[f] = r;
  }
  free(fill);
}

/* ------------------------------------------------------------------------ */
/* expert FFN                                                                 */
/* ------------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert: g = Wg x, u = Wu x, a = silu(g) * u, y = Wd a,
 * with Wg, Wu [I][H] and Wd [H][I]; fp64 accumulation in index order. */
static void swiglu(int H, int I, const double *x, const float *Wg, const float *Wu,
                   const float *Wd, double *a, double *y) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < I; i++) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; h++) {
      g += x[h] * (double)Wg[(int64_t)i * H + h];
      u += x[h] * (double)Wu[(int64_t)i * H + h];
    }
    a[i] = silu(g) * u;
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < H; n++) {
    double acc = 0.0;
    for (int i = 0; i < I; i++) acc += a[i] * (double)Wd[(int64_t)n * I + i];
    y[n] = acc;
  }
}

/* The A8 variant in its two stages: gate/up on the MX-FP8 projection of x,
 * whose SwiGLU output is itself quantized to MX-FP8 (codes + E8M0 scales),
 * then down on the decoded codes.  Each MX-FP8 rounding is the OCP MX v1.0
 * rule of mx8_group below. */
static unsigned mx8_group(const double *v, int n, uint8_t *codes);
static void mx8_round(int K, double *v);

static void a8_gateup(int H, int I, const double *x, const float *Wg, const float *Wu,
                      double *a, uint8_t *codes, uint8_t *scales) {
  double *xq = (double *)malloc((size_t)H * sizeof(double));
  memcpy(xq, x, (size_t)H * sizeof(double));
  mx8_round(H, xq);
#pragma omp parallel for schedule(static)
  for (int i = 0; i < I; i++) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; h++) {
      g += xq[h] * (double)Wg[(int64_t)i * H + h];
      u += xq[h] * (double)Wu[(int64_t)i * H + h];
    }
    a[i] = silu(g) * u;
  }
  for (int g = 0; g < I; g += 32)
    scales[g / 32] = (uint8_t)mx8_group(a + g, (I - g) < 32 ? (I - g) : 32, codes + g);
  free(xq);
}

/* a = E4M3(codes) * 2^(scale - 127), per 32 along I */
static void mx8_decode(int I, const uint8_t *codes, const uint8_t *scales, double *a) {
  for (int i = 0; i < I; i++) a[i] = (double)orc_e4m3(codes[i]) * orc_e8m0(scales[i / 32]);
}

static void down_d(int H, int I, const double *a, const float *Wd, double *y) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < H; n++) {
    double acc = 0.0;
    for (int i = 0; i < I; i++) acc += a[i] * (double)Wd[(int64_t)n * I + i];
    y[n] = acc;
  }
}

/* the SwiGLU expert with the activations entering each projection passed
 * through MX-FP8 quantization */
static void swiglu_a8(int H, int I, const double *x, const float *Wg, const float *Wu,
                      const float *Wd, double *a, double *y) {
  uint8_t *codes = (uint8_t *)malloc((size_t)I + 32);
  uint8_t *scales = (uint8_t *)malloc((size_t)I / 32 + 2);
  a8_gateup(H, I, x, Wg, Wu, a, codes, scales);
  mx8_decode(I, codes, scales, a);
  down_d(H, I, a, Wd, y);
  free(codes), free(scales);
}

typedef struct {
  float *g, *u, *d;
} expert_w;

static int load_expert(const orc_layer *L, int e, expert_w *w) {
  w->g = dequant_all(&L->gate, e);
  w->u = dequant_all(&L->up, e);
  w->d = dequant_all(&L->down, e);
  if (!w->g || !w->u || !w->d) {
    free(w->g), free(w->u), free(w->d);
    return -1;
  }
  return 0;
}

static void free_expert(expert_w *w) { free(w->g), free(w->u), free(w->d); }

static int check_layer(const orc_layer *L) {
  if (L->H < 1 || L->I < 1 || L->E < 1 || L->k < 1 || L->k > L->E || L->k > 64) return -1;
  if (L->gate.N != L->I || L->gate.K != L->H || L->up.N != L->I || L->up.K != L->H) return -1;
  if (L->down.N != L->H || L->down.K != L->I) return -1;
  if (L->gate.E != L->E || L->up.E != L->E || L->down.E != L->E) return -1;
  return 0;
}

static void token_x(int H, const uint16_t *x, int t, double *xd) {
  for (int h = 0; h < H; h++) xd[h] = (double)orc_bf16(x[(int64_t)t * H + h]);
}

/* y_rows (double) for every bucket row; shared core of the bucketed paths */
static int expert_rows_d(const orc_layer *L, int T, const uint16_t *x, const int32_t *offsets,
                         const int32_t *sorted_token, double *y, int a8) {
  int H = L->H, I = L->I;
  double *xd = (double *)malloc((size_t)H * sizeof(double));
  double *a = (double *)malloc((size_t)I * sizeof(double));
  int rc = 0;
  (void)T;
  for (int e = 0; e < L->E && rc == 0; e++) {
    if (offsets[e + 1] == offsets[e]) continue;
    expert_w w;
    if (load_expert(L, e, &w)) {
      rc = -1;
      break;
    }
    for (int r = offsets[e]; r < offsets[e + 1]; r++) {
      token_x(H, x, sorted_token[r], xd);
      if (a8)
        swiglu_a8(H, I, xd, w.g, w.u, w.d, a, y + (int64_t)r * H);
      else
        swiglu(H, I, xd, w.g, w.u, w.d, a, y + (int64_t)r * H);
    }
    free_expert(&w);
  }
  free(xd), free(a);
  return rc;
}

int orc_expert_ffn(const orc_layer *L, int T, const uint16_t *x, const int32_t *offsets,
                   const int32_t *sorted_token, float *y_rows) {
  if (check_layer(L)) return -1;
  int64_t rows = offsets[L->E];
  double *y = (double *)malloc((size_t)(rows ? rows : 1) * L->H * sizeof(double));
  int rc = expert_rows_d(L, T, x, offsets, sorted_token, y, 0);
  for (int64_t i = 0; i < rows * L->H; i++) y_rows[i] = (float)y[i];
  free(y);
  return rc;
}

/* The A8 variant's intermediate: for every bucket row r, the MX-FP8 codes
 * [I] and E8M0 scales [I/32] of the SwiGLU output of its expert on the
 * MX-FP8 projection of its token (the first stage of swiglu_a8). */
int orc_a8_swiglu_codes(const orc_layer *L, int T, const uint16_t *x, const int32_t *offsets,
                        const int32_t *sorted_token, uint8_t *codes, uint8_t *scales) {
  if (check_layer(L) || L->I % 32) return -1;
  int H = L->H, I = L->I;
  double *xd = (double *)malloc((size_t)H * sizeof(double));
  double *a = (double *)malloc((size_t)I * sizeof(double));
  int rc = 0;
  (void)T;
  for (int e = 0; e < L->E && rc == 0; e++) {
    if (offsets[e + 1] == offsets[e]) continue;
    expert_w w;
    if (load_expert(L, e, &w)) {
      rc = -1;
      break;
    }
    for (int r = offsets[e]; r < offsets[e + 1]; r++) {
      token_x(H, x, sorted_token[r], xd);
      a8_gateup(H, I, xd, w.g, w.u, a, codes + (int64_t)r * I, scales + (int64_t)r * (I / 32));
    }
    free_expert(&w);
  }
  free(xd), free(a);
  return rc;
}

/* The A8 variant's second stage on given codes: y_rows[r] = Wd_e a_r with
 * a_r decoded from codes[r], scales[r] (fp64 accumulation, rounded once). */
int orc_a8_down(const orc_layer *L, const int32_t *offsets, const uint8_t *codes,
                const uint8_t *scales, float *y_rows) {
  if (check_layer(L) || L->I % 32) return -1;
  int H = L->H, I = L->I;
  double *a = (double *)malloc((size_t)I * sizeof(double));
  double *y = (double *)malloc((size_t)H * sizeof(double));
  int rc = 0;
  for (int e = 0; e < L->E && rc == 0; e++) {
    if (offsets[e + 1] == offsets[e]) continue;
    float *wd = dequant_all(&L->down, e);
    if (!wd) {
      rc = -1;
      break;
    }
    for (int r = offsets[e]; r < offsets[e + 1]; r++) {
      mx8_decode(I, codes + (int64_t)r * I, scales + (int64_t)r * (I / 32), a);
      down_d(H, I, a, wd, y);
      for (int n = 0; n < H; n++) y_rows[(int64_t)r * H + n] = (float)y[n];
    }
    free(wd);
  }
  free(a), free(y);
  return rc;
}

static int shared_d(const orc_layer *L, int T, const uint16_t *x, double *y) {
  int H = L->H, Is = L->I_shared;
  if (!L->sh_gate || Is < 1) {
    memset(y, 0, (size_t)T * H * sizeof(double));
    return 0;
  }
  orc_proj pg = {ORC_FMT_BF16, 1, Is, H, L->sh_gate, NULL, NULL};
  orc_proj pu = {ORC_FMT_BF16, 1, Is, H, L->sh_up, NULL, NULL};
  orc_proj pd = {ORC_FMT_BF16, 1, H, Is, L->sh_down, NULL, NULL};
  expert_w w = {dequant_all(&pg, 0), dequant_all(&pu, 0), dequant_all(&pd, 0)};
  double *xd = (double *)malloc((size_t)H * sizeof(double));
  double *a = (double *)malloc((size_t)Is * sizeof(double));
  for (int t = 0; t < T; t++) {
    token_x(H, x, t, xd);
    swiglu(H, Is, xd, w.g, w.u, w.d, a, y + (int64_t)t * H);
  }
  free(xd), free(a);
  free_expert(&w);
  return 0;
}

int orc_shared_ffn(const orc_layer *L, int T, const uint16_t *x, float *y) {
  double *yd = (double *)malloc((size_t)T * L->H * sizeof(double) + 8);
  int rc = shared_d(L, T, x, yd);
  for (int64_t i = 0; i < (int64_t)T * L->H; i++) y[i] = (float)yd[i];
  free(yd);
  return rc;
}

/* Activation steering (grapeot.me ds4 post, the paragraphs on
 * --dir-steering-ffn): at run time a per-layer direction, scaled by a chosen
 * strength, is added to the FFN's output; the weights are untouched.
 * Reading: it is added to the whole MoE layer output, after the routed sum. */
static double steer_term(const float *dir, float alpha, int n) {
  return dir ? (double)alpha * (double)dir[n] : 0.0;
}

/* out[t][n] = shared[t][n] + sum_j w[t][j] * y_rows[slot_pos[t*k + j]][n]
 *             + alpha * dir[n],
 * the sum taken in that order (j ascending) in fp64, stored as fp32 */
void orc_combine(int T, int H, int k, const float *y_rows, const int32_t *slot_pos, const float *w,
                 const float *shared_y, const float *steer_dir, float steer_alpha, float *out) {
  for (int t = 0; t < T; t++)
    for (int n = 0; n < H; n++) {
      double acc = shared_y ? (double)shared_y[(int64_t)t * H + n] : 0.0;
      for (int j = 0; j < k; j++)
        acc += (double)w[(int64_t)t * k + j] *
               (double)y_rows[(int64_t)slot_pos[(int64_t)t * k + j] * H + n];
      if (steer_dir) acc += steer_term(steer_dir, steer_alpha, n);
      out[(int64_t)t * H + n] = (float)acc;
    }
}

static int forward_impl(const orc_layer *L, int T, const uint16_t *x, const float *logits_in,
                        const int64_t *tid, float *out, int32_t *idx, float *w, int a8) {
  if (check_layer(L) || T < 0) return -1;
  if (T == 0) return 0;
  int H = L->H, E = L->E, k = L->k;
  int64_t n = (int64_t)T * k;
  if (orc_route(L->route_mode, T, H, E, k, x, L->w_router, logits_in, tid, idx, w, NULL))
    return -1;
  int32_t *off = (int32_t *)malloc((size_t)(E + 1) * sizeof(int32_t));
  int32_t *st = (int32_t *)malloc((size_t)n * sizeof(int32_t));
  int32_t *ss = (int32_t *)malloc((size_t)n * sizeof(int32_t));
  int32_t *sp = (int32_t *)malloc((size_t)n * sizeof(int32_t));
  double *y = (double *)malloc((size_t)n * H * sizeof(double));
  double *sh = (double *)malloc((size_t)T * H * sizeof(double));
  orc_dispatch(T, E, k, idx, off, st, ss, sp);
  int rc = expert_rows_d(L, T, x, off, st, y, a8);
  if (rc == 0) rc = shared_d(L, T, x, sh);
  if (rc == 0)
    for (int t = 0; t < T; t++)
      for (int h = 0; h < H; h++) {
        double acc = sh[(int64_t)t * H + h];
        for (int j = 0; j < k; j++)
          acc += (double)w[(int64_t)t * k + j] * y[(int64_t)sp[(int64_t)t * k + j] * H + h];
        if (L->steer_dir) acc += steer_term(L->steer_dir, L->steer_alpha, h);
        out[(int64_t)t * H + h] = (float)acc;
      }
  free(off), free(st), free(ss), free(sp), free(y), free(sh);
  return rc;
}

int orc_forward(const orc_layer *L, int T, const uint16_t *x, const float *logits_in,
                const int64_t *tid, float *out, int32_t *idx, float *w) {
  return forward_impl(L, T, x, logits_in, tid, out, idx, w, 0);
}

int orc_forward_a8(const orc_layer *L, int T, const uint16_t *x, const float *logits_in,
                   const int64_t *tid, float *out, int32_t *idx, float *w) {
  return forward_impl(L, T, x, logits_in, tid, out, idx, w, 1);
}

int orc_dense_masked(const orc_layer *L, int T, const uint16_t *x, const int32_t *idx,
                     const float *w, float *out) {
  if (check_layer(L)) return -1;
  int H = L->H, I = L->I, E = L->E, k = L->k;
  double *sh = (double *)malloc((size_t)T * H * sizeof(double) + 8);
  double *acc = (double *)calloc((size_t)T * H + 1, sizeof(double));
  double *xd = (double *)malloc((size_t)H * sizeof(double));
  double *a = (double *)malloc((size_t)I * sizeof(double));
  double *y = (double *)malloc((size_t)H * sizeof(double));
  int rc = shared_d(L, T, x, sh);
  for (int e = 0; e < E && rc == 0; e++) {
    expert_w ew;
    if (load_expert(L, e, &ew)) {
      rc = -1;
      break;
    }
    for (int t = 0; t < T; t++) {
      double gate = 0.0; /* dense gate G[t][e]: the weight where e was chosen, else 0 */
      for (int j = 0; j < k; j++)
        if (idx[(int64_t)t * k + j] == e) gate += (double)w[(int64_t)t * k + j];
      token_x(H, x, t, xd);
      swiglu(H, I, xd, ew.g, ew.u, ew.d, a, y);
      for (int h = 0; h < H; h++) acc[(int64_t)t * H + h] += gate * y[h];
    }
    free_expert(&ew);
  }
  if (rc == 0)
    for (int64_t i = 0; i < (int64_t)T * H; i++)
      out[i] = (float)(sh[i] + acc[i] + steer_term(L->steer_dir, L->steer_alpha, (int)(i % H)));
  free(sh), free(acc), free(xd), free(a), free(y);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* MX-FP8 activations (A8 variant)                                            */
/* ------------------------------------------------------------------------ */

/*
 * OCP MX v1.0 quantization of one 32-element group to E4M3 with an E8M0
 * scale: X = 2^(floor(log2(amax)) - 8) (8 = largest E4M3 exponent),
 * element = nearest E4M3 of v / X (ties to even, saturating at 448).
 * amax == 0 gives scale byte 0 and zero codes.  Scale byte = clamp(log2 X
 * + 127, 0, 254).
 */
static unsigned mx8_group(const double *v, int n, uint8_t *codes) {
  double amax = 0.0;
  for (int i = 0; i < n; i++) amax = fmax(amax, fabs(v[i]));
  if (amax == 0.0) {
    for (int i = 0; i < n; i++) codes[i] = 0;
    return 0;
  }
  int ex;
  frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
  int s = (ex - 1) - 8;
  int e8 = s + 127;
  if (e8 < 0) e8 = 0;
  if (e8 > 254) e8 = 254;
  double X = ldexp(1.0, e8 - 127);
  for (int i = 0; i < n; i++) codes[i] = orc_to_e4m3(v[i] / X);
  return (unsigned)e8;
}

static void mx8_round(int K, double *v) {
  uint8_t codes[32];
  for (int g = 0; g < K; g += 32) {
    int n = (K - g) < 32 ? (K - g) : 32;
    unsigned e8 = mx8_group(v + g, n, codes);
    double X = ldexp(1.0, (int)e8 - 127);
    for (int i = 0; i < n; i++) v[g + i] = (double)orc_e4m3(codes[i]) * X;
  }
}

void orc_mxfp8_quant(int rows, int K, const float *in, uint8_t *codes, uint8_t *scales) {
  double v[32];
  int G = (K + 31) / 32;
  for (int r = 0; r < rows; r++)
    for (int g = 0; g < G; g++) {
      int n = (K - g * 32) < 32 ? (K - g * 32) : 32;
      for (int i = 0; i < n; i++) v[i] = (double)in[(int64_t)r * K + g * 32 + i];
      scales[(int64_t)r * G + g] = (uint8_t)mx8_group(v, n, codes + (int64_t)r * K + g * 32);
    }
}
