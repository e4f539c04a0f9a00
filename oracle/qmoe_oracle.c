/*
 * CPU oracle for the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain reference that the GPU
 * library is checked against. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never links, calls or
 * includes anything from this directory, and this file includes nothing of the GPU
 * library.
 *
 * What it computes (sources: the Strata pages; items marked "workload definition"
 * are fixed by the workload description rather than by the pages):
 *   route    - per token, the k experts with the largest router logits, and routing
 *              weights over those k (Strata engine explainer, m.lqnn.cn/news/264700,
 *              sections "Architecture overview" and "Doorbell handshake": the router
 *              picks 10 of 512 experts per token and hands over expert ids together
 *              with routing weights);
 *   group    - token-expert pairs grouped by expert, as consumed by the grouped
 *              verify-window kernel (same page, section "Expert cache");
 *   quant    - int8 block-32 activation quantization, symmetric, round half to even
 *              (workload definition; the int8 activation dots of the same page's
 *              section "CPU expert pool");
 *   ffn      - per pair: dequantized gate/up projections w = scale*q + min evaluated
 *              through exact int32 per-block dot products, SwiGLU, int8 quantization of
 *              the hidden vector, down projection (workload definition; per-block int8
 *              dots as in section "CPU expert pool");
 *   combine  - routing-weighted sum of the k expert outputs added into the residual
 *              (same page, "Doorbell handshake": combine expert outputs, write back
 *              the residual).
 *   router   - the router's logits of a token: the dot product of its MoE input x with
 *              each expert's router row (the router runs on the GPU per the memory table
 *              of "Architecture overview"; its weight precision is not given by the pages:
 *              rows are bf16 here, x fp32, each product exact in binary64, the sum over
 *              the model dimension in binary64, rounded once to binary32);
 *   shared   - optionally one always-active shared expert of the routed experts' shape
 *              and quantization, run for every token and added with weight 1 after the
 *              routed slots (reading of the model table's "10+1" active experts per
 *              token and the GPU-resident shared expert of the Strata pages; the pages
 *              give no gate for it, so its weight is 1).
 *   prefill  - the same layer for a long chunk with bf16 weights and activations
 *              (chunks of up to 8192 tokens, "Architecture overview").
 *
 * Precision: binary64 throughout, except where a float decides an integer (the int8
 * activation codes), which is done in binary32, the precision the GPU kernels decide
 * in. Each block term scale*act_scale*dot and min*act_scale*sum is exact in binary64
 * (fp16 x fp32 x 16-bit integer products have at most 51 significant bits), so only
 * the sums round.
 *
 * Packed layout read (the layout the input generator writes):
 *   codes     uint32 [E][cols/32][rows][bits]
 *   scale_min uint16 [E][cols/32][rows][2]   (fp16 scale, fp16 min)
 * code i (0..31) of a block sits in word i/(32/bits) at bit offset bits*(i%(32/bits)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  const uint32_t* codes;
  const uint16_t* scale_min;
  int32_t rows, cols, bits;
} orc_matrix;

/* Optional intermediate outputs of orc_ffn_decode (each pointer may be NULL).
 * Pair index p = t*k + j for selected-token position t and slot j; with a shared expert,
 * its pair of token position t follows all routed pairs: p = n*k + t (Q pairs in all). */
typedef struct {
  int8_t* xq;         /* [n][d]          */
  float* xs;          /* [n][d/32]       */
  int32_t* gate_dots; /* [Q][f][d/32]    */
  int32_t* up_dots;   /* [Q][f][d/32]    */
  double* g;          /* [Q][f]          */
  double* u;          /* [Q][f]          */
  float* h;           /* [Q][f]          */
  int8_t* hq;         /* [Q][f]          */
  float* hs;          /* [Q][f/32]       */
  int32_t* down_dots; /* [Q][d][f/32]    */
  double* y;          /* [Q][d]          */
} orc_trace;

/* binary16 -> binary64 from the IEEE 754 definition */
static double half_to_double(uint16_t h) {
  const int sign = h >> 15, ex = (h >> 10) & 31, man = h & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man + 1024), ex - 25); /* (1 + man/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

/* binary32 -> bfloat16, round to nearest even */
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double bf16_to_double(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static size_t blk_index(const orc_matrix* M, int e, int r, int b) {
  return ((size_t)e * (size_t)(M->cols / 32) + (size_t)b) * (size_t)M->rows + (size_t)r;
}

/* unsigned code q of weight (row r, column c) of expert e */
static int orc_code(const orc_matrix* M, int e, int r, int c) {
  const int per = 32 / M->bits, b = c / 32, i = c % 32;
  const uint32_t word = M->codes[blk_index(M, e, r, b) * (size_t)M->bits + (size_t)(i / per)];
  return (int)((word >> (M->bits * (i % per))) & ((1u << M->bits) - 1u));
}

static double orc_scale(const orc_matrix* M, int e, int r, int b) {
  return half_to_double(M->scale_min[blk_index(M, e, r, b) * 2]);
}

static double orc_min(const orc_matrix* M, int e, int r, int b) {
  return half_to_double(M->scale_min[blk_index(M, e, r, b) * 2 + 1]);
}

/* Dequantized weight w = scale*q + min, in binary64 (exact). */
double orc_weight(const orc_matrix* M, int e, int r, int c) {
  return orc_scale(M, e, r, c / 32) * (double)orc_code(M, e, r, c) + orc_min(M, e, r, c / 32);
}

/* Dequantized weight as the bf16 prefill path sees it: fp32 scale*q (exact) + fp32 min,
 * rounded once to fp32, then rounded to bf16. */
uint16_t orc_weight_bf16(const orc_matrix* M, int e, int r, int c) {
  const float s = (float)orc_scale(M, e, r, c / 32);
  const float m = (float)orc_min(M, e, r, c / 32);
  const float q = (float)orc_code(M, e, r, c);
  const float w = s * q + m;
  return bf16_rne(w);
}

/* ---- route: top-k selection and routing weights ---------------------------------- */

/* Order: larger logit first; equal logits (-0 equals +0) -> lower expert id first.
 * Weights: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected, slot 0 the
 * largest; identical to softmax over all E experts followed by renormalisation over
 * the selected k. Returns 0, or 1 on bad arguments. */
int orc_route(const float* logits, int n, int E, int k, int32_t* ids, float* w) {
  if (n < 0 || E < 1 || k < 1 || k > E) return 1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  double* ex = (double*)malloc(sizeof(double) * (size_t)k);
  if (!taken || !ex) {
    free(taken);
    free(ex);
    return 1;
  }
  for (int t = 0; t < n; ++t) {
    const float* l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower id */
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    const double l0 = (double)l[ids[(size_t)t * k]];
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      ex[j] = exp((double)l[ids[(size_t)t * k + j]] - l0);
      sum += ex[j];
    }
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = (float)(ex[j] / sum);
  }
  free(taken);
  free(ex);
  return 0;
}

/* ---- router: logits[t][e] = sum_c x[t][c] * W[e][c] ----------------------------- */

/* W: bf16 bit patterns, [E][d] row-major (row e holds expert e's router weights).
 * Each product bf16 x fp32 is exact in binary64; the sum runs over c in increasing order
 * in binary64 and is rounded to binary32 once. Returns 0, or 1 on bad arguments. */
int orc_router_logits(const uint16_t* W, const float* x, int n, int d, int E, float* logits) {
  if (n < 0 || d < 1 || E < 1) return 1;
  for (int t = 0; t < n; ++t) {
    const float* xt = x + (size_t)t * d;
    for (int e = 0; e < E; ++e) {
      const uint16_t* we = W + (size_t)e * d;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += bf16_to_double(we[c]) * (double)xt[c];
      logits[(size_t)t * E + e] = (float)acc;
    }
  }
  return 0;
}

/* ---- group: stable counting sort of pairs p = t*k + j by expert ------------------ */

int orc_group(const int32_t* ids, int n, int k, int E, int32_t* offsets, int32_t* pair_index) {
  if (n < 0 || k < 1 || E < 1) return 1;
  const int P = n * k;
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!fill) return 1;
  for (int e = 0; e <= E; ++e) offsets[e] = 0;
  for (int p = 0; p < P; ++p) {
    if (ids[p] < 0 || ids[p] >= E) {
      free(fill);
      return 1;
    }
    offsets[ids[p] + 1] += 1;
  }
  for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  for (int p = 0; p < P; ++p) {
    const int e = ids[p];
    pair_index[offsets[e] + fill[e]] = p;
    fill[e] += 1;
  }
  free(fill);
  return 0;
}

/* ---- int8 block quantization (decided in binary32) ------------------------------- */

/* 32 values -> codes in [-127,127] and a scale: amax = max|v|; scale = amax/127;
 * code = rne(v * (127/amax)); an all-zero block gets scale 0 and codes 0. */
static void orc_quant32(const float* v, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    const float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    *scale = 0.0f;
    for (int i = 0; i < 32; ++i) q[i] = 0;
    return;
  }
  *scale = amax / 127.0f;
  const float inv = 127.0f / amax;
  for (int i = 0; i < 32; ++i) {
    float t = rintf(v[i] * inv);
    if (t > 127.0f) t = 127.0f;
    if (t < -127.0f) t = -127.0f;
    q[i] = (int8_t)t;
  }
}

void orc_quant_act(const float* x, int64_t len, int8_t* q, float* s) {
  for (int64_t b = 0; b < len / 32; ++b) orc_quant32(x + 32 * b, q + 32 * b, s + b);
}

/* ---- one matrix-vector product through exact per-block integer dots --------------- */

/* out[r] = sum_c (scale*q + min)[r][c] * (as[c/32]*aq[c]) for expert e, written as
 * sum_b  scale_b*as_b*dot_b + min_b*as_b*sum_b  with dot_b = sum_i q_i*aq_i and
 * sum_b = sum_i aq_i (exact int32). dots (optional) receives [rows][cols/32]. */
static void orc_qmatvec(const orc_matrix* M, int e, const int8_t* aq, const float* as,
                        double* out, int32_t* dots) {
  const int nb = M->cols / 32;
  for (int r = 0; r < M->rows; ++r) {
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) {
      int32_t dot = 0, sum = 0;
      for (int i = 0; i < 32; ++i) {
        const int c = 32 * b + i;
        dot += orc_code(M, e, r, c) * (int32_t)aq[c];
        sum += (int32_t)aq[c];
      }
      if (dots) dots[(size_t)r * nb + b] = dot;
      acc += orc_scale(M, e, r, b) * (double)as[b] * (double)dot;
      acc += orc_min(M, e, r, b) * (double)as[b] * (double)sum;
    }
    out[r] = acc;
  }
}

static int matrices_ok(const orc_matrix* gate, const orc_matrix* up, const orc_matrix* down, int d,
                       int f) {
  const orc_matrix* m[3] = {gate, up, down};
  for (int i = 0; i < 3; ++i)
    if (!m[i] || (m[i]->bits != 2 && m[i]->bits != 4)) return 0;
  return gate->rows == f && gate->cols == d && up->rows == f && up->cols == d && down->rows == d &&
         down->cols == f && d % 32 == 0 && f % 32 == 0 && d > 0 && f > 0;
}

/* ---- decode layer: quant -> gate/up -> SwiGLU -> quant -> down -> combine ---------- */

/* One expert e of (gate, up, down) on one quantized token (aq, as): gate and up through
 * int32 block dots, SwiGLU, int8 quantization of h, down; y [d] in binary64. Trace slot p
 * of tr receives the intermediates when tr is given. */
static void orc_expert_ffn(const orc_matrix* gate, const orc_matrix* up, const orc_matrix* down,
                           int e, const int8_t* aq, const float* as, int d, int f, double* y,
                           const orc_trace* tr, size_t p) {
  const int nbd = d / 32, nbf = f / 32;
  double* g = (double*)malloc(sizeof(double) * (size_t)f);
  double* u = (double*)malloc(sizeof(double) * (size_t)f);
  float* h = (float*)malloc(sizeof(float) * (size_t)f);
  int8_t* hq = (int8_t*)malloc((size_t)f);
  float* hs = (float*)malloc(sizeof(float) * (size_t)nbf);
  orc_qmatvec(gate, e, aq, as, g, tr && tr->gate_dots ? tr->gate_dots + p * f * nbd : NULL);
  orc_qmatvec(up, e, aq, as, u, tr && tr->up_dots ? tr->up_dots + p * f * nbd : NULL);
  for (int r = 0; r < f; ++r) {
    const double silu = g[r] / (1.0 + exp(-g[r])); /* SwiGLU: silu(gate) * up */
    h[r] = (float)(silu * u[r]);
  }
  orc_quant_act(h, f, hq, hs);
  orc_qmatvec(down, e, hq, hs, y, tr && tr->down_dots ? tr->down_dots + p * d * nbf : NULL);
  if (tr) {
    if (tr->g) memcpy(tr->g + p * f, g, sizeof(double) * (size_t)f);
    if (tr->u) memcpy(tr->u + p * f, u, sizeof(double) * (size_t)f);
    if (tr->h) memcpy(tr->h + p * f, h, sizeof(float) * (size_t)f);
    if (tr->hq) memcpy(tr->hq + p * f, hq, (size_t)f);
    if (tr->hs) memcpy(tr->hs + p * nbf, hs, sizeof(float) * (size_t)nbf);
    if (tr->y) memcpy(tr->y + p * d, y, sizeof(double) * (size_t)d);
  }
  free(g);
  free(u);
  free(h);
  free(hq);
  free(hs);
}

/* Tokens `tokens[0..n_sel)` (all n tokens in order when tokens == NULL) are evaluated:
 *   out[s][:] = residual[t][:] + sum_j w[t][j] * y_{t,j}[:]  (+ y_shared_t[:])
 * in binary64, slot order j = 0..k-1 and the shared expert last, with t = tokens[s]; the
 * expert FFN of pair (t, j) uses expert ids[t][j], the shared one (when sgate, sup and
 * sdown are given, each holding one expert) expert 0 of those matrices.
 * x, residual: [n][d] fp32; out: [n_sel][d] fp32. Returns 0, or 1 on bad arguments. */
int orc_ffn_decode(const orc_matrix* gate, const orc_matrix* up, const orc_matrix* down, int d,
                   int f, int E, int k, const float* x, int n, const int32_t* ids, const float* w,
                   const float* residual, const int32_t* tokens, int n_sel, float* out,
                   const orc_trace* tr, int nthreads, const orc_matrix* sgate,
                   const orc_matrix* sup, const orc_matrix* sdown) {
  if (!matrices_ok(gate, up, down, d, f) || k < 1 || k > E || n < 0) return 1;
  const int shared = sgate != NULL;
  if (shared && (!sup || !sdown || !matrices_ok(sgate, sup, sdown, d, f))) return 1;
  if (!tokens) n_sel = n;
  for (int s = 0; s < n_sel; ++s) {
    const int t = tokens ? tokens[s] : s;
    if (t < 0 || t >= n) return 1;
    for (int j = 0; j < k; ++j)
      if (ids[(size_t)t * k + j] < 0 || ids[(size_t)t * k + j] >= E) return 1;
  }
  const int nbd = d / 32;
  const int P = n_sel * k, Q = P + (shared ? n_sel : 0);
  double* y = (double*)malloc(sizeof(double) * ((size_t)Q + 1) * d);
  int8_t* xq = (int8_t*)malloc((size_t)n_sel * d + 1);
  float* xs = (float*)malloc(sizeof(float) * ((size_t)n_sel * nbd + 1));
  if (!y || !xq || !xs) {
    free(y);
    free(xq);
    free(xs);
    return 1;
  }
  for (int s = 0; s < n_sel; ++s) {
    const int t = tokens ? tokens[s] : s;
    orc_quant_act(x + (size_t)t * d, d, xq + (size_t)s * d, xs + (size_t)s * nbd);
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int p = 0; p < Q; ++p) {
    if (p < P) {
      const int s = p / k, j = p % k;
      const int t = tokens ? tokens[s] : s;
      orc_expert_ffn(gate, up, down, ids[(size_t)t * k + j], xq + (size_t)s * d,
                     xs + (size_t)s * nbd, d, f, y + (size_t)p * d, tr, (size_t)p);
    } else {
      const int s = p - P;
      orc_expert_ffn(sgate, sup, sdown, 0, xq + (size_t)s * d, xs + (size_t)s * nbd, d, f,
                     y + (size_t)p * d, tr, (size_t)p);
    }
  }
  for (int s = 0; s < n_sel; ++s) {
    const int t = tokens ? tokens[s] : s;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += (double)w[(size_t)t * k + j] * y[((size_t)s * k + j) * d + c];
      if (shared) acc += y[((size_t)P + s) * d + c];
      out[(size_t)s * d + c] = (float)((double)residual[(size_t)t * d + c] + acc);
    }
  }
  if (tr && tr->xq) memcpy(tr->xq, xq, (size_t)n_sel * d);
  if (tr && tr->xs) memcpy(tr->xs, xs, sizeof(float) * (size_t)n_sel * nbd);
  free(y);
  free(xq);
  free(xs);
  return 0;
}

/* ---- prefill layer: bf16 weights and activations ---------------------------------- */

/* Same layer as orc_ffn_decode with the activations in bf16 instead of int8:
 *   g, u  = W_bf16 . x_bf16     (binary64 sums of bf16 products)
 *   h     = bf16(fp32(silu(g) * u))
 *   y     = Wd_bf16 . h         (binary64)
 *   out   = residual + sum_j w_j * y_j
 * where W_bf16 = bf16(fp32(scale*q + min)). Optional traces g, u [n_sel*k][f] (binary64),
 * hb [n_sel*k][f] (bf16 bits), y [n_sel*k][d] (binary64). */
int orc_ffn_prefill(const orc_matrix* gate, const orc_matrix* up, const orc_matrix* down, int d,
                    int f, int E, int k, const uint16_t* x_bf16, int n, const int32_t* ids,
                    const float* w, const float* residual, const int32_t* tokens, int n_sel,
                    float* out, double* tr_g, double* tr_u, uint16_t* tr_hb, double* tr_y,
                    int nthreads) {
  if (!matrices_ok(gate, up, down, d, f) || k < 1 || k > E || n < 0) return 1;
  if (!tokens) n_sel = n;
  for (int s = 0; s < n_sel; ++s) {
    const int t = tokens ? tokens[s] : s;
    if (t < 0 || t >= n) return 1;
    for (int j = 0; j < k; ++j)
      if (ids[(size_t)t * k + j] < 0 || ids[(size_t)t * k + j] >= E) return 1;
  }
  const int P = n_sel * k;
  double* y = (double*)malloc(sizeof(double) * (size_t)P * d);
  if (!y) return 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int p = 0; p < P; ++p) {
    const int s = p / k, j = p % k;
    const int t = tokens ? tokens[s] : s;
    const int e = ids[(size_t)t * k + j];
    const uint16_t* xt = x_bf16 + (size_t)t * d;
    uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)f);
    /* each weight is bf16(fp32(s*q + m)) as orc_weight_bf16 computes it; the block's
     * scale and min are read once per 32 columns instead of once per column */
    for (int r = 0; r < f; ++r) {
      double g = 0.0, u = 0.0;
      for (int b = 0; b < d / 32; ++b) {
        const float gs = (float)orc_scale(gate, e, r, b), gm = (float)orc_min(gate, e, r, b);
        const float us = (float)orc_scale(up, e, r, b), um = (float)orc_min(up, e, r, b);
        for (int i = 0; i < 32; ++i) {
          const int c = 32 * b + i;
          const double xv = bf16_to_double(xt[c]);
          const float gw = gs * (float)orc_code(gate, e, r, c) + gm;
          const float uw = us * (float)orc_code(up, e, r, c) + um;
          g += bf16_to_double(bf16_rne(gw)) * xv;
          u += bf16_to_double(bf16_rne(uw)) * xv;
        }
      }
      const double silu = g / (1.0 + exp(-g));
      hb[r] = bf16_rne((float)(silu * u));
      if (tr_g) tr_g[(size_t)p * f + r] = g;
      if (tr_u) tr_u[(size_t)p * f + r] = u;
      if (tr_hb) tr_hb[(size_t)p * f + r] = hb[r];
    }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int b = 0; b < f / 32; ++b) {
        const float ds = (float)orc_scale(down, e, c, b), dm = (float)orc_min(down, e, c, b);
        for (int i = 0; i < 32; ++i) {
          const int r = 32 * b + i;
          const float dw = ds * (float)orc_code(down, e, c, r) + dm;
          acc += bf16_to_double(bf16_rne(dw)) * bf16_to_double(hb[r]);
        }
      }
      y[(size_t)p * d + c] = acc;
      if (tr_y) tr_y[(size_t)p * d + c] = acc;
    }
    free(hb);
  }
  for (int s = 0; s < n_sel; ++s) {
    const int t = tokens ? tokens[s] : s;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += (double)w[(size_t)t * k + j] * y[((size_t)s * k + j) * d + c];
      out[(size_t)s * d + c] = (float)((double)residual[(size_t)t * d + c] + acc);
    }
  }
  free(y);
  return 0;
}

/* number of threads an OpenMP region of this library uses with the given request */
int orc_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) return nthreads;
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}
