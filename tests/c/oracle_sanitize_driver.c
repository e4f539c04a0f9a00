/* Drives every entry point of the CPU oracle on small seeded inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (the oracle source is compiled into
 * this program). Inputs come from a 64-bit linear congruential generator; the program
 * checks nothing about the values (the pins do that) and exits 0 unless an entry point
 * reports bad arguments. */
#include "../../oracle/qmoe_oracle.c"

#include <stdio.h>

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg_state >> 32);
}

static float next_f(void) { /* roughly uniform in [-2, 2) */
  return ((float)(next_u32() >> 8) / 16777216.0f) * 4.0f - 2.0f;
}

/* finite fp16 bit patterns of modest magnitude for scales and mins */
static uint16_t next_half(void) {
  static const uint16_t pool[8] = {0x2000, 0x2A00, 0x1C00, 0xA400, 0x9C00, 0x0000, 0x2400, 0xA000};
  return pool[next_u32() & 7];
}

static orc_matrix make_matrix(int E, int rows, int cols, int bits, uint32_t** codes,
                              uint16_t** sm) {
  const size_t blocks = (size_t)E * (size_t)(cols / 32) * (size_t)rows;
  *codes = (uint32_t*)malloc(sizeof(uint32_t) * blocks * (size_t)bits);
  *sm = (uint16_t*)malloc(sizeof(uint16_t) * blocks * 2);
  for (size_t i = 0; i < blocks * (size_t)bits; ++i) (*codes)[i] = next_u32();
  for (size_t i = 0; i < blocks * 2; ++i) (*sm)[i] = next_half();
  orc_matrix m = {*codes, *sm, rows, cols, bits};
  return m;
}

static int run(int E, int d, int f, int k, int n, int bits) {
  int bad = 0;
  uint32_t *gc, *uc, *dc, *sgc, *suc, *sdc;
  uint16_t *gs, *us, *ds, *sgs, *sus, *sds;
  orc_matrix g = make_matrix(E, f, d, bits, &gc, &gs);
  orc_matrix u = make_matrix(E, f, d, bits, &uc, &us);
  orc_matrix dn = make_matrix(E, d, f, bits, &dc, &ds);
  orc_matrix sg = make_matrix(1, f, d, bits, &sgc, &sgs);
  orc_matrix su = make_matrix(1, f, d, bits, &suc, &sus);
  orc_matrix sd = make_matrix(1, d, f, bits, &sdc, &sds);
  float* x = (float*)malloc(sizeof(float) * (size_t)n * d);
  float* res = (float*)malloc(sizeof(float) * (size_t)n * d);
  float* lg = (float*)malloc(sizeof(float) * (size_t)n * E);
  uint16_t* xb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * d);
  uint16_t* rw = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)E * d);
  for (int i = 0; i < n * d; ++i) {
    x[i] = next_f();
    res[i] = next_f();
    xb[i] = bf16_rne(x[i]);
  }
  for (int i = 0; i < 32 && i < d; ++i) x[i] = 0.0f; /* an all-zero block */
  for (int i = 0; i < n * E; ++i) lg[i] = (float)(int)(next_f() * 2.0f); /* ties */
  for (int i = 0; i < E * d; ++i) rw[i] = bf16_rne(next_f() * 0.1f);

  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)n * k);
  float* w = (float*)malloc(sizeof(float) * (size_t)n * k);
  int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* pidx = (int32_t*)malloc(sizeof(int32_t) * (size_t)n * k + 1);
  float* lgp = (float*)malloc(sizeof(float) * (size_t)n * E);
  bad |= orc_route(lg, n, E, k, ids, w);
  bad |= orc_group(ids, n, k, E, off, pidx);
  bad |= orc_router_logits(rw, x, n, d, E, lgp);

  int8_t* q = (int8_t*)malloc((size_t)n * d);
  float* qs = (float*)malloc(sizeof(float) * (size_t)n * (d / 32));
  orc_quant_act(x, (int64_t)n * d, q, qs);

  const int Q = n * k + n;
  orc_trace tr;
  tr.xq = (int8_t*)malloc((size_t)n * d);
  tr.xs = (float*)malloc(sizeof(float) * (size_t)n * (d / 32));
  tr.gate_dots = (int32_t*)malloc(sizeof(int32_t) * (size_t)Q * f * (d / 32));
  tr.up_dots = (int32_t*)malloc(sizeof(int32_t) * (size_t)Q * f * (d / 32));
  tr.g = (double*)malloc(sizeof(double) * (size_t)Q * f);
  tr.u = (double*)malloc(sizeof(double) * (size_t)Q * f);
  tr.h = (float*)malloc(sizeof(float) * (size_t)Q * f);
  tr.hq = (int8_t*)malloc((size_t)Q * f);
  tr.hs = (float*)malloc(sizeof(float) * (size_t)Q * (f / 32));
  tr.down_dots = (int32_t*)malloc(sizeof(int32_t) * (size_t)Q * d * (f / 32));
  tr.y = (double*)malloc(sizeof(double) * (size_t)Q * d);
  float* out = (float*)malloc(sizeof(float) * (size_t)n * d);
  bad |= orc_ffn_decode(&g, &u, &dn, d, f, E, k, x, n, ids, w, res, NULL, 0, out, &tr, 2, &sg,
                        &su, &sd);
  bad |= orc_ffn_decode(&g, &u, &dn, d, f, E, k, x, n, ids, w, res, NULL, 0, out, NULL, 1, NULL,
                        NULL, NULL);
  int32_t tokens[2] = {n - 1, 0};
  bad |= orc_ffn_decode(&g, &u, &dn, d, f, E, k, x, n, ids, w, res, tokens, 2, out, NULL, 0, NULL,
                        NULL, NULL);
  double* tg = (double*)malloc(sizeof(double) * (size_t)n * k * f);
  double* tu = (double*)malloc(sizeof(double) * (size_t)n * k * f);
  uint16_t* thb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n * k * f);
  double* ty = (double*)malloc(sizeof(double) * (size_t)n * k * d);
  bad |= orc_ffn_prefill(&g, &u, &dn, d, f, E, k, xb, n, ids, w, res, NULL, 0, out, tg, tu, thb,
                         ty, 2);
  bad |= orc_ffn_prefill(&g, &u, &dn, d, f, E, k, xb, n, ids, w, res, tokens, 2, out, NULL, NULL,
                         NULL, NULL, 1);
  (void)orc_weight(&g, E - 1, f - 1, d - 1);
  (void)orc_weight_bf16(&dn, 0, d - 1, f - 1);
  /* rejected arguments report 1 and touch nothing */
  if (orc_route(lg, n, E, E + 1, ids, w) != 1) bad = 1;
  if (orc_ffn_decode(&g, &u, &dn, d + 32, f, E, k, x, n, ids, w, res, NULL, 0, out, NULL, 0,
                     NULL, NULL, NULL) != 1)
    bad = 1;

  printf("E=%d d=%d f=%d k=%d n=%d bits=%d out[0]=%g\n", E, d, f, k, n, bits, (double)out[0]);
  free(gc); free(gs); free(uc); free(us); free(dc); free(ds);
  free(sgc); free(sgs); free(suc); free(sus); free(sdc); free(sds);
  free(x); free(res); free(lg); free(xb); free(rw); free(ids); free(w); free(off); free(pidx);
  free(lgp); free(q); free(qs); free(out); free(tg); free(tu); free(thb); free(ty);
  free(tr.xq); free(tr.xs); free(tr.gate_dots); free(tr.up_dots); free(tr.g); free(tr.u);
  free(tr.h); free(tr.hq); free(tr.hs); free(tr.down_dots); free(tr.y);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run(5, 96, 64, 2, 7, 4);
  bad |= run(3, 64, 96, 3, 4, 2);  /* k = E */
  bad |= run(8, 256, 128, 1, 3, 4);
  (void)orc_threads(0);
  printf(bad ? "FAILED\n" : "oracle driver ok\n");
  return bad;
}
