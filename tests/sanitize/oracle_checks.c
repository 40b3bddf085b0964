/* The oracle under AddressSanitizer / UndefinedBehaviorSanitizer: every exported entry point
 * on small seeded problems that cover the shapes the parity tests use -- single tokens, ragged
 * tiles, N != M, both causal alignments, d = 64 and 128, bf16 and fp16 inputs -- and every
 * option bit, plus the arguments each call must reject.  Checks only that the calls return what
 * their headers promise and that the outputs are finite; the values themselves are pinned by the
 * oracle's own tests.  Built and run by tests/test_sanitizers.py (test infrastructure only). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "sage_oracle.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      failures++;                                                         \
    }                                                                     \
  } while (0)

/* splitmix64: seeded draws, mapped to roughly N(0, s^2) 16-bit codes (bf16 or fp16) */
static uint64_t rng_state;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static float draw(float s) { /* sum of four uniforms: mean 0, variance 1/3 -> scaled */
  float a = 0.0f;
  for (int i = 0; i < 4; i++) a += (float)(next_u64() >> 40) / 16777216.0f - 0.5f;
  return a * 1.7320508f * s;
}
static uint16_t to_bf16(float x) {
  union { float f; uint32_t u; } v = {x};
  return (uint16_t)((v.u + 0x7FFFu + ((v.u >> 16) & 1u)) >> 16);
}
static uint16_t to_fp16(float x) { /* only the normal range is needed here */
  union { float f; uint32_t u; } v = {x};
  const uint32_t s = (v.u >> 16) & 0x8000u;
  int e = (int)((v.u >> 23) & 0xFF) - 127 + 15;
  uint32_t m = v.u & 0x7FFFFFu;
  if (e <= 0) return (uint16_t)s;
  uint32_t r = (m >> 13) + (((m >> 12) & 1u) & ((m & 0x17FFu) != 0 || ((m >> 13) & 1u)));
  if (r == 0x400u) { r = 0; e++; }
  if (e >= 31) return (uint16_t)(s | 0x7BFFu);
  return (uint16_t)(s | ((uint32_t)e << 10) | r);
}
static uint16_t* tensor(int rows, int d, int fp16, float off, uint64_t seed) {
  uint16_t* t = malloc(sizeof(uint16_t) * (size_t)(rows > 0 ? rows : 1) * d);
  rng_state = seed;
  float o[128];
  for (int c = 0; c < d; c++) o[c] = draw(off);
  for (int r = 0; r < rows; r++)
    for (int c = 0; c < d; c++) {
      const float x = draw(1.0f) + o[c];
      t[(size_t)r * d + c] = fp16 ? to_fp16(x) : to_bf16(x);
    }
  return t;
}
static int all_finite(const double* x, size_t n) {
  for (size_t i = 0; i < n; i++)
    if (!isfinite(x[i])) return 0;
  return 1;
}

struct shape {
  int N, M, d, fp16, causal;
};

static void one_shape(struct shape s, uint64_t seed) {
  const int N = s.N, M = s.M, d = s.d;
  const double sm = 1.0 / sqrt((double)d);
  uint16_t* q = tensor(N, d, s.fp16, 1.0f, seed);
  uint16_t* k = tensor(M, d, s.fp16, 3.0f, seed + 1);
  uint16_t* v = tensor(M, d, s.fp16, 0.5f, seed + 2);
  uint16_t* dout = tensor(N, d, s.fp16, 0.0f, seed + 3);
  const int nqb = (N + ORC_BQ - 1) / ORC_BQ, nkt = (M + ORC_BK - 1) / ORC_BK;
  double* out = calloc((size_t)(N > 3 ? N : 3) * d, sizeof(double)); /* all rows, or 3 sampled ones */
  /* forward of every option combination the tests use */
  const unsigned fwd_flags[] = {0, ORC_SMOOTH_V, ORC_NO_SMOOTH_K, ORC_NO_SMOOTH_Q, ORC_QK_IDENTITY,
                                ORC_QK_PER_BLOCK, ORC_QK_PER_TOKEN, ORC_QK_PER_TENSOR, ORC_PV_IDENTITY,
                                ORC_PV_E5M2, ORC_PV_INT8, ORC_MXFP4, ORC_MXFP4 | ORC_SMOOTH_V,
                                ORC_MXFP4 | ORC_MX_P_TWO_LEVEL, ORC_QK_E4M3, ORC_QK_E4M3 | ORC_SMOOTH_V};
  for (size_t f = 0; f < sizeof fwd_flags / sizeof fwd_flags[0]; f++) {
    EXPECT(orc_forward_head(q, k, v, s.fp16, N, M, d, s.causal, sm, fwd_flags[f], NULL, N, out) == 0);
    EXPECT(all_finite(out, (size_t)N * d));
  }
  /* a row subset, with the tie diagnostic (and the FP8-QK score margin) */
  int rows[3] = {0, N / 2, N - 1};
  int ties[3];
  double bound[3];
  EXPECT(orc_forward_head_ties(q, k, v, s.fp16, N, M, d, s.causal, sm, 0, rows, 3, out, 1e-4, 0.0, ties,
                               bound) == 0);
  EXPECT(all_finite(out, (size_t)3 * d) && all_finite(bound, 3));
  EXPECT(orc_forward_head_ties(q, k, v, s.fp16, N, M, d, s.causal, sm, ORC_QK_E4M3, rows, 3, out, 1e-4,
                               1e-3, ties, bound) == 0);
  EXPECT(orc_forward_head_ties(q, k, v, s.fp16, N, M, d, s.causal, sm, ORC_MXFP4 | ORC_MX_P_TWO_LEVEL, rows,
                               3, out, 1e-4, 0.0, ties, NULL) == 0);
  EXPECT(orc_exact_head(q, k, v, s.fp16, N, M, d, s.causal, sm, rows, 3, out) == 0);
  EXPECT(all_finite(out, (size_t)3 * d));
  /* preprocessing */
  float *kmean = malloc(sizeof(float) * d), *vmean = malloc(sizeof(float) * d);
  int8_t *khat = malloc((size_t)M * d), *qhat = malloc((size_t)N * d);
  uint8_t* vhat = malloc((size_t)M * d);
  float *dk = malloc(sizeof(float) * nkt * 4), *dv = malloc(sizeof(float) * d), *dq = malloc(sizeof(float) * N);
  float* qmean = malloc(sizeof(float) * (size_t)nqb * d);
  double* ds = malloc(sizeof(double) * (size_t)nqb * M);
  const unsigned pre_flags[] = {0, ORC_SMOOTH_V, ORC_QK_PER_BLOCK, ORC_QK_E4M3, ORC_NO_SMOOTH_K | ORC_NO_SMOOTH_Q};
  for (size_t f = 0; f < sizeof pre_flags / sizeof pre_flags[0]; f++)
    EXPECT(orc_preprocess_head(q, k, v, s.fp16, N, M, d, pre_flags[f], kmean, vmean, khat, dk, vhat, dv, qhat,
                               dq, qmean, ds) == 0);
  EXPECT(all_finite(ds, (size_t)nqb * M));
  uint8_t *qc = malloc((size_t)N * d), *kc = malloc((size_t)M * d), *vc = malloc((size_t)M * d);
  int *qe = malloc(sizeof(int) * (size_t)N * (d / 32)), *ke = malloc(sizeof(int) * (size_t)M * (d / 32));
  int* ve = malloc(sizeof(int) * (size_t)((M + 31) / 32) * d);
  EXPECT(orc_preprocess_mx_head(q, k, v, s.fp16, N, M, d, ORC_SMOOTH_V, qc, qe, kc, ke, vc, ve) == 0);
  /* SageBwd: forward, backward (plain and ablations), quantize with optional outputs absent */
  if (N == M || s.causal != 2) {
    double* lse = malloc(sizeof(double) * N);
    double *gq = malloc(sizeof(double) * (size_t)N * d), *gk = malloc(sizeof(double) * (size_t)M * d);
    double* gv = malloc(sizeof(double) * (size_t)M * d);
    const unsigned sb_flags[] = {0, ORC_SB_IDENTITY, ORC_SB_NO_SMOOTH_K, ORC_SB_DP_INT8};
    for (size_t f = 0; f < sizeof sb_flags / sizeof sb_flags[0]; f++) {
      EXPECT(orc_sagebwd_forward(q, k, v, s.fp16, N, M, d, s.causal, sm, sb_flags[f], out, lse) == 0);
      EXPECT(orc_sagebwd_backward(q, k, v, dout, s.fp16, N, M, d, s.causal, sm, sb_flags[f], out, lse, gq, gk,
                                  gv) == 0);
      EXPECT(all_finite(gq, (size_t)N * d) && all_finite(gk, (size_t)M * d) && all_finite(gv, (size_t)M * d));
    }
    int8_t* code = malloc((size_t)(N > M ? N : M) * d);
    float* sc = malloc(sizeof(float) * (size_t)(N > M ? N : M));
    EXPECT(orc_sagebwd_quantize(q, k, v, NULL, s.fp16, N, M, d, 0, code, sc, NULL, NULL, NULL, NULL, NULL, NULL,
                                kmean) == 0);
    free(lse), free(gq), free(gk), free(gv), free(code), free(sc);
  }
  free(q), free(k), free(v), free(dout), free(out), free(kmean), free(vmean), free(khat), free(qhat);
  free(vhat), free(dk), free(dv), free(dq), free(qmean), free(ds), free(qc), free(kc), free(vc);
  free(qe), free(ke), free(ve);
}

int main(void) {
  const struct shape shapes[] = {
      {1, 1, 64, 0, 0},    {5, 3, 128, 1, 0},   {130, 70, 64, 0, 1}, {70, 130, 128, 1, 2},
      {200, 333, 64, 0, 2}, {257, 200, 128, 0, 1}, {300, 300, 128, 0, 0},
  };
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; i++) one_shape(shapes[i], 1000 + 17 * i);
  /* arguments every call must reject */
  uint16_t x[64] = {0};
  double o[64];
  EXPECT(orc_forward_head(NULL, x, x, 0, 1, 1, 64, 0, 0.125, 0, NULL, 1, o) == -1);
  EXPECT(orc_forward_head(x, x, x, 0, 1, 1, 96, 0, 0.125, 0, NULL, 1, o) == -1);
  EXPECT(orc_forward_head(x, x, x, 0, 2, 1, 64, 2, 0.125, 0, NULL, 2, o) == -1); /* causal 2 needs N <= M */
  EXPECT(orc_exact_head(x, x, x, 0, 1, 1, 64, 3, 0.125, NULL, 1, o) == -1);
  EXPECT(orc_sagebwd_forward(x, x, x, 0, 0, 1, 64, 0, 0.125, 0, o, o) == -1);
  /* the element codecs over their whole code spaces */
  for (int c = 0; c < 256; c++) {
    const double e4 = orc_e4m3_decode((uint8_t)c), e5 = orc_e5m2_decode((uint8_t)c);
    if (!isnan(e4)) EXPECT(orc_e4m3_decode(orc_e4m3_encode(e4)) == e4);
    if (isfinite(e5)) EXPECT(orc_e5m2_decode(orc_e5m2_encode(e5)) == e5);
  }
  for (int c = 0; c < 16; c++) EXPECT(orc_e2m1_decode(orc_e2m1_encode(orc_e2m1_decode((uint8_t)c))) ==
                                      orc_e2m1_decode((uint8_t)c));
  EXPECT(orc_e8m0_exponent(0.0) == -127 && orc_e8m0_exponent(6.0) == 0);
  if (failures) {
    fprintf(stderr, "%d oracle checks failed\n", failures);
    return 1;
  }
  printf("oracle checks ok\n");
  return 0;
}
