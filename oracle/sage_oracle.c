/*
 * sage_oracle.c -- CPU oracle for the SageAttention2-style quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY: the plain, slow, obviously correct reference for the GPU path.
 * Only the test-suite, the package smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header or table with the HIP library.
 *
 * The method is an approximation defined by where its quantizers sit, so this file takes
 * the pages' algorithm step by step ([SA2] "The Complete Algorithm (Algorithm 1)" and the
 * paragraphs it summarises; [SA2R] forward-pass listing), in the pages' notation:
 *
 *   preprocessing   K <- K - mean(K);  (dV, V^) = psi_V(V)               [SA2 Alg. 1 step 1]
 *   per Q block i   q_i = mean(Q_i); (dQ, Q^_i) = psi_Q(Q_i - q_i)       [SA2 Alg. 1 step 2]
 *   per KV tile j   S = deq(Q^_i K^_j^T) + Delta S_ij                     [SA2 "Smoothing Q"]
 *                   m, P~, l = online softmax                             [SA2 Alg. 1 step 3]
 *                   R = (448 P~ -> E4M3) V^_j ;  O = diag(e^{m_old-m}) O + R   [two-level]
 *   epilogue        O = O / l / 448 * dV  (+ V_m when V is smoothed)      [SA2 Alg. 1 step 4]
 *
 * Everything the method keeps in full precision is FP64 here; the preprocessing follows a
 * pinned FP32/FP64 evaluation order so that Q^, K^, V^, their scales and the means have
 * exactly one correct value.  Where the pages are silent or garbled the reading taken is
 * stated at the step.
 *
 * Build: plain C11, -O2 -fno-fast-math -ffp-contract=off (FP32 steps must round exactly
 * as written), optionally -fopenmp (rows are independent; results do not depend on the
 * thread count).
 */
#include "sage_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ========================================================================================
 * Scalar formats
 * ====================================================================================== */

/* bf16 is the top half of an IEEE binary32: widening is a shift (exact). */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits.  Widening is exact. */
float orc_fp16_to_f32(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return (float)(s ? -v : v);
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 is
 * subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity; the largest finite
 * magnitude is 1.75 * 2^8 = 448 ([SA2] "FP8 Quantization": 448 is the E4M3 maximum).
 * The pages' derivation of that maximum is garbled; the format definition is used. */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

/* Round-to-nearest-even onto a sorted table of non-negative magnitudes vals[0..n-1]
 * (vals[0] = 0, codes equal table indices, an even index has an even mantissa LSB).
 * Magnitudes at or beyond the last entry saturate to it. */
static int nearest_even_index(const double* vals, int n, double a) {
  if (a >= vals[n - 1]) return n - 1;
  int lo = 0, hi = n - 1; /* vals[lo] <= a < vals[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (vals[mid] <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - vals[lo], dhi = vals[hi] - a;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo % 2 == 0) ? lo : hi; /* tie: even mantissa */
}

static double e4m3_mag[127];
static double e5m2_mag[124];
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static int tables_ready = 0;

static void init_tables(void) {
  if (tables_ready) return;
  for (int c = 0; c < 127; c++) e4m3_mag[c] = orc_e4m3_decode((uint8_t)c);
  for (int c = 0; c < 124; c++) e5m2_mag[c] = orc_e5m2_decode((uint8_t)c);
  tables_ready = 1;
}

/* Cast to E4M3FN with round-to-nearest-even and saturation to +-448 (the P~ and V
 * quantizers never exceed 448 by more than a rounding error, which must map to 448). */
uint8_t orc_e4m3_encode(double x) {
  init_tables();
  if (isnan(x)) return 0x7F;
  uint8_t s = signbit(x) ? 0x80 : 0x00;
  return (uint8_t)(s | nearest_even_index(e4m3_mag, 127, fabs(x)));
}

/* The same cast over an array of FP32 values (for exhaustive checks of a device conversion). */
void orc_e4m3_encode_f32_array(const float* x, uint8_t* out, size_t n) {
  init_tables();
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; i++) out[i] = orc_e4m3_encode((double)x[i]);
}

/* OCP E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits, IEEE-like Inf/NaN. */
double orc_e5m2_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
  double v;
  if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
  if (e == 0)
    v = ldexp((double)m, -16);
  else
    v = ldexp(4.0 + m, e - 17);
  return s ? -v : v;
}

uint8_t orc_e5m2_encode(double x) {
  init_tables();
  if (isnan(x)) return 0x7F;
  uint8_t s = signbit(x) ? 0x80 : 0x00;
  return (uint8_t)(s | nearest_even_index(e5m2_mag, 124, fabs(x)));
}

/* E2M1 ([SA3] "The NVFP4 Microscaling Format": values {0, +-0.5, +-1, +-1.5, +-2, +-3,
 * +-4, +-6}).  Code = sign<<3 | magnitude index.  The page's own derivation reaches a
 * maximum of 3 (garbled); the stated value set with maximum 6 is used. */
double orc_e2m1_decode(uint8_t c) {
  double v = e2m1_mag[c & 7];
  return (c & 8) ? -v : v;
}

/* Rounding is "to the nearest representable value"; ties go to the even mantissa
 * (the pages leave the tie rule open; RNE is the reading taken). */
uint8_t orc_e2m1_encode(double x) {
  if (isnan(x)) return 0x7; /* no NaN in E2M1: map to the largest magnitude */
  uint8_t s = signbit(x) ? 0x8 : 0x0;
  return (uint8_t)(s | nearest_even_index(e2m1_mag, 8, fabs(x)));
}

/* E8M0 block scale for an MX block whose largest magnitude is amax: 2^e with the
 * smallest e such that amax <= 6 * 2^e, so that no element clips (reading taken: the
 * pages give s = max/6 for E4M3 scales and are silent on rounding to a power of two).
 * An all-zero block uses e = -127. */
int orc_e8m0_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int e = -127;
  while (e < 127 && amax > 6.0 * ldexp(1.0, e)) e++;
  return e;
}

/* ========================================================================================
 * Step 3 group map.  The per-thread principle ([SA2] "Per-Thread INT4 Quantization"):
 * every element one thread dequantizes shares one (dQ, dK) pair.  The GPU computes
 * S^T = K^ Q^T with 32x32 accumulator tiles; in that tile a lane holds one query column
 * and the 16 key rows {8b + 4h + k : b, k in 0..3} of a 32-key half, h being the lane's
 * half of the wavefront.  So within a 64-key tile, key t has half T = (t mod 64) / 32,
 * row r = t mod 32, and group 2T + ((r >> 2) & 1): four groups of 16 keys, the same
 * count per 64-key tile as the pages' grouping, and Q is quantized per token.
 * ====================================================================================== */
int orc_k_group(int t) {
  int u = t & 63;
  return 2 * (u >> 5) + ((u >> 2) & 1);
}

/* ========================================================================================
 * Per-head state
 * ====================================================================================== */
typedef struct {
  int N, M, d, nqb, nkt;
  unsigned flags;
  float *Qf, *Kf, *Vf;  /* widened inputs                                  */
  float *kmean, *vmean; /* [d]                                              */
  float *gk;            /* FP32 gamma(K) = K - kmean            [M][d]      */
  double *gkd;          /* FP64 gamma(K) (identity mode)        [M][d]      */
  int8_t *khat;         /* INT8 K^                              [M][d]      */
  float *dk_key;        /* dK of each key (expanded)            [M]         */
  float *dk_grp;        /* dK per (tile, group)                 [nkt][4]    */
  float *qmean;         /* per block mean                       [nqb][d]    */
  float *gq;            /* FP32 gamma(Q)                        [N][d]      */
  double *gqd;          /* FP64 gamma(Q) (identity mode)        [N][d]      */
  int8_t *qhat;         /* INT8 Q^                              [N][d]      */
  float *dq;            /* dQ of each token (expanded)          [N]         */
  uint8_t *vhat;        /* E4M3 V^ codes                        [M][d]      */
  double *vq;           /* value of V^ entering the product     [M][d]      */
  float *dv;            /* per-channel V scale                  [d]         */
  double pscale;        /* static P~ scale (448 for E4M3)                    */
  /* MX variant */
  double *qx, *kx;      /* E2M1 values of Q^, K^                [N][d],[M][d] */
  int *qe, *ke;         /* E8M0 exponents per 32 channels       [N][d/32],[M][d/32] */
  double *vx;           /* E2M1 values of V^ (blocks of 32 tokens per channel) [M][d] */
  int *ve;              /* exponents                            [ceil(M/32)][d] */
} head_t;

static void* xcalloc(size_t n, size_t sz) {
  void* p = calloc(n ? n : 1, sz);
  return p;
}

static void head_free(head_t* h) {
  free(h->Qf); free(h->Kf); free(h->Vf); free(h->kmean); free(h->vmean); free(h->gk);
  free(h->gkd); free(h->khat); free(h->dk_key); free(h->dk_grp); free(h->qmean); free(h->gq);
  free(h->gqd); free(h->qhat); free(h->dq); free(h->vhat); free(h->vq); free(h->dv);
  free(h->qx); free(h->kx); free(h->qe); free(h->ke); free(h->vx); free(h->ve);
  memset(h, 0, sizeof(*h));
}

static void widen(const uint16_t* src, int in_fp16, size_t n, float* dst) {
  for (size_t i = 0; i < n; i++) dst[i] = in_fp16 ? orc_fp16_to_f32(src[i]) : orc_bf16_to_f32(src[i]);
}

/* Step 1 (K mean, also V_m) -- [SA2] "Smoothing Q": k = mean(K) over all tokens of the
 * head; [QA] "Failure modes": the mean covers valid tokens only.  Order pinned (reading):
 * each 64-token chunk is summed in token order in FP64, the chunk sums are added in chunk
 * order in FP64, the total is divided by the token count in FP64 and rounded to FP32. */
static void token_mean(const float* X, int T, int d, float* mean) {
  for (int c = 0; c < d; c++) {
    double tot = 0.0;
    for (int u0 = 0; u0 < T; u0 += ORC_BK) {
      double part = 0.0;
      int u1 = u0 + ORC_BK < T ? u0 + ORC_BK : T;
      for (int t = u0; t < u1; t++) part += (double)X[(size_t)t * d + c];
      tot += part;
    }
    mean[c] = (float)(tot / (double)T);
  }
}

/* Symmetric INT8 quantizer ([QA] "Worked example": scale = amax / 127; [SA2] "Smoothing Q":
 * round to nearest).  Readings: range +-127, round half to even, FP32 division by the
 * scale, amax floored at 1e-8 so an all-zero group has a finite scale. */
static float int8_scale(float amax) {
  float a = amax > 1e-8f ? amax : 1e-8f;
  return a / 127.0f;
}
static int8_t int8_code(float x, float scale) {
  float y = nearbyintf(x / scale); /* FP32 division, then RNE (default rounding mode) */
  if (!(y == y)) return 0;
  if (y > 127.0f) y = 127.0f;
  if (y < -127.0f) y = -127.0f;
  return (int8_t)y;
}

/* The E4M3 knob for Q and K ([SA2] the missing FP8-QK ablation the review section names;
 * "FP8 Quantization" fixes the E4M3 range the same way for V): scale = amax / 448 with the
 * same groups as INT8, code = E4M3 of the FP32 quotient (round to nearest even, saturated).
 * Readings: the amax floor 1e-8 and the FP32 division as for INT8. */
static float e4m3_scale(float amax) {
  float a = amax > 1e-8f ? amax : 1e-8f;
  return a / 448.0f;
}
static float qk_scale(const head_t* h, float amax) {
  return (h->flags & ORC_QK_E4M3) ? e4m3_scale(amax) : int8_scale(amax);
}
/* The stored code byte: INT8 two's complement, or the E4M3 code. */
static int8_t qk_code(const head_t* h, float x, float scale) {
  if (h->flags & ORC_QK_E4M3) return (int8_t)orc_e4m3_encode((double)(x / scale));
  return int8_code(x, scale);
}
/* The value a stored code stands for, before its scale. */
static double qk_value(const head_t* h, int8_t c) {
  if (h->flags & ORC_QK_E4M3) return orc_e4m3_decode((uint8_t)c);
  return (double)c;
}

/* Max of |x| that ignores NaN (a NaN element does not set the scale). */
static float amax_upd(float m, float x) {
  float a = fabsf(x);
  return (a > m) ? a : m;
}

/* ---- K side: steps 1-3 ---- */
static int setup_k(head_t* h) {
  int M = h->M, d = h->d;
  size_t Md = (size_t)M * d;
  h->kmean = xcalloc(d, sizeof(float));
  h->gk = xcalloc(Md, sizeof(float));
  h->gkd = xcalloc(Md, sizeof(double));
  h->khat = xcalloc(Md, 1);
  h->dk_key = xcalloc(M, sizeof(float));
  h->dk_grp = xcalloc((size_t)h->nkt * 4, sizeof(float));
  if (!h->kmean || !h->gk || !h->gkd || !h->khat || !h->dk_key || !h->dk_grp) return -1;
  if (!(h->flags & ORC_NO_SMOOTH_K)) token_mean(h->Kf, M, d, h->kmean);
  /* Step 2: gamma(K) = K - kmean, one FP32 subtraction per element. */
  for (size_t i = 0; i < Md; i++) {
    int c = (int)(i % d);
    h->gk[i] = h->Kf[i] - h->kmean[c];
    h->gkd[i] = (double)h->Kf[i] - (double)h->kmean[c];
  }
  if (h->flags & (ORC_QK_IDENTITY | ORC_MXFP4)) return 0;
  /* Step 3: scale groups per the selected granularity, then the INT8 (or E4M3) codes. */
  unsigned g = h->flags;
  if (g & ORC_QK_PER_TENSOR) {
    float am = 0.0f;
    for (size_t i = 0; i < Md; i++) am = amax_upd(am, h->gk[i]);
    float s = qk_scale(h, am);
    for (int t = 0; t < M; t++) h->dk_key[t] = s;
  } else if (g & ORC_QK_PER_TOKEN) {
    for (int t = 0; t < M; t++) {
      float am = 0.0f;
      for (int c = 0; c < d; c++) am = amax_upd(am, h->gk[(size_t)t * d + c]);
      h->dk_key[t] = qk_scale(h, am);
    }
  } else if (g & ORC_QK_PER_BLOCK) {
    for (int u = 0; u < h->nkt; u++) {
      float am = 0.0f;
      for (int t = u * ORC_BK; t < M && t < (u + 1) * ORC_BK; t++)
        for (int c = 0; c < d; c++) am = amax_upd(am, h->gk[(size_t)t * d + c]);
      float s = qk_scale(h, am);
      for (int t = u * ORC_BK; t < M && t < (u + 1) * ORC_BK; t++) h->dk_key[t] = s;
    }
  } else { /* per-thread groups (default); a group with no valid key (ragged last tile)
            * has amax 0 and so the floor scale 1e-8/127 (1e-8/448) */
    for (int u = 0; u < h->nkt; u++) {
      float am[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int t = u * ORC_BK; t < M && t < (u + 1) * ORC_BK; t++) {
        int gr = orc_k_group(t);
        for (int c = 0; c < d; c++) am[gr] = amax_upd(am[gr], h->gk[(size_t)t * d + c]);
      }
      for (int gr = 0; gr < 4; gr++) h->dk_grp[(size_t)u * 4 + gr] = qk_scale(h, am[gr]);
      for (int t = u * ORC_BK; t < M && t < (u + 1) * ORC_BK; t++)
        h->dk_key[t] = h->dk_grp[(size_t)u * 4 + orc_k_group(t)];
    }
  }
  for (size_t i = 0; i < Md; i++) h->khat[i] = qk_code(h, h->gk[i], h->dk_key[i / d]);
  return 0;
}

/* ---- V side: step 4 ([SA2] "FP8 Quantization": per-channel dV = max|V[:,c]| / 448,
 * V^ = E4M3(V / dV); [SA2] "Optional Smoothing of V": V' = V - V_m). ---- */
static int setup_v(head_t* h) {
  int M = h->M, d = h->d;
  size_t Md = (size_t)M * d;
  h->vmean = xcalloc(d, sizeof(float));
  h->vhat = xcalloc(Md, 1);
  h->vq = xcalloc(Md, sizeof(double));
  h->dv = xcalloc(d, sizeof(float));
  float* vp = xcalloc(Md, sizeof(float));
  if (!h->vmean || !h->vhat || !h->vq || !h->dv || !vp) { free(vp); return -1; }
  if (h->flags & ORC_SMOOTH_V) token_mean(h->Vf, M, d, h->vmean);
  for (size_t i = 0; i < Md; i++) vp[i] = h->Vf[i] - h->vmean[i % d]; /* FP32 V' */
  if (h->flags & ORC_MXFP4) {
    /* MX: V' quantized along tokens (the reduction dim of P~V), 32 tokens per block. */
    int nb = (M + 31) / 32;
    h->vx = xcalloc(Md, sizeof(double));
    h->ve = xcalloc((size_t)nb * d, sizeof(int));
    if (!h->vx || !h->ve) { free(vp); return -1; }
    for (int b = 0; b < nb; b++)
      for (int c = 0; c < d; c++) {
        double am = 0.0;
        for (int t = b * 32; t < M && t < b * 32 + 32; t++) {
          double a = fabs((double)vp[(size_t)t * d + c]);
          if (a > am) am = a;
        }
        int e = orc_e8m0_exponent(am);
        h->ve[(size_t)b * d + c] = e;
        for (int t = b * 32; t < M && t < b * 32 + 32; t++)
          h->vx[(size_t)t * d + c] = orc_e2m1_decode(orc_e2m1_encode(ldexp((double)vp[(size_t)t * d + c], -e)));
      }
    h->pscale = 1.0;
    free(vp);
    return 0;
  }
  double vmax = 448.0;
  if (h->flags & ORC_PV_E5M2) vmax = 57344.0;
  if (h->flags & ORC_PV_INT8) vmax = 127.0;
  h->pscale = vmax;
  for (int c = 0; c < d; c++) {
    float am = 0.0f;
    for (int t = 0; t < M; t++) am = amax_upd(am, vp[(size_t)t * d + c]);
    float a = am > 1e-8f ? am : 1e-8f;
    h->dv[c] = a / (float)vmax;
  }
  for (size_t i = 0; i < Md; i++) {
    int c = (int)(i % d);
    if (h->flags & ORC_PV_IDENTITY) {
      /* identity: V' taken in FP64 so that no rounding enters at all */
      h->vq[i] = ((double)h->Vf[i] - (double)h->vmean[c]) / (double)h->dv[c];
      h->vhat[i] = orc_e4m3_encode((double)(vp[i] / h->dv[c]));
    } else if (h->flags & ORC_PV_E5M2) {
      h->vhat[i] = orc_e5m2_encode((double)(vp[i] / h->dv[c]));
      h->vq[i] = orc_e5m2_decode(h->vhat[i]);
    } else if (h->flags & ORC_PV_INT8) {
      int8_t qv = int8_code(vp[i], h->dv[c]);
      h->vhat[i] = (uint8_t)qv;
      h->vq[i] = (double)qv;
    } else {
      /* FP32 division, then one rounding to E4M3 (saturating). */
      h->vhat[i] = orc_e4m3_encode((double)(vp[i] / h->dv[c]));
      h->vq[i] = orc_e4m3_decode(h->vhat[i]);
    }
  }
  free(vp);
  return 0;
}

/* ---- Q side: step 5 ([SA2] "Smoothing Q": q_i = mean(Q_i) over the block's tokens,
 * gamma(Q_i) = Q_i - q_i; per-token INT8 scale under the group map above). ---- */
static int setup_q(head_t* h) {
  int N = h->N, d = h->d;
  size_t Nd = (size_t)N * d;
  h->qmean = xcalloc((size_t)h->nqb * d, sizeof(float));
  h->gq = xcalloc(Nd, sizeof(float));
  h->gqd = xcalloc(Nd, sizeof(double));
  h->qhat = xcalloc(Nd, 1);
  h->dq = xcalloc(N, sizeof(float));
  if (!h->qmean || !h->gq || !h->gqd || !h->qhat || !h->dq) return -1;
  for (int i = 0; i < h->nqb; i++) {
    int r0 = i * ORC_BQ, r1 = r0 + ORC_BQ < N ? r0 + ORC_BQ : N;
    if (!(h->flags & ORC_NO_SMOOTH_Q))
      for (int c = 0; c < d; c++) {
        double s = 0.0; /* rows in order, FP64, then / row count, rounded to FP32 */
        for (int r = r0; r < r1; r++) s += (double)h->Qf[(size_t)r * d + c];
        h->qmean[(size_t)i * d + c] = (float)(s / (double)(r1 - r0));
      }
    for (int r = r0; r < r1; r++)
      for (int c = 0; c < d; c++) {
        size_t x = (size_t)r * d + c;
        h->gq[x] = h->Qf[x] - h->qmean[(size_t)i * d + c];
        h->gqd[x] = (double)h->Qf[x] - (double)h->qmean[(size_t)i * d + c];
      }
  }
  if (h->flags & (ORC_QK_IDENTITY | ORC_MXFP4)) return 0;
  unsigned g = h->flags;
  if (g & ORC_QK_PER_TENSOR) {
    float am = 0.0f;
    for (size_t x = 0; x < Nd; x++) am = amax_upd(am, h->gq[x]);
    for (int r = 0; r < N; r++) h->dq[r] = qk_scale(h, am);
  } else if (g & ORC_QK_PER_BLOCK) {
    for (int i = 0; i < h->nqb; i++) {
      int r0 = i * ORC_BQ, r1 = r0 + ORC_BQ < N ? r0 + ORC_BQ : N;
      float am = 0.0f;
      for (size_t x = (size_t)r0 * d; x < (size_t)r1 * d; x++) am = amax_upd(am, h->gq[x]);
      for (int r = r0; r < r1; r++) h->dq[r] = qk_scale(h, am);
    }
  } else { /* per token: the default per-thread map and the per-token ablation agree */
    for (int r = 0; r < N; r++) {
      float am = 0.0f;
      for (int c = 0; c < d; c++) am = amax_upd(am, h->gq[(size_t)r * d + c]);
      h->dq[r] = qk_scale(h, am);
    }
  }
  for (size_t x = 0; x < Nd; x++) h->qhat[x] = qk_code(h, h->gq[x], h->dq[x / d]);
  return 0;
}

/* MX quantization of a row-major [T][d] FP32 matrix along channels, 32 per block. */
static int mx_rows(const float* X, int T, int d, double** vals, int** exps) {
  int nb = d / 32;
  *vals = xcalloc((size_t)T * d, sizeof(double));
  *exps = xcalloc((size_t)T * nb, sizeof(int));
  if (!*vals || !*exps) return -1;
  for (int t = 0; t < T; t++)
    for (int b = 0; b < nb; b++) {
      double am = 0.0;
      for (int c = b * 32; c < b * 32 + 32; c++) {
        double a = fabs((double)X[(size_t)t * d + c]);
        if (a > am) am = a;
      }
      int e = orc_e8m0_exponent(am);
      (*exps)[(size_t)t * nb + b] = e;
      for (int c = b * 32; c < b * 32 + 32; c++)
        (*vals)[(size_t)t * d + c] = orc_e2m1_decode(orc_e2m1_encode(ldexp((double)X[(size_t)t * d + c], -e)));
    }
  return 0;
}

static int head_setup(head_t* h, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      int in_fp16, int N, int M, int d, unsigned flags) {
  memset(h, 0, sizeof(*h));
  init_tables(); /* filled once here, before any parallel region reads them */
  if (N < 1 || M < 1 || (d != 64 && d != 128)) return -1;
  h->N = N; h->M = M; h->d = d; h->flags = flags;
  h->nqb = (N + ORC_BQ - 1) / ORC_BQ;
  h->nkt = (M + ORC_BK - 1) / ORC_BK;
  h->Qf = xcalloc((size_t)N * d, sizeof(float));
  h->Kf = xcalloc((size_t)M * d, sizeof(float));
  h->Vf = xcalloc((size_t)M * d, sizeof(float));
  if (!h->Qf || !h->Kf || !h->Vf) return -1;
  widen(q, in_fp16, (size_t)N * d, h->Qf);
  widen(k, in_fp16, (size_t)M * d, h->Kf);
  widen(v, in_fp16, (size_t)M * d, h->Vf);
  if (setup_k(h) || setup_v(h) || setup_q(h)) return -1;
  if (flags & ORC_MXFP4) {
    if (mx_rows(h->gq, N, d, &h->qx, &h->qe) || mx_rows(h->gk, M, d, &h->kx, &h->ke)) return -1;
  }
  return 0;
}

/* Step 6: Delta S_i[t] = q_i . gamma(K)[t] ([SA2] "Smoothing Q": the GEMV correction, a
 * 1 x b_k row per (i, j) broadcast over the block's rows).  Reading: it is taken from the
 * unquantized FP32 gamma(K) (FP64 gamma(K) in identity mode) and summed in FP64 in channel
 * order, which keeps the decomposition exact as the page states. */
static void delta_s_row(const head_t* h, int i, double* ds) {
  int d = h->d;
  const float* qm = h->qmean + (size_t)i * d;
  for (int t = 0; t < h->M; t++) {
    double s = 0.0;
    if (h->flags & ORC_QK_IDENTITY)
      for (int c = 0; c < d; c++) s += (double)qm[c] * h->gkd[(size_t)t * d + c];
    else
      for (int c = 0; c < d; c++) s += (double)qm[c] * (double)h->gk[(size_t)t * d + c];
    ds[t] = s;
  }
}

/* The unscaled score of (row r, key t) before Delta S: the dequantized quantized product. */
static double qk_term(const head_t* h, int r, int t) {
  int d = h->d;
  if (h->flags & ORC_QK_IDENTITY) {
    double s = 0.0;
    for (int c = 0; c < d; c++) s += h->gqd[(size_t)r * d + c] * h->gkd[(size_t)t * d + c];
    return s;
  }
  if (h->flags & ORC_MXFP4) {
    /* S = sum over 32-channel blocks of X_Q X_K (Q^ . K^)_blk  (exact in FP64) */
    int nb = d / 32;
    double s = 0.0;
    for (int b = 0; b < nb; b++) {
      double p = 0.0;
      for (int c = b * 32; c < b * 32 + 32; c++) p += h->qx[(size_t)r * d + c] * h->kx[(size_t)t * d + c];
      s += ldexp(p, h->qe[(size_t)r * nb + b] + h->ke[(size_t)t * nb + b]);
    }
    return s;
  }
  if (h->flags & ORC_QK_E4M3) {
    /* exact in FP64: each product has at most 8 significant bits between 2^-18 and 2^18 */
    double acc = 0.0;
    for (int c = 0; c < d; c++)
      acc += qk_value(h, h->qhat[(size_t)r * d + c]) * qk_value(h, h->khat[(size_t)t * d + c]);
    return acc * (double)h->dq[r] * (double)h->dk_key[t];
  }
  long acc = 0; /* exact integer dot product (|acc| <= 127*127*128 < 2^31) */
  for (int c = 0; c < d; c++) acc += (long)h->qhat[(size_t)r * d + c] * (long)h->khat[(size_t)t * d + c];
  return (double)acc * (double)h->dq[r] * (double)h->dk_key[t];
}

/* P~ -> the value of P^ entering the P~V product (static scale, [SA2] "FP8 Quantization":
 * P^ = E4M3(448 * P~)). */
static double quant_p(const head_t* h, double p) {
  if (h->flags & ORC_PV_IDENTITY) return h->pscale * p;
  if (h->flags & ORC_PV_E5M2) return orc_e5m2_decode(orc_e5m2_encode(h->pscale * p));
  if (h->flags & ORC_PV_INT8) {
    double y = nearbyint(h->pscale * p);
    return y > 127.0 ? 127.0 : y;
  }
  return orc_e4m3_decode(orc_e4m3_encode(h->pscale * p));
}

/* The causal mask: key t is visible to query row r iff t <= r + off.  causal = 1 aligns the
 * first query with the first key (off = 0; the pages' reference code masks the upper
 * triangle of the N x M score matrix); causal = 2 aligns the last query with the last key
 * (off = M - N, the reading of K and V as a cache of M >= N earlier tokens that the N queries
 * follow; needs N <= M so that no row is empty).  Returns -1 for other values. */
static int causal_offset(int causal, int N, int M, int* off) {
  if (causal == 0 || causal == 1) { *off = 0; return 0; }
  if (causal == 2 && N <= M) { *off = M - N; return 0; }
  return -1;
}

/* ---- rounding-decision margins (a diagnostic, not part of the method) ----
 * A quantizer's output code is decided by comparing its input with the midpoints between
 * adjacent representable values (and, for an E8M0 block scale, the block maximum with
 * 6 * 2^e).  The oracle decides in FP64 from exact exponentials; a kernel decides in FP32
 * from its own exp2, so an input within a few FP32 ulps of such a boundary may land on the
 * other side there, and both codes are correct roundings of the method's value.  These
 * helpers say whether x lies within relative distance eps of a boundary. */
static int near_rel(double x, double b, double eps) { return fabs(x - b) <= eps * fabs(b); }

/* The gap between the two E4M3 values around y when y lies within relative eps of their
 * midpoint (the change of the code's value should it round the other way), else 0. */
static double e4m3_tie_step(double y, double eps) {
  if (!(y > 0.0) || y >= 448.0) return 0.0;
  uint8_t c = orc_e4m3_encode(y);
  double v = orc_e4m3_decode(c);
  double w = v <= y ? orc_e4m3_decode((uint8_t)(c + 1)) : orc_e4m3_decode((uint8_t)(c - 1));
  return near_rel(y, 0.5 * (v + w), eps) ? fabs(w - v) : 0.0;
}

/* The same for E2M1 (midpoints of the value set and the gaps around them). */
static double e2m1_tie_step(double y, double eps) {
  static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  static const double gap[7] = {0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0};
  for (int i = 0; i < 7; i++)
    if (near_rel(fabs(y), mid[i], eps)) return gap[i];
  return 0.0;
}

/* Per-row margin bookkeeping: the count of near-boundary decisions, and a bound on how far
 * the row's output moves if every one of them rounds the other way -- the change of each
 * affected P^ value times the largest dequantized V value of its key, carried through the
 * tile loop like O (scaled by alpha, divided by l at the end). */
typedef struct { int count; double mass; } margin_t;

/* The score error a kernel may make under the E4M3 QK knob when its matrix core sums each
 * 64-channel step of Q^ K^ with an error of at most qk_step_err times the step's largest product
 * of code values: sum over the steps of that, times dQ dK sm_scale (natural-log units, so that
 * exp turns it into the same relative error of P~). */
static double qk_score_err(const head_t* h, int r, int t, double sm_scale, double qk_step_err) {
  int d = h->d;
  double e = 0.0;
  for (int c0 = 0; c0 < d; c0 += 64) {
    double mx = 0.0;
    for (int c = c0; c < c0 + 64; c++) {
      double p = fabs(qk_value(h, h->qhat[(size_t)r * d + c]) * qk_value(h, h->khat[(size_t)t * d + c]));
      if (p > mx) mx = p;
    }
    e += mx;
  }
  return qk_step_err * e * (double)h->dq[r] * (double)h->dk_key[t] * sm_scale;
}

/* Steps 7-8 for one row: the tile loop and the epilogue.  With mg != NULL, *ties and *bound
 * receive the row's near-boundary decisions (inputs within relative tie_eps of a rounding
 * boundary) and the bound on the output change they can cause. */
static void forward_row(const head_t* h, int r, int causal, int off, double sm_scale, const double* ds,
                        double* S, double* Pt, double* Ph, double* R, double* out, double tie_eps,
                        double qk_step_err, int* ties, double* bound) {
  margin_t mg = {0, 0.0};
  const int track = ties != NULL || bound != NULL;
  /* score errors of the keys of this tile and the largest of the keys seen so far (the running
   * maximum carries at most that), when the E4M3 QK kernel model is asked for */
  const int qk_err = track && (h->flags & ORC_QK_E4M3) && qk_step_err > 0.0;
  double E[ORC_BK], emax = 0.0;
  int d = h->d, M = h->M;
  double m = -INFINITY, l = 0.0;
  for (int c = 0; c < d; c++) out[c] = 0.0;
  for (int j = 0; j < h->nkt; j++) {
    int t0 = j * ORC_BK;
    /* Causal: a tile whose first key is past row r is fully masked for this row; with its
     * row maximum at -inf it leaves m, l and O unchanged, so it is not visited. */
    if (causal && t0 > r + off) break;
    int t1 = t0 + ORC_BK < M ? t0 + ORC_BK : M;
    int n = t1 - t0;
    double mt = -INFINITY;
    for (int x = 0; x < n; x++) {
      int t = t0 + x;
      if (causal && t > r + off) { S[x] = -INFINITY; continue; }
      S[x] = (qk_term(h, r, t) + ds[t]) * sm_scale; /* [SA2 Alg. 1] S = deq(QK) + Delta S */
      if (S[x] > mt) mt = S[x];
      if (qk_err) {
        E[x] = qk_score_err(h, r, t, sm_scale, qk_step_err);
        if (E[x] > emax) emax = E[x];
      }
    }
    /* Online softmax ([SA2 Alg. 1] step 3; [QA] datapath): running max, then exp. */
    double mnew = mt > m ? mt : m;
    double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
    double sum = 0.0;
    for (int x = 0; x < n; x++) {
      Pt[x] = (S[x] == -INFINITY) ? 0.0 : exp(S[x] - mnew);
      sum += Pt[x];
    }
    /* Reading: l accumulates the unquantized P~ (the online softmax precedes the cast). */
    l = alpha * l + sum;
    mg.mass *= alpha;
    if (h->flags & ORC_MXFP4) {
      /* P~ in E2M1 with one E8M0 scale per 32 keys of the row (2 blocks per 64-key tile);
       * R = sum_blk X_P X_V (P^ . V^)_blk. */
      /* Two-level knob ([SA3] "Two-Level Quantization for the Attention Map P"): level one
       * divides the row's P~ of this tile by an FP32 factor s1 taken from the row maximum
       * (which is exp(rowmax S - m), the softmax's own maximum), level two is the block
       * quantizer above, and the tile's product is multiplied back by s1.  Reading: the pages
       * send the row maximum to 448 * 6 because their block scales are E4M3; with E8M0 block
       * scales any power of two in s1 is absorbed by the block scale, so only the mantissa of
       * the target matters, and 448 * 6 = 1.3125 * 2^11 would put the maximum at 5.25 times
       * its block scale, off the E2M1 grid.  The target kept is 6, the largest E2M1 value,
       * which is what the pages' choice achieves for their format: s1 = rowmax / 6. */
      /* P2 = P~ / s1 is formed as 6 (P~ / rowmax), so that the row maximum is 6 exactly. */
      const int two = (h->flags & ORC_MX_P_TWO_LEVEL) != 0;
      double pm = 0.0;
      if (two)
        for (int x = 0; x < n; x++) if (Pt[x] > pm) pm = Pt[x];
      /* pm > 0: a visited tile holds at least one visible key of the row */
      const double s1 = two ? pm / 6.0 : 1.0;
      for (int x = 0; x < n; x++) Pt[x] = two ? 6.0 * (Pt[x] / pm) : Pt[x]; /* l already summed */
      for (int c = 0; c < d; c++) R[c] = 0.0;
      for (int b0 = 0; b0 < n; b0 += 32) {
        int b1 = b0 + 32 < n ? b0 + 32 : n;
        double am = 0.0;
        for (int x = b0; x < b1; x++) if (Pt[x] > am) am = Pt[x];
        int ep = orc_e8m0_exponent(am);
        for (int x = b0; x < b1; x++) Ph[x] = orc_e2m1_decode(orc_e2m1_encode(ldexp(Pt[x], -ep)));
        int vb = (t0 + b0) / 32;
        if (track) {
          /* the largest dequantized V' value of key x, over channels */
          double blk = 0.0;
          for (int x = b0; x < b1; x++) {
            double vm = 0.0;
            for (int c = 0; c < d; c++) {
              double a = fabs(ldexp(h->vx[(size_t)(t0 + x) * d + c], h->ve[(size_t)vb * d + c]));
              if (a > vm) vm = a;
            }
            double st = e2m1_tie_step(ldexp(Pt[x], -ep), tie_eps);
            mg.count += st > 0.0;
            blk += st * vm;
            S[x] = vm; /* kept for the exponent decision below (S is not read again) */
          }
          /* the block exponent: a near-boundary maximum may move the whole block one octave,
           * each value by at most one top step (2) of the coarser grid (the two-level row
           * maximum is exactly 6 by construction, not a rounded input) */
          if (am > 0.0 && !(two && am == 6.0) &&
              (near_rel(am, 6.0 * ldexp(1.0, ep), tie_eps) || near_rel(am, 6.0 * ldexp(1.0, ep - 1), tie_eps))) {
            mg.count++;
            for (int x = b0; x < b1; x++) blk += 4.0 * S[x];
          }
          mg.mass += s1 * ldexp(blk, ep);
        }
        for (int c = 0; c < d; c++) {
          double p = 0.0;
          for (int x = b0; x < b1; x++) p += Ph[x] * h->vx[(size_t)(t0 + x) * d + c];
          R[c] += ldexp(p, ep + h->ve[(size_t)vb * d + c]);
        }
      }
      for (int c = 0; c < d; c++) R[c] *= s1;
    } else {
      for (int x = 0; x < n; x++) Ph[x] = quant_p(h, Pt[x]);
      if (track && !(h->flags & (ORC_PV_IDENTITY | ORC_PV_E5M2 | ORC_PV_INT8)))
        for (int x = 0; x < n; x++) {
          double st = e4m3_tie_step(h->pscale * Pt[x], tie_eps + (qk_err ? E[x] + emax : 0.0));
          if (st == 0.0) continue;
          double vm = 0.0; /* the largest dequantized V value of the key (V^ times dV) */
          for (int c = 0; c < d; c++) {
            double a = fabs(h->vq[(size_t)(t0 + x) * d + c] * (double)h->dv[c]);
            if (a > vm) vm = a;
          }
          mg.count++;
          mg.mass += st * vm / h->pscale;
        }
      /* R = P^ V^ over this tile only (the per-tile inner accumulator). */
      for (int c = 0; c < d; c++) {
        double acc = 0.0;
        for (int x = 0; x < n; x++)
          if (Ph[x] != 0.0) acc += Ph[x] * h->vq[(size_t)(t0 + x) * d + c];
        R[c] = acc;
      }
    }
    /* Two-level accumulation ([SA2] "Two-Level Accumulation"): O = diag(alpha) O + R. */
    for (int c = 0; c < d; c++) out[c] = alpha * out[c] + R[c];
    m = mnew;
  }
  /* Epilogue ([SA2 Alg. 1] step 4): O / l / 448 * dV; V smoothing adds V_m back after
   * normalisation ([SA2] "Optional Smoothing of V": rows of P~/l sum to one). */
  for (int c = 0; c < d; c++) {
    double o = out[c] / l;
    if (!(h->flags & ORC_MXFP4)) o = o / h->pscale * (double)h->dv[c];
    out[c] = o + (double)h->vmean[c];
  }
  if (ties) *ties = mg.count;
  if (bound) *bound = mg.mass / l;
}

int orc_forward_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                     int N, int M, int d, int causal, double sm_scale, unsigned flags,
                     const int* rows, int nrows, double* out) {
  return orc_forward_head_ties(q, k, v, in_fp16, N, M, d, causal, sm_scale, flags, rows, nrows, out, 0.0, 0.0,
                               NULL, NULL);
}

int orc_forward_head_ties(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                          int N, int M, int d, int causal, double sm_scale, unsigned flags,
                          const int* rows, int nrows, double* out, double tie_eps, double qk_step_err,
                          int* ties, double* bound) {
  int off;
  if (!q || !k || !v || !out || nrows < 0) return -1;
  if (causal_offset(causal, N, M, &off)) return -1;
  if ((flags & ORC_MXFP4) && (flags & (ORC_QK_IDENTITY | ORC_PV_IDENTITY | ORC_PV_E5M2 | ORC_PV_INT8))) return -1;
  if ((flags & ORC_QK_E4M3) && (flags & (ORC_QK_IDENTITY | ORC_MXFP4))) return -1;
  if ((flags & ORC_MX_P_TWO_LEVEL) && !(flags & ORC_MXFP4)) return -1;
  if (!rows && nrows != N) return -1;
  head_t h;
  if (head_setup(&h, q, k, v, in_fp16, N, M, d, flags)) { head_free(&h); return -1; }
  for (int x = 0; x < nrows; x++) {
    int r = rows ? rows[x] : x;
    if (r < 0 || r >= N) { head_free(&h); return -1; }
  }
  /* Delta S rows for the blocks that hold requested rows. */
  char* need = xcalloc(h.nqb, 1);
  double** dsr = xcalloc(h.nqb, sizeof(double*));
  int fail = (!need || !dsr);
  for (int x = 0; !fail && x < nrows; x++) need[(rows ? rows[x] : x) / ORC_BQ] = 1;
  for (int i = 0; !fail && i < h.nqb; i++)
    if (need[i]) {
      dsr[i] = xcalloc(M, sizeof(double));
      if (!dsr[i]) { fail = 1; break; }
    }
  if (!fail) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < h.nqb; i++)
      if (need[i]) delta_s_row(&h, i, dsr[i]);
#pragma omp parallel
    {
      double* S = malloc(sizeof(double) * ORC_BK);
      double* Pt = malloc(sizeof(double) * ORC_BK);
      double* Ph = malloc(sizeof(double) * ORC_BK);
      double* R = malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 4)
      for (int x = 0; x < nrows; x++) {
        int r = rows ? rows[x] : x;
        forward_row(&h, r, causal, off, sm_scale, dsr[r / ORC_BQ], S, Pt, Ph, R, out + (size_t)x * d, tie_eps,
                    qk_step_err, ties ? ties + x : NULL, bound ? bound + x : NULL);
      }
      free(S); free(Pt); free(Ph); free(R);
    }
  }
  for (int i = 0; dsr && i < h.nqb; i++) free(dsr[i]);
  free(dsr);
  free(need);
  head_free(&h);
  return fail ? -1 : 0;
}

int orc_preprocess_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                        int N, int M, int d, unsigned flags,
                        float* kmean, float* vmean, int8_t* khat, float* dk,
                        uint8_t* vhat, float* dv, int8_t* qhat, float* dq,
                        float* qmean, double* ds) {
  if (!q || !k || !v) return -1;
  if (flags & ~(ORC_SMOOTH_V | ORC_NO_SMOOTH_K | ORC_NO_SMOOTH_Q | ORC_QK_PER_BLOCK | ORC_QK_E4M3)) return -1;
  head_t h;
  if (head_setup(&h, q, k, v, in_fp16, N, M, d, flags)) { head_free(&h); return -1; }
  if (kmean) memcpy(kmean, h.kmean, sizeof(float) * d);
  if (vmean) memcpy(vmean, h.vmean, sizeof(float) * d);
  if (khat) memcpy(khat, h.khat, (size_t)M * d);
  if (dk) { /* the scale of each (tile, group); with ORC_QK_PER_BLOCK all four are equal */
    if (flags & ORC_QK_PER_BLOCK) {
      for (int u = 0; u < h.nkt; u++)
        for (int g = 0; g < 4; g++) dk[(size_t)u * 4 + g] = h.dk_key[(size_t)u * ORC_BK];
    } else {
      memcpy(dk, h.dk_grp, sizeof(float) * 4 * h.nkt);
    }
  }
  if (vhat) memcpy(vhat, h.vhat, (size_t)M * d);
  if (dv) memcpy(dv, h.dv, sizeof(float) * d);
  if (qhat) memcpy(qhat, h.qhat, (size_t)N * d);
  if (dq) memcpy(dq, h.dq, sizeof(float) * N);
  if (qmean) memcpy(qmean, h.qmean, sizeof(float) * d * h.nqb);
  if (ds) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < h.nqb; i++) delta_s_row(&h, i, ds + (size_t)i * M);
  }
  head_free(&h);
  return 0;
}

/* The MX variant's quantized tensors of one head, as codes: the E2M1 code (sign << 3 |
 * magnitude index) of every element of gamma(Q) [N][d] and gamma(K) [M][d] with their E8M0
 * exponents per 32 channels [N][d/32], [M][d/32]; the codes of V' [M][d] with one exponent
 * per 32 tokens of each channel [ceil(M/32)][d] ([SA3] 3.4: 1x32 blocks along the reduction
 * dimension of each product).  The E2M1 decode is injective (signed zeros included), so the
 * codes are those the quantizer chose.  Any output may be NULL. */
int orc_preprocess_mx_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                           int N, int M, int d, unsigned flags,
                           uint8_t* qcode, int* qexp, uint8_t* kcode, int* kexp,
                           uint8_t* vcode, int* vexp) {
  if (!q || !k || !v) return -1;
  if (flags & ~(ORC_SMOOTH_V | ORC_NO_SMOOTH_K | ORC_NO_SMOOTH_Q)) return -1;
  head_t h;
  if (head_setup(&h, q, k, v, in_fp16, N, M, d, flags | ORC_MXFP4)) { head_free(&h); return -1; }
  int nb = d / 32, nvb = (M + 31) / 32;
  if (qcode) for (size_t x = 0; x < (size_t)N * d; x++) qcode[x] = orc_e2m1_encode(h.qx[x]);
  if (kcode) for (size_t x = 0; x < (size_t)M * d; x++) kcode[x] = orc_e2m1_encode(h.kx[x]);
  if (vcode) for (size_t x = 0; x < (size_t)M * d; x++) vcode[x] = orc_e2m1_encode(h.vx[x]);
  if (qexp) memcpy(qexp, h.qe, sizeof(int) * (size_t)N * nb);
  if (kexp) memcpy(kexp, h.ke, sizeof(int) * (size_t)M * nb);
  if (vexp) memcpy(vexp, h.ve, sizeof(int) * (size_t)nvb * d);
  head_free(&h);
  return 0;
}

/* Number of keys row r sees under the causal mask t <= r + off (at most M). */
static int visible(int r, int off, int M) { return r + off + 1 < M ? r + off + 1 : M; }

/* Textbook attention: softmax(Q K^T * sm_scale) V, FP64, row by row. */
static void exact_row(const double* qr, const double* K, const double* V, int M, int d, int lim,
                      double sm_scale, double* s, double* out) {
  double m = -INFINITY;
  for (int t = 0; t < lim; t++) {
    double a = 0.0;
    for (int c = 0; c < d; c++) a += qr[c] * K[(size_t)t * d + c];
    s[t] = a * sm_scale;
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int t = 0; t < lim; t++) { s[t] = exp(s[t] - m); l += s[t]; }
  for (int c = 0; c < d; c++) out[c] = 0.0;
  for (int t = 0; t < lim; t++)
    for (int c = 0; c < d; c++) out[c] += s[t] * V[(size_t)t * d + c];
  for (int c = 0; c < d; c++) out[c] /= l;
  (void)M;
}

int orc_exact_f64(const double* q, const double* k, const double* v, int N, int M, int d,
                  int causal, double sm_scale, double* out) {
  int off;
  if (!q || !k || !v || !out || N < 1 || M < 1 || d < 1) return -1;
  if (causal_offset(causal, N, M, &off)) return -1;
#pragma omp parallel
  {
    double* s = malloc(sizeof(double) * M);
#pragma omp for schedule(dynamic, 4)
    for (int r = 0; r < N; r++)
      exact_row(q + (size_t)r * d, k, v, M, d, causal ? visible(r, off, M) : M, sm_scale, s, out + (size_t)r * d);
    free(s);
  }
  return 0;
}

int orc_exact_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                   int N, int M, int d, int causal, double sm_scale,
                   const int* rows, int nrows, double* out) {
  int off;
  if (!q || !k || !v || !out || N < 1 || M < 1 || d < 1 || nrows < 0) return -1;
  if (causal_offset(causal, N, M, &off)) return -1;
  if (!rows && nrows != N) return -1;
  double* K = malloc(sizeof(double) * (size_t)M * d);
  double* V = malloc(sizeof(double) * (size_t)M * d);
  if (!K || !V) { free(K); free(V); return -1; }
  for (size_t i = 0; i < (size_t)M * d; i++) {
    K[i] = in_fp16 ? orc_fp16_to_f32(k[i]) : orc_bf16_to_f32(k[i]);
    V[i] = in_fp16 ? orc_fp16_to_f32(v[i]) : orc_bf16_to_f32(v[i]);
  }
  int bad = 0;
#pragma omp parallel
  {
    double* s = malloc(sizeof(double) * M);
    double* qr = malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 4)
    for (int x = 0; x < nrows; x++) {
      int r = rows ? rows[x] : x;
      if (r < 0 || r >= N) { bad = 1; continue; }
      for (int c = 0; c < d; c++)
        qr[c] = in_fp16 ? orc_fp16_to_f32(q[(size_t)r * d + c]) : orc_bf16_to_f32(q[(size_t)r * d + c]);
      exact_row(qr, K, V, M, d, causal ? visible(r, off, M) : M, sm_scale, s, out + (size_t)x * d);
    }
    free(s);
    free(qr);
  }
  free(K);
  free(V);
  return bad ? -1 : 0;
}
