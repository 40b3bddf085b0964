/*
 * sagebwd_oracle.c -- CPU oracle for SageBwd, the trainable 8-bit attention: the forward
 * with the row log-sum-exp, and the backward.
 *
 * TEST INFRASTRUCTURE ONLY: the plain, slow reference the GPU path is checked against (see
 * sage_oracle.h).  It shares no code with the HIP library.
 *
 * Source: "SageAttention3: Microscaling FP4 Attention for Inference and An Exploration of
 * 8-Bit Training" (structured summary of arXiv 2505.11594), sections "SageBwd Forward Pass:
 * INT8 Quantization for Training" and "SageBwd Backward Pass and the Critical dOV^T
 * Decision".  In their notation, per query block i (128 rows) and key block j (64 keys):
 *
 *   forward   K <- K - mean(K);  s_X = max|X| / 127, X^ = X / s_X per block for Q, K, V
 *             S = Q^ K^T s_Q s_K;  m, P = exp(S - m), l as in the online softmax
 *             s_P = exp(rowmax(S_ij) - m_ij) / 127 per row of the block, P^ = P / s_P
 *             O = diag(e^{m_old - m}) O + P^ V^ s_P s_V;   out = O / l,  L = m + ln l
 *   backward  D = rowsum(dO o O);  S recomputed as above, P = exp(S - L)
 *             dV_j += P^^T dO^_i s_P s_dO          (P, dO per block, INT8)
 *             dP    = dO_i V_j^T                    (16-bit inputs, kept unquantized)
 *             dS    = P o (dP - D_i);  dS^ per block (INT8)
 *             dQ_i += dS^ K^_j s_dS s_K,  dK_j += dS^^T Q^_i s_dS s_Q
 *             dQ_i += rowsum(dS) k^T   (the smoothing-K correction, FP32 on the pages)
 *
 * Readings (where the pages are silent):
 *   - scaled scores: S carries sm_scale (S = sm_scale Q K^T), so dQ and dK carry it too;
 *   - blocks: 128 queries, 64 keys (the forward kernel's tiles); a block's scale covers its
 *     valid rows and keys only (masked pairs have P = dS = 0);
 *   - INT8 quantizer: the INT8 path's (scale = max(amax, 1e-8) / 127 in FP32, code = round
 *     half to even of the FP32 quotient, clamped to +-127); P^ and dS^ round the FP64 value;
 *   - a block whose P (or dS) is all zero gets scale 0 and codes 0;
 *   - L is the log-sum-exp of the scores actually used, after K smoothing (it differs
 *     from that of Q K^T by sm_scale q . k per row; out and the gradients do not).
 * Everything not quantized is FP64.
 */
#include "sage_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define SB_BQ 128
#define SB_BK 64

static float sb_widen(uint16_t h, int fp16) { return fp16 ? orc_fp16_to_f32(h) : orc_bf16_to_f32(h); }

/* The INT8 path's quantizer (scale in FP32 from the block amax; RNE of the FP32 quotient). */
static float sb_scale(float amax) {
  float a = amax > 1e-8f ? amax : 1e-8f;
  return a / 127.0f;
}
static int sb_code(float x, float s) {
  float y = nearbyintf(x / s);
  if (!(y == y)) return 0;
  if (y > 127.0f) y = 127.0f;
  if (y < -127.0f) y = -127.0f;
  return (int)y;
}
/* RNE of an FP64 value against an FP64 scale (P^ and dS^); scale 0 -> 0. */
static double sb_code64(double x, double s) {
  if (!(s > 0.0)) return 0.0;
  double y = nearbyint(x / s);
  if (y > 127.0) y = 127.0;
  if (y < -127.0) y = -127.0;
  return y;
}

typedef struct {
  int N, M, d, nqb, nkt, causal, off, identity, dp_int8;
  double sm;
  float *Q, *K, *V, *dO; /* widened; K smoothed                                     */
  float *kmean;          /* [d]                                                      */
  double *qv, *kv, *vv;  /* the values entering the products: codes, or FP32 values  */
  double *sq, *sk, *sv;  /* block scales (1 in identity mode)                        */
  double *dov, *sdo;     /* dO entering P^T dO: codes per 128-row block, or values   */
} sb_t;

static void sb_free(sb_t* h) {
  free(h->Q); free(h->K); free(h->V); free(h->dO); free(h->kmean);
  free(h->qv); free(h->kv); free(h->vv); free(h->sq); free(h->sk); free(h->sv);
  free(h->dov); free(h->sdo);
  memset(h, 0, sizeof(*h));
}

/* Quantize rows [r0, r1) of X [T][d] as one block: values (codes or identity) and scale. */
static void sb_block(const float* X, int r0, int r1, int d, int identity, double* vals, double* scale) {
  float am = 0.0f;
  for (int r = r0; r < r1; r++)
    for (int c = 0; c < d; c++) {
      float a = fabsf(X[(size_t)r * d + c]);
      if (a > am) am = a;
    }
  if (identity) {
    *scale = 1.0;
    for (int r = r0; r < r1; r++)
      for (int c = 0; c < d; c++) vals[(size_t)r * d + c] = (double)X[(size_t)r * d + c];
    return;
  }
  float s = sb_scale(am);
  *scale = (double)s;
  for (int r = r0; r < r1; r++)
    for (int c = 0; c < d; c++) vals[(size_t)r * d + c] = (double)sb_code(X[(size_t)r * d + c], s);
}

static int sb_setup(sb_t* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                    int in_fp16, int N, int M, int d, int causal, double sm, unsigned flags) {
  memset(h, 0, sizeof(*h));
  if (N < 1 || M < 1 || (d != 64 && d != 128)) return -1;
  if (causal < 0 || causal > 2 || (causal == 2 && N > M)) return -1;
  h->N = N; h->M = M; h->d = d; h->causal = causal; h->off = causal == 2 ? M - N : 0;
  h->nqb = (N + SB_BQ - 1) / SB_BQ;
  h->nkt = (M + SB_BK - 1) / SB_BK;
  h->identity = (flags & ORC_SB_IDENTITY) != 0;
  h->dp_int8 = (flags & ORC_SB_DP_INT8) != 0;
  h->sm = sm;
  size_t Nd = (size_t)N * d, Md = (size_t)M * d;
  h->Q = malloc(Nd * sizeof(float)); h->K = malloc(Md * sizeof(float)); h->V = malloc(Md * sizeof(float));
  h->kmean = calloc(d, sizeof(float));
  h->qv = malloc(Nd * sizeof(double)); h->kv = malloc(Md * sizeof(double)); h->vv = malloc(Md * sizeof(double));
  h->sq = malloc(h->nqb * sizeof(double)); h->sk = malloc(h->nkt * sizeof(double));
  h->sv = malloc(h->nkt * sizeof(double));
  if (!h->Q || !h->K || !h->V || !h->kmean || !h->qv || !h->kv || !h->vv || !h->sq || !h->sk || !h->sv) return -1;
  for (size_t x = 0; x < Nd; x++) h->Q[x] = sb_widen(q[x], in_fp16);
  for (size_t x = 0; x < Md; x++) {
    h->K[x] = sb_widen(k[x], in_fp16);
    h->V[x] = sb_widen(v[x], in_fp16);
  }
  /* smoothing K: the token mean in the INT8 path's pinned order (64-token chunks in token
   * order, chunk sums in order, FP64, one division, rounded to FP32) */
  if (!(flags & ORC_SB_NO_SMOOTH_K)) {
    for (int c = 0; c < d; c++) {
      double tot = 0.0;
      for (int u0 = 0; u0 < M; u0 += SB_BK) {
        double part = 0.0;
        for (int t = u0; t < M && t < u0 + SB_BK; t++) part += (double)h->K[(size_t)t * d + c];
        tot += part;
      }
      h->kmean[c] = (float)(tot / (double)M);
    }
    /* FP32 subtraction, as the quantizer sees it; identity mode keeps K - k exact (FP64) so
     * that the shift leaves the softmax exactly unchanged */
    if (h->identity)
      for (size_t x = 0; x < Md; x++) h->kv[x] = (double)h->K[x] - (double)h->kmean[x % d];
    for (size_t x = 0; x < Md; x++) h->K[x] = h->K[x] - h->kmean[x % d];
  }
  for (int i = 0; i < h->nqb; i++) {
    int r1 = (i + 1) * SB_BQ < N ? (i + 1) * SB_BQ : N;
    sb_block(h->Q, i * SB_BQ, r1, d, h->identity, h->qv, &h->sq[i]);
  }
  const int exact_k = h->identity && !(flags & ORC_SB_NO_SMOOTH_K);
  for (int j = 0; j < h->nkt; j++) {
    int t1 = (j + 1) * SB_BK < M ? (j + 1) * SB_BK : M;
    if (exact_k)
      h->sk[j] = 1.0; /* kv already holds the FP64 K - k */
    else
      sb_block(h->K, j * SB_BK, t1, d, h->identity, h->kv, &h->sk[j]);
    sb_block(h->V, j * SB_BK, t1, d, h->identity, h->vv, &h->sv[j]);
  }
  if (dout) {
    h->dO = malloc(Nd * sizeof(float));
    h->dov = malloc(Nd * sizeof(double));
    h->sdo = malloc(h->nqb * sizeof(double));
    if (!h->dO || !h->dov || !h->sdo) return -1;
    for (size_t x = 0; x < Nd; x++) h->dO[x] = sb_widen(dout[x], in_fp16);
    for (int i = 0; i < h->nqb; i++) {
      int r1 = (i + 1) * SB_BQ < N ? (i + 1) * SB_BQ : N;
      sb_block(h->dO, i * SB_BQ, r1, d, h->identity, h->dov, &h->sdo[i]);
    }
  }
  return 0;
}

/* key t visible to row r */
static int sb_vis(const sb_t* h, int r, int t) { return !h->causal || t <= r + h->off; }

/* the scaled score of (r, t): S = Q^ K^T s_Q s_K sm_scale (exact FP64 dot of the codes) */
static double sb_score(const sb_t* h, int r, int t) {
  int d = h->d;
  double acc = 0.0;
  for (int c = 0; c < d; c++) acc += h->qv[(size_t)r * d + c] * h->kv[(size_t)t * d + c];
  return acc * h->sq[r / SB_BQ] * h->sk[t / SB_BK] * h->sm;
}

/* Forward of one row ("SageBwd Forward Pass"): out[d], *lse. */
static void sb_forward_row(const sb_t* h, int r, double* S, double* out, double* lse) {
  int d = h->d;
  double m = -INFINITY, l = 0.0;
  for (int c = 0; c < d; c++) out[c] = 0.0;
  for (int j = 0; j < h->nkt; j++) {
    int t0 = j * SB_BK, t1 = t0 + SB_BK < h->M ? t0 + SB_BK : h->M;
    double rm = -INFINITY;
    for (int t = t0; t < t1; t++) {
      S[t - t0] = sb_vis(h, r, t) ? sb_score(h, r, t) : -INFINITY;
      if (S[t - t0] > rm) rm = S[t - t0];
    }
    if (rm == -INFINITY) continue; /* no visible key in this block: nothing to add */
    double mn = m > rm ? m : rm;
    double alpha = exp(m - mn); /* 0 on the first visible block */
    double ps = 0.0;
    /* per-token P scale from the block's row max (the softmax max, reused) */
    double sp = h->identity ? 1.0 : exp(rm - mn) / 127.0;
    for (int c = 0; c < d; c++) out[c] *= alpha;
    for (int t = t0; t < t1; t++) {
      if (S[t - t0] == -INFINITY) continue;
      double p = exp(S[t - t0] - mn);
      ps += p;
      double ph = h->identity ? p : sb_code64(p, sp) * sp;
      for (int c = 0; c < d; c++) out[c] += ph * h->vv[(size_t)t * d + c] * h->sv[j];
    }
    l = alpha * l + ps;
    m = mn;
  }
  for (int c = 0; c < d; c++) out[c] /= l;
  *lse = m + log(l);
}

int orc_sagebwd_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16, int N, int M, int d,
                        int causal, double sm_scale, unsigned flags, double* out, double* lse) {
  if (!q || !k || !v || !out || !lse) return -1;
  if (flags & ~(ORC_SB_IDENTITY | ORC_SB_NO_SMOOTH_K | ORC_SB_DP_INT8)) return -1;
  sb_t h;
  if (sb_setup(&h, q, k, v, NULL, in_fp16, N, M, d, causal, sm_scale, flags)) { sb_free(&h); return -1; }
  int fail = 0;
#pragma omp parallel
  {
    double* S = malloc(sizeof(double) * SB_BK);
    if (!S) fail = 1;
#pragma omp for schedule(dynamic, 8)
    for (int r = 0; r < N; r++)
      if (S) sb_forward_row(&h, r, S, out + (size_t)r * d, lse + r);
    free(S);
  }
  sb_free(&h);
  return fail ? -1 : 0;
}

/* The per-block backward quantities of (query block i, key block j): P (exact), P^ values
 * with its scale folded in, dS (exact) and dS^ values with its scale folded in; returns 0 if
 * the block has no visible pair.  Arrays are [SB_BQ][SB_BK], row-major. */
static int sb_pair(const sb_t* h, int i, int j, const double* L, const double* D, double* P, double* Ph,
                   double* dS, double* dSh) {
  int d = h->d, r0 = i * SB_BQ, r1 = r0 + SB_BQ < h->N ? r0 + SB_BQ : h->N;
  int t0 = j * SB_BK, t1 = t0 + SB_BK < h->M ? t0 + SB_BK : h->M;
  int any = 0;
  double pmax = 0.0, dsmax = 0.0;
  for (int r = r0; r < r1; r++)
    for (int t = t0; t < t1; t++) {
      int x = (r - r0) * SB_BK + (t - t0);
      if (!sb_vis(h, r, t)) {
        P[x] = dS[x] = 0.0;
        continue;
      }
      any = 1;
      P[x] = exp(sb_score(h, r, t) - L[r]);
      double dp = 0.0; /* dP = dO V^T: unquantized (16-bit inputs), or the INT8 ablation */
      if (h->dp_int8)
        for (int c = 0; c < d; c++)
          dp += h->dov[(size_t)r * d + c] * h->vv[(size_t)t * d + c] * h->sdo[i] * h->sv[j];
      else
        for (int c = 0; c < d; c++) dp += (double)h->dO[(size_t)r * d + c] * (double)h->V[(size_t)t * d + c];
      dS[x] = P[x] * (dp - D[r]);
      if (P[x] > pmax) pmax = P[x];
      if (fabs(dS[x]) > dsmax) dsmax = fabs(dS[x]);
    }
  if (!any) return 0;
  double sp = pmax / 127.0, sds = dsmax / 127.0;
  for (int r = r0; r < r1; r++)
    for (int t = t0; t < t1; t++) {
      int x = (r - r0) * SB_BK + (t - t0);
      Ph[x] = h->identity ? P[x] : sb_code64(P[x], sp) * sp;
      dSh[x] = h->identity ? dS[x] : sb_code64(dS[x], sds) * sds;
    }
  return 1;
}

int orc_sagebwd_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         int in_fp16, int N, int M, int d, int causal, double sm_scale, unsigned flags,
                         double* out, double* lse, double* dq, double* dk, double* dv) {
  if (!q || !k || !v || !dout || !out || !lse || !dq || !dk || !dv) return -1;
  if (orc_sagebwd_forward(q, k, v, in_fp16, N, M, d, causal, sm_scale, flags, out, lse)) return -1;
  sb_t h;
  if (sb_setup(&h, q, k, v, dout, in_fp16, N, M, d, causal, sm_scale, flags)) { sb_free(&h); return -1; }
  double* D = malloc(sizeof(double) * N);
  int fail = !D;
  for (int r = 0; !fail && r < N; r++) { /* D = rowsum(dO o O) */
    double s = 0.0;
    for (int c = 0; c < d; c++) s += (double)h.dO[(size_t)r * d + c] * out[(size_t)r * d + c];
    D[r] = s;
  }
  memset(dq, 0, sizeof(double) * N * d);
  memset(dk, 0, sizeof(double) * M * d);
  memset(dv, 0, sizeof(double) * M * d);
  if (!fail) {
    /* dK, dV: one key block at a time over the query blocks in order */
#pragma omp parallel
    {
      size_t bs = (size_t)SB_BQ * SB_BK;
      double* P = malloc(sizeof(double) * bs * 4);
      if (!P) fail = 1;
#pragma omp for schedule(dynamic, 1)
      for (int j = 0; j < h.nkt; j++) {
        if (!P) continue;
        double *Ph = P + bs, *dS = P + 2 * bs, *dSh = P + 3 * bs;
        int t0 = j * SB_BK, t1 = t0 + SB_BK < M ? t0 + SB_BK : M;
        for (int i = 0; i < h.nqb; i++) {
          if (!sb_pair(&h, i, j, lse, D, P, Ph, dS, dSh)) continue;
          int r0 = i * SB_BQ, r1 = r0 + SB_BQ < N ? r0 + SB_BQ : N;
          for (int t = t0; t < t1; t++)
            for (int c = 0; c < d; c++) {
              double sv = 0.0, sk = 0.0;
              for (int r = r0; r < r1; r++) {
                int x = (r - r0) * SB_BK + (t - t0);
                sv += Ph[x] * h.dov[(size_t)r * d + c];
                sk += dSh[x] * h.qv[(size_t)r * d + c];
              }
              dv[(size_t)t * d + c] += sv * h.sdo[i];
              dk[(size_t)t * d + c] += sk * h.sq[i] * sm_scale;
            }
        }
      }
      free(P);
    }
    /* dQ: one query block at a time over the key blocks in order, plus the smoothing term */
#pragma omp parallel
    {
      size_t bs = (size_t)SB_BQ * SB_BK;
      double* P = malloc(sizeof(double) * bs * 4);
      if (!P) fail = 1;
#pragma omp for schedule(dynamic, 1)
      for (int i = 0; i < h.nqb; i++) {
        if (!P) continue;
        double *Ph = P + bs, *dS = P + 2 * bs, *dSh = P + 3 * bs;
        int r0 = i * SB_BQ, r1 = r0 + SB_BQ < N ? r0 + SB_BQ : N;
        double rs[SB_BQ];
        for (int r = 0; r < SB_BQ; r++) rs[r] = 0.0;
        for (int j = 0; j < h.nkt; j++) {
          if (!sb_pair(&h, i, j, lse, D, P, Ph, dS, dSh)) continue;
          int t0 = j * SB_BK, t1 = t0 + SB_BK < M ? t0 + SB_BK : M;
          for (int r = r0; r < r1; r++) {
            for (int c = 0; c < d; c++) {
              double s = 0.0;
              for (int t = t0; t < t1; t++) s += dSh[(r - r0) * SB_BK + (t - t0)] * h.kv[(size_t)t * d + c];
              dq[(size_t)r * d + c] += s * h.sk[j] * sm_scale;
            }
            for (int t = t0; t < t1; t++) rs[r - r0] += dS[(r - r0) * SB_BK + (t - t0)];
          }
        }
        for (int r = r0; r < r1; r++)
          for (int c = 0; c < d; c++) dq[(size_t)r * d + c] += sm_scale * rs[r - r0] * (double)h.kmean[c];
      }
      free(P);
    }
  }
  free(D);
  sb_free(&h);
  return fail ? -1 : 0;
}

/* The quantized tensors of one head as the SageBwd forward and backward use them: INT8
 * codes of Q [N][d] and dO [N][d] per 128-row block, of smoothed K and of V [M][d] per 64-key
 * block, with their FP32 scales [ceil(N/128)] / [ceil(M/64)], and the K mean [d].  dout and
 * its outputs may be NULL.  flags: ORC_SB_NO_SMOOTH_K. */
int orc_sagebwd_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         int in_fp16, int N, int M, int d, unsigned flags, int8_t* qcode, float* sq,
                         int8_t* kcode, float* sk, int8_t* vcode, float* sv, int8_t* docode, float* sdo,
                         float* kmean) {
  if (!q || !k || !v) return -1;
  if (flags & ~ORC_SB_NO_SMOOTH_K) return -1;
  sb_t h;
  if (sb_setup(&h, q, k, v, dout, in_fp16, N, M, d, 0, 1.0, flags)) { sb_free(&h); return -1; }
  for (size_t x = 0; x < (size_t)N * d; x++) {
    if (qcode) qcode[x] = (int8_t)h.qv[x];
    if (docode && dout) docode[x] = (int8_t)h.dov[x];
  }
  for (size_t x = 0; x < (size_t)M * d; x++) {
    if (kcode) kcode[x] = (int8_t)h.kv[x];
    if (vcode) vcode[x] = (int8_t)h.vv[x];
  }
  for (int i = 0; i < h.nqb; i++) {
    if (sq) sq[i] = (float)h.sq[i];
    if (sdo && dout) sdo[i] = (float)h.sdo[i];
  }
  for (int j = 0; j < h.nkt; j++) {
    if (sk) sk[j] = (float)h.sk[j];
    if (sv) sv[j] = (float)h.sv[j];
  }
  if (kmean) memcpy(kmean, h.kmean, sizeof(float) * d);
  sb_free(&h);
  return 0;
}
