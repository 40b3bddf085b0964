/*
 * sage_oracle.h -- CPU oracle for the SageAttention2-style quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the plain, slow reference that the GPU
 * path is checked against.  It is called from the test-suite, from the package's smoke
 * check and from the benchmark's CPU-baseline leg -- never from the product path.  It
 * shares no code with the HIP library.
 *
 * Sources (the pages this follows, cited by title and section):
 *   [SA2]  "SageAttention2 Technical Report: Accurate 4 Bit Attention for Plug-and-play
 *          Inference Acceleration" (structured summary of arXiv 2411.10958), section 3.4:
 *          "Smoothing Q", "Per-Thread INT4 Quantization", "FP8 Quantization for P~V",
 *          "Two-Level Accumulation", "Optional Smoothing of V", "The Complete Algorithm
 *          (Algorithm 1)".
 *   [SA2R] "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and
 *          Per-thread INT4 Quantization" (paper review blog), "core formulas" and the
 *          forward-pass algorithm listing.
 *   [SA3]  "SageAttention3 ..." summary (arXiv 2505.11594), section 3.4 "The NVFP4
 *          Microscaling Format and Quantization Operator" (E2M1 value set, 1x32 E8M0
 *          blocks for MXFP4).
 *   [QA]   "Quantization for Attention, in depth" blog: "The datapath and its quantize
 *          points", "Worked example: what smoothing buys at INT8", "Failure modes".
 *
 * Conventions: tensors of one (batch, head) are row-major [tokens][d]; inputs arrive as
 * raw bf16 or fp16 bit patterns and are widened exactly to FP32.  Every quantity the
 * method keeps in full precision is computed here in FP64; the preprocessing is FP32/FP64
 * with a pinned evaluation order so that the quantized tensors and scales have exactly one
 * correct value (see sage_oracle.c for each step and the reading it takes).
 */
#ifndef SAGE_ORACLE_H
#define SAGE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_BQ 128 /* Q smoothing block (FlashAttention query tile) */
#define ORC_BK 64  /* KV tile: running-max step and two-level accumulation granularity */

/* ---- option bits (default 0 = the method as the pages define it) ---- */
#define ORC_SMOOTH_V      0x0001u /* V' = V - mean_t(V), O += V_m            [SA2 optional V smoothing] */
#define ORC_NO_SMOOTH_K   0x0002u /* ablation: skip K - mean(K)                                          */
#define ORC_NO_SMOOTH_Q   0x0004u /* ablation: skip per-block Q mean / Delta S                           */
#define ORC_QK_IDENTITY   0x0010u /* no Q/K quantization, smoothing done in FP64                         */
#define ORC_QK_PER_BLOCK  0x0020u /* ablation: one scale per Q block (128) and per K tile (64)           */
#define ORC_QK_PER_TOKEN  0x0040u /* ablation: one scale per Q token and per K token                     */
#define ORC_QK_PER_TENSOR 0x0080u /* ablation: one scale for all of Q (per head), one for all of K       */
#define ORC_PV_IDENTITY   0x0100u /* no P/V quantization (448*P~ and V'/dV kept exact)                   */
#define ORC_PV_E5M2       0x0200u /* ablation: P~ and V in E5M2 (static scale 1/57344, per-channel V)    */
#define ORC_PV_INT8       0x0400u /* ablation: naive INT8 P~ (static 1/127) and per-channel INT8 V       */
#define ORC_MXFP4         0x1000u /* MX variant: E2M1 values, E8M0 scale per 32 along the reduction dim  */
#define ORC_QK_E4M3       0x2000u /* knob: Q^, K^ in E4M3 (scale amax/448, same groups) instead of INT8  */
#define ORC_MX_P_TWO_LEVEL 0x4000u /* MX knob: P~ of each tile row divided by rowmax/6 before the E2M1  */
                                   /* quantizer, the tile's P^V product multiplied back by it [SA3]      */

/* ---- scalar formats ---- */
float   orc_bf16_to_f32(uint16_t h);
float   orc_fp16_to_f32(uint16_t h);
double  orc_e4m3_decode(uint8_t code);  /* OCP E4M3FN: bias 7, max 448, no Inf, S.1111.111 = NaN */
uint8_t orc_e4m3_encode(double x);      /* round-to-nearest-even, saturate to +-448, NaN -> 0x7F */
void    orc_e4m3_encode_f32_array(const float* x, uint8_t* out, size_t n); /* the cast above, per element */
double  orc_e5m2_decode(uint8_t code);  /* OCP E5M2: bias 15, max 57344                           */
uint8_t orc_e5m2_encode(double x);      /* RNE, saturate to +-57344                               */
double  orc_e2m1_decode(uint8_t code);  /* 4-bit E2M1: {0, .5, 1, 1.5, 2, 3, 4, 6} and negatives   */
uint8_t orc_e2m1_encode(double x);      /* RNE (ties to even mantissa), saturate to +-6           */
int     orc_e8m0_exponent(double amax); /* smallest e with amax <= 6*2^e, clamped to [-127,127]   */

/* Quantization group of key t inside its 64-key tile (0..3), see sage_oracle.c step 3. */
int orc_k_group(int t);

/* ---- whole-head preprocessing (the quantities the GPU must reproduce bit for bit) ----
 * q: [N][d], k, v: [M][d] raw 16-bit codes; in_fp16 selects fp16 (else bf16).
 * Outputs (natural layouts, all caller-allocated):
 *   kmean[d], vmean[d] (zeros unless ORC_SMOOTH_V), khat[M][d], dk[ceil(M/64)][4],
 *   vhat[M][d] (E4M3 codes), dv[d], qhat[N][d], dq[N], qmean[ceil(N/128)][d],
 *   ds[ceil(N/128)][M] (FP64 Delta S).
 * Only the default quantizers (per-thread INT8 QK, E4M3 PV) are written by this call;
 * flags may hold ORC_SMOOTH_V, ORC_NO_SMOOTH_K, ORC_NO_SMOOTH_Q, ORC_QK_PER_BLOCK (the
 * per-block ablation; dk then repeats the tile scale) and ORC_QK_E4M3 (khat and qhat then
 * hold E4M3 codes, dk and dq the E4M3 scales).  Returns 0, or -1 on a bad argument. */
int orc_preprocess_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                        int N, int M, int d, unsigned flags,
                        float* kmean, float* vmean, int8_t* khat, float* dk,
                        uint8_t* vhat, float* dv, int8_t* qhat, float* dq,
                        float* qmean, double* ds);

/* MX variant (ORC_MXFP4 implied): E2M1 codes of gamma(Q) [N][d], gamma(K) [M][d], V' [M][d];
 * E8M0 exponents (unbiased) [N][d/32], [M][d/32] per 32 channels and [ceil(M/32)][d] per 32
 * tokens of each V channel.  flags: ORC_SMOOTH_V / ORC_NO_SMOOTH_K / ORC_NO_SMOOTH_Q. */
int orc_preprocess_mx_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                           int N, int M, int d, unsigned flags,
                           uint8_t* qcode, int* qexp, uint8_t* kcode, int* kexp,
                           uint8_t* vcode, int* vexp);
/* ---- SageBwd (trainable INT8 attention; sagebwd_oracle.c): forward with the row
 * log-sum-exp, and the backward, for one head.  q, dout: [N][d], k, v: [M][d] raw 16-bit
 * codes; causal as orc_forward_head.  Outputs in FP64: out [N][d], lse [N] (natural log, of
 * the scores after K smoothing), dq [N][d], dk, dv [M][d].  The backward runs the forward
 * itself (out and lse are written by both calls).  Returns 0, or -1 on a bad argument. */
#define ORC_SB_IDENTITY    0x0001u /* no quantizer anywhere: exact attention and its gradients    */
#define ORC_SB_NO_SMOOTH_K 0x0002u /* ablation: skip K - mean(K)                                   */
#define ORC_SB_DP_INT8     0x0004u /* ablation: dP = dO V^T from per-block INT8 dO and V           */
int orc_sagebwd_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16, int N, int M, int d,
                        int causal, double sm_scale, unsigned flags, double* out, double* lse);
int orc_sagebwd_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         int in_fp16, int N, int M, int d, int causal, double sm_scale, unsigned flags,
                         double* out, double* lse, double* dq, double* dk, double* dv);
/* SageBwd's quantized tensors: INT8 codes of Q, dO per 128 rows and of smoothed K, V per 64
 * keys, the FP32 block scales, and the K mean.  Any output may be NULL (dout too). */
int orc_sagebwd_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         int in_fp16, int N, int M, int d, unsigned flags, int8_t* qcode, float* sq,
                         int8_t* kcode, float* sk, int8_t* vcode, float* sv, int8_t* docode, float* sdo,
                         float* kmean);

/* ---- forward of one head: the quantized method, FP64 everywhere it is not quantized ----
 * rows: the query rows to produce (NULL with nrows = N means all rows in order);
 * out: [nrows][d] in FP64.  causal: 0 none; 1 key t visible to row r iff t <= r (first
 * query aligned with the first key); 2 iff t <= r + M - N (last query aligned with the last
 * key; needs N <= M).
 * Returns 0, or -1 on a bad argument. */
int orc_forward_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                     int N, int M, int d, int causal, double sm_scale, unsigned flags,
                     const int* rows, int nrows, double* out);
/* orc_forward_head, and per output row (ties and bound may each be NULL) the number of its P
 * quantization decisions (E4M3 codes of 448 P~; MX: E2M1 codes and E8M0 block exponents) whose
 * input lies within relative distance tie_eps of a rounding boundary -- a kernel working in
 * FP32 may round those the other way, and either result is a correct rounding -- and a bound
 * on how far the row's output can move if all of them do (a diagnostic for parity tests).
 * qk_step_err (ORC_QK_E4M3 only; 0 otherwise): a kernel whose matrix core sums each 64-channel
 * step of Q^ K^ with an error of at most qk_step_err times the step's largest code product; the
 * margin of each E4M3 decision of P^ then widens by the score errors this allows (that of the
 * key and that of the row maximum). */
int orc_forward_head_ties(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                          int N, int M, int d, int causal, double sm_scale, unsigned flags,
                          const int* rows, int nrows, double* out, double tie_eps, double qk_step_err,
                          int* ties, double* bound);

/* ---- textbook attention softmax(Q K^T * sm_scale) V in FP64 on the widened inputs ---- */
int orc_exact_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int in_fp16,
                   int N, int M, int d, int causal, double sm_scale,
                   const int* rows, int nrows, double* out);

/* Same, on FP64 inputs (used by the pins that build exactly representable cases). */
int orc_exact_f64(const double* q, const double* k, const double* v, int N, int M, int d,
                  int causal, double sm_scale, double* out);

/* Number of threads the OpenMP loops use (1 when built without OpenMP). */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
