/*
 * sage_attn.h -- C ABI of the MI355X (gfx950) quantized attention forward.
 *
 * The operation is the SageAttention2 forward pass, INT8-QK / FP8-PV variant:
 *   "SageAttention2 Technical Report: Accurate 4 Bit Attention for Plug-and-play Inference
 *   Acceleration" (summary of arXiv 2411.10958), section 3.4, "The Complete Algorithm
 *   (Algorithm 1)": K is smoothed by its token mean, each 128-query block of Q by its own
 *   mean with the GEMV correction Delta S = q_i gamma(K)^T ("Smoothing Q"), smoothed Q and K
 *   are quantized to INT8 with one scale per thread fragment ("Per-Thread INT4
 *   Quantization", here per query token and per 16-key group), P~ = exp(S - m) is cast to
 *   FP8 E4M3 with the static scale 1/448 and V per channel to E4M3 ("FP8 Quantization for
 *   P~V"), the online softmax runs in FP32, and each 64-key tile's P^ V^ is accumulated
 *   into an FP32 output buffer ("Two-Level Accumulation"); the epilogue is O / l / 448 * dV
 *   (+ V_m with the optional V smoothing, "Optional Smoothing of V").  The drop-in API the
 *   pages describe replaces scaled-dot-product attention: softmax(Q K^T * sm_scale) V
 *   ("SageAttention Guide": API usage; "Quantization for Attention, in depth").
 *
 * Conventions for every entry point
 *   - Q is [B][H][N][d], K and V are [B][H][M][d], out is [B][H][N][d]; all contiguous,
 *     row-major, 16-byte aligned device pointers on the current HIP device.  Inputs are bf16
 *     or fp16 (SAGE_IN_*); out is the input type, or FP32 with SAGE_OUT_FP32.
 *   - d is 64 or 128; B, H, N, M >= 1; B*H*max(N,M)*d < 2^40; B*H <= 65535 and
 *     B*H*ceil(max(N/128, M/64)) < 2^24 (the kernels' grid sizes); SAGE_ERR_INVALID_ARG otherwise.
 *   - causal: 0 no mask; 1 key t visible to query r iff t <= r (the first query aligned with
 *     the first key: the upper triangle of the N x M score matrix is masked, as the pages'
 *     reference code does; any N, M); 2 iff t <= r + M - N (the last query aligned with the
 *     last key: the N queries follow the M - N earlier tokens of a key/value cache; needs
 *     N <= M, else SAGE_ERR_UNSUPPORTED).  Other values are SAGE_ERR_INVALID_ARG.
 *   - sm_scale <= 0 or not finite selects 1/sqrt(d).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work on it and
 *     never synchronize the host; the caller keeps every buffer alive until the stream has
 *     passed the call.  Buffers must not overlap (out may not alias an input).
 *   - Argument errors are detected before anything is enqueued and return a negative
 *     sage_status.  A failed launch returns SAGE_ERR_LAUNCH; faults inside kernels surface
 *     at the caller's next synchronization.
 *   - NaN inputs propagate to the output rows that attend to them (INT8/FP8 path; E2M1 has
 *     no NaN code, and the MX variant codes a NaN element as the largest magnitude, 6).
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad variant bits      */
  SAGE_ERR_UNSUPPORTED = -2, /* valid request this build does not serve (d, causal = 2 with
                                N > M, non-gfx950 device)                                  */
  SAGE_ERR_NO_MEMORY = -3,   /* workspace allocation failed, or a given workspace is small */
  SAGE_ERR_LAUNCH = -4,      /* a kernel launch or stream call failed                      */
  SAGE_ERR_DEVICE = -5       /* no usable HIP device                                       */
} sage_status;

/* ---- variant bit-field ---- */
#define SAGE_PATH_I8F8  0x0000u /* INT8 QK (per-token Q, 4 groups / 64 keys K), FP8 E4M3 PV   */
#define SAGE_PATH_MXFP4 0x0001u /* MXFP4 ("SageAttention3" summary, 3.4 "The NVFP4 Microscaling
                                   Format and Quantization Operator"): smoothed Q and K, P~ and
                                   V' in E2M1 with one E8M0 power-of-two scale per 32 elements
                                   along each product's reduction dimension (Q, K: 32 channels
                                   of a token; P~: 32 keys of a query row; V': 32 tokens of a
                                   channel), on the block-scaled FP4 MFMA.  No 448 and no dV:
                                   the epilogue is O / l (+ V_m).  Means and Delta S as above. */
#define SAGE_QK_FP8     0x0002u /* Q^ and K^ in FP8 E4M3 instead of INT8, with the same groups
                                   (per-token Q, 4 groups / 64 keys K) and the scale
                                   max(amax, 1e-8) / 448; Q K^T on the FP8 MFMA ("SageAttention2
                                   Technical Report" summary, "Critical Assessment": the FP8-QK
                                   form of SageAttention2-8b the pages do not evaluate).  Not
                                   combinable with SAGE_PATH_MXFP4 (SAGE_ERR_INVALID_ARG). */
#define SAGE_MX_P_TWO_LEVEL 0x0004u /* MXFP4 only: two-level quantization of P~ ("SageAttention3"
                                   summary, 3.4 "Two-Level Quantization for the Attention Map
                                   P").  Each row of a tile's P~ is divided by the FP32 factor
                                   s1 = rowmax(P~) / 6 before the E2M1 block quantizer, so that
                                   the row's largest value is exactly 6 (the pages' 448 * 6
                                   targets E4M3 block scales; with E8M0 scales only the
                                   factor's mantissa matters), and the tile's product is
                                   multiplied back by s1.  Costs one rescale of O per tile.
                                   SAGE_ERR_INVALID_ARG without SAGE_PATH_MXFP4 or together
                                   with SAGE_ACC_VALU. */
#define SAGE_SMOOTH_V   0x0010u /* V' = V - mean_t(V) before quantization, O += V_m           */
#define SAGE_IN_BF16    0x0000u
#define SAGE_IN_FP16    0x0100u
#define SAGE_OUT_SAME   0x0000u
#define SAGE_OUT_FP32   0x1000u /* write FP32 output (removes output rounding from checks)    */
#define SAGE_ACC_VALU   0x2000u /* two-level accumulation in its literal form: each tile's
                                   P^V^ from a zero MFMA accumulator, added to O by a VALU FMA
                                   (default: the tile sum enters O through the MFMA C operand) */

/* Tile constants of the method (query smoothing block, key/value tile). */
#define SAGE_BQ 128
#define SAGE_BK 64

/*
 * sage_attn_fwd -- the whole forward pass: preprocessing (means, quantization, Delta S)
 * followed by the fused attention kernel, on `stream`.
 * Workspace: allocated and released on the stream (stream-ordered hipMallocAsync /
 * hipFreeAsync); sage_attn_workspace_bytes() tells its size.
 * Returns SAGE_OK or a negative sage_status.
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, void* out,
                  int B, int H, int N, int M, int d, int causal, float sm_scale,
                  unsigned variant, void* stream);

/* Bytes of device workspace sage_attn_fwd_ws needs for this problem (0 on bad arguments). */
size_t sage_attn_workspace_bytes(int B, int H, int N, int M, int d, int causal, unsigned variant);

/* As sage_attn_fwd, with a caller-owned device workspace of ws_bytes bytes (256-byte
 * aligned).  Returns SAGE_ERR_NO_MEMORY if ws_bytes is too small. */
int sage_attn_fwd_ws(const void* q, const void* k, const void* v, void* out,
                     int B, int H, int N, int M, int d, int causal, float sm_scale,
                     unsigned variant, void* workspace, size_t ws_bytes, void* stream);

/*
 * sage_attn_quantize -- the preprocessing step alone, written into caller buffers (device
 * pointers; any may be NULL to skip it).  Layouts, with BH = B*H, nqb = ceil(N/128),
 * nkt = ceil(M/64), Np = 128*nqb, Mp = 64*nkt:
 *   q_hat   int8  [BH][Np][d]   smoothed, quantized Q; rows >= N are 0
 *   k_hat   int8  [BH][Mp][d]   smoothed, quantized K; keys >= M are 0
 *   v_hat   uint8 [BH][nkt][d][64]  E4M3 codes of V (or V'), transposed per 64-key tile;
 *           byte p = 32h + b of channel c holds key 64*tile + kperm(h, b) with
 *           kperm(h, b) = 32*(b/16) + 8*((b%16)/4) + 4*h + b%4 (the order in which a
 *           lane half h of the FP8 MFMA consumes the keys of its P fragment); keys >= M are 0
 *   dq      float [BH][Np]      per-token Q scale (1.0 for rows >= N)
 *   dk      float [BH][nkt][4]  K scale of (tile, group); group of key t in its tile is
 *           2*((t%64)/32) + (((t%32)>>2)&1)
 *   dv      float [BH][d]       per-channel V scale (max|V'| / 448)
 *   k_mean  float [BH][d]       token mean of K
 *   v_mean  float [BH][d]       token mean of V (0 unless SAGE_SMOOTH_V)
 *   q_mean  float [BH][nqb][d]  per-block mean of Q
 *   delta_s float [BH][nqb][Mp] Delta S_i[t] = q_i . gamma(K)[t] (FP32); with causal only
 *           the 64-key tiles that block i attends to (t < 128*(i+1) + (M - N for causal = 2))
 *           are written
 * With SAGE_QK_FP8, q_hat and k_hat hold OCP E4M3 codes (round to nearest even of the FP32
 * quotient, saturated to +-448) in the same layouts, and dq, dk the scales amax / 448.
 * With SAGE_PATH_MXFP4 the quantized tensors are E2M1 codes (sign << 3 | magnitude index
 * into {0, 0.5, 1, 1.5, 2, 3, 4, 6}), two per byte, the lower-indexed element in the low
 * nibble, and the scales are E8M0 bytes (2^(byte - 127)):
 *   q_hat   uint8 [BH][Np][d/2]   gamma(Q) / 2^e per 32-channel block; rows >= N are 0
 *   k_hat   uint8 [BH][Mp][d/2]   gamma(K) / 2^e per 32-channel block; keys >= M are 0
 *   v_hat   uint8 [BH][nkt][d][32]  V' / 2^e per 32-token block, transposed per 64-key tile:
 *           nibble p = 32h + j of channel c holds key 64*tile + vperm(h, j) with
 *           vperm(h, j) = 32*h + 8*((j%16)/4) + 4*(j/16) + j%4 (the keys a lane half h of
 *           the FP4 MFMA consumes after the P fragments of the two lane halves are swapped
 *           so that half h holds the contiguous keys 32h..32h+31); keys >= M are 0
 *   mx_scales_q uint8 [BH][Np][d/32]  E8M0 of (row, 32-channel block); rows >= N are 0
 *   mx_scales_k uint8 [BH][nkt][64][4] byte 4*l + 2*T + c (c < d/64) of tile u holds the E8M0
 *           of key 64u + 32T + l%32, channel block 2c + l/32 (the A-operand scale of MFMA lane
 *           l); bytes with c >= d/64 are 0
 *   mx_scales_v uint8 [BH][nkt][64][4] byte 4*l + g (g < d/32) of tile u holds the E8M0 of
 *           channel 32g + l%32, tokens 64u + 32*(l/32) .. +31; bytes with g >= d/32 are 0
 *   dq and dk are not written; dv is written (it is not used by the MX forward).
 * The E8M0 exponent of a block is the smallest e with max|x| <= 6 * 2^e, clamped to
 * [-127, 127] (an all-zero block has e = -127, byte 0).
 * Returns SAGE_OK or a negative sage_status.
 */
typedef struct {
  void* q_hat;
  void* k_hat;
  void* v_hat;
  float* dq;
  float* dk;
  float* dv;
  float* k_mean;
  float* v_mean;
  float* q_mean;
  float* delta_s;
  void* mx_scales_q; /* SAGE_PATH_MXFP4 only (ignored otherwise); NULL skips */
  void* mx_scales_k;
  void* mx_scales_v;
} sage_quant_views;

int sage_attn_quantize(const void* q, const void* k, const void* v,
                       int B, int H, int N, int M, int d, int causal, unsigned variant,
                       const sage_quant_views* dst, void* stream);

/*
 * Extended entry points: the same forward pass, preprocessing and workspace query for a
 * shape given as a struct, which also carries grouped key/value heads.
 *
 * Grouped heads (Hkv < Hq, Hq % Hkv == 0): query head h attends with key/value head
 * h / (Hq / Hkv) (consecutive query heads share one key/value head).  The method is applied
 * per (query head, key/value head) pair exactly as for Hkv == Hq: the K mean, V_m, the K and
 * V quantization and their scales belong to the key/value head; the Q block means, Q^, its
 * scales and Delta S_i[t] = q_i . gamma(K)[t] belong to the query head.  (The pages' example
 * 8B layer leaves grouped-query attention aside; this is the plain extension.)
 * Layouts: q and out [B][Hq][N][d]; k and v [B][Hkv][M][d].  In the quantize views the
 * K/V-side tensors (k_hat, v_hat, dk, dv, k_mean, v_mean, mx_scales_k, mx_scales_v) have
 * B*Hkv heads, the Q-side ones (q_hat, dq, q_mean, delta_s, mx_scales_q) B*Hq heads.
 * Argument errors as for the plain entry points; Hkv < 1 or Hq % Hkv != 0 is
 * SAGE_ERR_INVALID_ARG; a NULL shape is SAGE_ERR_INVALID_ARG (0 bytes from the size query).
 */
typedef struct {
  int B;            /* batch                                                   */
  int Hq;           /* query heads                                             */
  int Hkv;          /* key/value heads (Hq % Hkv == 0; Hkv == Hq: no grouping) */
  int N, M, d;      /* query tokens, key tokens, head dimension                */
  int causal;       /* 0, 1 or 2, as above                                     */
  float sm_scale;   /* <= 0 or not finite: 1/sqrt(d)                           */
  unsigned variant; /* SAGE_* bits                                             */
} sage_attn_shape;

/* Workspace bytes sage_attn_fwd_ex needs for this shape (0 on bad arguments). */
size_t sage_attn_workspace_bytes_ex(const sage_attn_shape* shape);

/* The forward pass.  workspace: a caller-owned device buffer of ws_bytes bytes (256-byte
 * aligned; SAGE_ERR_NO_MEMORY if smaller than sage_attn_workspace_bytes_ex), or NULL to
 * allocate and release it on the stream (stream-ordered). */
int sage_attn_fwd_ex(const sage_attn_shape* shape, const void* q, const void* k, const void* v, void* out,
                     void* workspace, size_t ws_bytes, void* stream);

/* The preprocessing step alone, into caller buffers (layouts as for sage_attn_quantize, with
 * the per-head counts above). */
int sage_attn_quantize_ex(const sage_attn_shape* shape, const void* q, const void* k, const void* v,
                          const sage_quant_views* dst, void* stream);

/*
 * Variable-length batches ("Handling Varying Sequence Lengths with VarLen Kernels": a ragged
 * batch of `batch` sequences concatenated along the token axis, no padding, described by
 * cumulative offsets and the bounds on the lengths).
 *
 * Layouts: q and out [total_q][Hq][d], k and v [total_k][Hkv][d] (token-major, heads
 * interleaved), contiguous, 16-byte aligned, the same dtypes as sage_attn_fwd.  Sequence b owns
 * query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key/value rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1.  Every sequence is computed exactly as sage_attn_fwd_ex computes it on
 * its own (B = 1, N and M its lengths): its own K mean, V_m, scales, 128-query blocks from its
 * first query, Delta S and causal alignment (causal = 2 aligns its last query with its last
 * key).  Rows of a sequence that see no key (a sequence without keys, or causal = 2 with more
 * queries than keys) are written as 0.  Rows of `out` outside every sequence are not written.
 *
 * The offsets stay on the device (the call does not synchronize): cu_seqlens_q[0] = 0,
 * non-decreasing, cu_seqlens_q[batch] = total_q; likewise for k.  The library clamps every
 * offset to [0, total] and every length to its max_seqlen bound, so a malformed array cannot
 * make it read or write outside q, k, v, out or the workspace; the values it then writes are
 * unspecified.  The workspace is laid out for `batch` sequences of the bound lengths
 * (sage_attn_varlen_workspace_bytes), so tight bounds keep it small.
 */
typedef struct {
  int batch;                       /* sequences, >= 1                                     */
  int Hq, Hkv, d;                  /* as in sage_attn_shape                               */
  int total_q, total_k;            /* rows of q (and out) and of k, v, >= 1               */
  int max_seqlen_q, max_seqlen_k;  /* bounds on the query / key length of a sequence, >= 1 */
  const int* cu_seqlens_q;         /* device, batch + 1 offsets into q and out, 4-aligned */
  const int* cu_seqlens_k;         /* device, batch + 1 offsets into k and v              */
  int causal;                      /* 0, 1, 2 per sequence, as in sage_attn_shape         */
  float sm_scale;                  /* <= 0 or non-finite: 1/sqrt(d)                       */
  unsigned variant;                /* as in sage_attn_shape                               */
} sage_attn_varlen_shape;

/* Workspace bytes of sage_attn_varlen_fwd (0 on bad arguments). */
size_t sage_attn_varlen_workspace_bytes(const sage_attn_varlen_shape* shape);

/* The forward of a variable-length batch on `stream`.  workspace: NULL for a stream-ordered
 * allocation, else a 256-byte aligned device buffer of ws_bytes bytes.  Returns SAGE_OK or a
 * negative sage_status (SAGE_ERR_INVALID_ARG for a NULL shape or offset array, a misaligned
 * pointer, a size below 1 or bad variant bits; SAGE_ERR_NO_MEMORY for a short workspace). */
int sage_attn_varlen_fwd(const sage_attn_varlen_shape* shape, const void* q, const void* k, const void* v,
                         void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * SageBwd, the trainable 8-bit attention ("SageAttention3: Microscaling FP4 Attention for
 * Inference and An Exploration of 8-Bit Training" summary, "SageBwd Forward Pass: INT8
 * Quantization for Training" and "SageBwd Backward Pass and the Critical dOV^T Decision").
 * A method of its own, beside the inference path above:
 *   forward  K smoothed (K - mean(K)); Q per 128 rows, K and V per 64 keys quantized to INT8
 *            (scale max|X| / 127); S = Q^ K^T s_Q s_K sm_scale; P per (row, 64-key block) to
 *            INT8 against the row's block max of P; O = sum P^ V^ s_P s_V / l, and the row's
 *            log-sum-exp L = m + ln l (natural log, of the scores after K smoothing: it differs
 *            from that of Q K^T by sm_scale q . mean(K));
 *   backward D = rowsum(dO o O); per (128-query, 64-key) block S again and P = exp(S - L), P
 *            and dS = P o (dP - D) quantized per block to INT8; dV = P^^T dO^ (dO per 128
 *            rows), dP = dO V^T from the 16-bit inputs (not quantized), dQ = dS^ K^ sm_scale
 *            + sm_scale rowsum(dS) mean(K), dK = dS^^T Q^ sm_scale.
 * Shapes as sage_attn_shape with Hkv = Hq (grouped heads: SAGE_ERR_UNSUPPORTED), d 64 or 128,
 * causal 0, 1 or 2 (2 needs N <= M).  variant: SAGE_IN_BF16 / SAGE_IN_FP16, SAGE_OUT_FP32 (the
 * dtype of out, which the backward reads back in the same dtype), SAGE_TRAIN_NO_SMOOTH_K;
 * other bits are SAGE_ERR_INVALID_ARG.  q, dout [B][H][N][d], k, v [B][H][M][d] (16-bit);
 * lse [B][H][N] FP32; dq [B][H][N][d], dk, dv [B][H][M][d] FP32.  workspace: NULL for a
 * stream-ordered allocation, else a 256-byte aligned buffer of
 * sage_attn_train_workspace_bytes() bytes (enough for either call).  All pointers are device
 * pointers, 16-byte aligned (lse 4-byte); outputs must not overlap inputs.
 */
#define SAGE_TRAIN_NO_SMOOTH_K 0x4000u /* ablation: K is not smoothed (training entry points) */
/* sage_attn_train_bwd keeps each (128-query, 64-key) block pair's INT8 dS^ (8.6 KiB per pair,
 * in the workspace) from its dK/dV kernel for its dQ kernel; with this bit, or when that
 * buffer would exceed 16 GiB, the dQ kernel recomputes S, P, dP and dS instead (slower, with a
 * workspace of a few bytes per token).  Both give the same dK and dV; dQ agrees to FP32
 * rounding (the order of the K-mean term's row sums). */
#define SAGE_TRAIN_RECOMPUTE_DS 0x8000u
/* Both training calls of one step, with this bit and the same caller workspace: the forward
 * leaves its INT8 Q^, K^, V^ (with their scales, the backward's transposed copies and K's mean)
 * in the workspace, and the backward takes them from there instead of quantizing q, k, v again,
 * as a training framework keeps the forward's activations for the backward.  The caller
 * guarantees that between the two calls nothing writes the workspace and q, k, v keep their
 * contents, and passes the same shape (SAGE_TRAIN_RECOMPUTE_DS may differ: the pair buffer is the
 * workspace's last part).  Either call with this bit and a NULL workspace returns
 * SAGE_ERR_INVALID_ARG.  Results are identical to those of the two calls without it. */
#define SAGE_TRAIN_KEEP_QUANT 0x10000u
size_t sage_attn_train_workspace_bytes(const sage_attn_shape* shape);
int sage_attn_train_fwd(const sage_attn_shape* shape, const void* q, const void* k, const void* v, void* out,
                        float* lse, void* workspace, size_t ws_bytes, void* stream);
int sage_attn_train_bwd(const sage_attn_shape* shape, const void* q, const void* k, const void* v,
                        const void* out, const void* dout, const float* lse, float* dq, float* dk, float* dv,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * sage_attn_fwd_noalloc -- the forward pass of sage_attn_fwd_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It calls no allocating routine.  Its workspace is a scratch array of
 * SAGE_NOALLOC_MAX_BYTES bytes that the library holds in device memory, one per GPU it runs on,
 * from the first call on that GPU until the process ends.
 * Arguments and layouts as for sage_attn_fwd_ex (no workspace arguments).  A problem whose
 * workspace (sage_attn_workspace_bytes_ex) exceeds SAGE_NOALLOC_MAX_BYTES returns
 * SAGE_ERR_NO_MEMORY before anything is enqueued.
 * Every call on one GPU uses that GPU's single scratch array: calls whose work overlaps on one
 * GPU (two streams, two host threads) race on it and must be ordered by the caller.  The array
 * keeps the last call's contents; nothing in it needs to start at zero.
 */
#define SAGE_NOALLOC_MAX_BYTES ((size_t)128 << 20)
int sage_attn_fwd_noalloc(const sage_attn_shape* shape, const void* q, const void* k, const void* v, void* out,
                          void* stream);

/*
 * sage_attn_set_profile_events -- measurement hook.  With both arguments non-NULL (two
 * hipEvent_t handles, created by the caller), the next forward call on this thread (any
 * sage_attn_fwd* entry point) launches its fused attention kernel with them as the launch's
 * start and stop events (hipExtLaunchKernel): they take the kernel's own start and end
 * times, and no separate event record enters the stream.  The pair is then forgotten (one
 * call, one pair).  NULL, NULL clears a pending pair.  Only the caller's events are touched;
 * no state is shared between threads.
 */
void sage_attn_set_profile_events(void* start, void* stop);

/* Human-readable text of a sage_status (static storage). */
const char* sage_attn_status_string(int status);

/* Library version: major*10000 + minor*100 + patch. */
int sage_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_ATTN_H */
