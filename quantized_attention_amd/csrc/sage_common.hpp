// sage_common.hpp -- shared definitions of the HIP library (gfx950 only).
//
// Problem description, workspace carving and the small device helpers the preprocessing
// and attention kernels share.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "sage_attn.h"

namespace sage {

constexpr int kBQ = SAGE_BQ;  // query block: Q smoothing and the attention work-group tile
constexpr int kBK = SAGE_BK;  // key/value tile: running-max step and two-level accumulation

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Where the rows of one (sequence, head) of a q / k / v / out tensor live.  Dense tensors are
// [B][H][T][d]; packed ones (variable-length batches) are [total][H][d], sequence b in rows
// cu[b] .. cu[b+1]-1.
struct SeqLayout {
  const int* cu;  // device offsets of the B + 1 sequence starts; null: dense
  int T;          // dense: tokens per sequence; packed: the bound on a sequence's length
  int total;      // packed: rows of the tensor
};
struct SeqRows {
  size_t base;    // element offset of (token 0, channel 0)
  size_t stride;  // elements from one token to the next
  int len;        // tokens of this sequence
};
// A packed sequence's offsets are clamped to [0, total] and its length to T, so that no
// offset array, however malformed, moves an access outside the tensor or the workspace.
__device__ inline SeqRows seq_rows(const SeqLayout& L, int b, int h, int H, int d) {
  if (L.cu == nullptr) return {((size_t)b * H + h) * (size_t)L.T * d, (size_t)d, L.T};
  int s = L.cu[b], e = L.cu[b + 1];
  s = s < 0 ? 0 : (s > L.total ? L.total : s);
  e = e < s ? s : (e > L.total ? L.total : e);
  return {((size_t)s * H + h) * d, (size_t)H * d, e - s < L.T ? e - s : L.T};
}

// Resolved problem: sizes, padded sizes and the variant bits.
struct Problem {
  int B, H, N, M, d;
  int Hkv, G;  // key/value heads; query head h reads key/value head h / G (G = H / Hkv)
  int causal;  // 0 none, 1 first query aligned with the first key, 2 last with the last
  float sm_scale;
  unsigned variant;
  int BH, BHkv, nqb, nkt, Np, Mp;  // BH = B*H query heads, BHkv = B*Hkv key/value heads
  bool fp16, out_fp32, smooth_v;
  bool mx;  // SAGE_PATH_MXFP4
  bool qf8;  // SAGE_QK_FP8
  // Rows of q / out (ql) and of k, v (kl): dense [B][H][T][d], or packed [total][H][d] for a
  // variable-length batch (then N and M are the bounds on the sequence lengths)
  SeqLayout ql, kl;
};

// Device workspace (all 256-byte aligned slices of one allocation).  Layouts of the
// quantized tensors and scales are those sage_attn.h documents for the quantize views
// (INT8/FP8, or E2M1 codes with E8M0 scales for the MX variant).  The Q side (qhat, dq,
// qmean, ds, qm_hi/lo, qsc) has one head per query head; the K/V side one per key/value head.
struct Workspace {
  int8_t* qhat;     // [BH][Np][d]            (MX: [BH][Np][d/2] E2M1 pairs)
  int8_t* khat;     // [BH][Mp][d]            (MX: [BH][Mp][d/2])
  uint8_t* vhat;    // [BH][nkt][d][64] keys permuted (MX: [BH][nkt][d][32])
  float* dq;        // [BH][Np]   (not used by MX)
  float* dk;        // [BH][nkt][4]   (not used by MX)
  float* dv;        // [BH][d]
  float* kmean;     // [BH][d]
  float* vmean;     // [BH][d]
  float* qmean;     // [BH][nqb][d]
  float* ds;        // [BH][nqb][Mp], Delta S (pre-multiplied by ds_scale)
  double* kpart;    // [BH][nkt][d] FP64 chunk sums of K
  double* vpart;    // [BH][nkt][d] FP64 chunk sums of V (V smoothing)
  float2* vmm;      // [BH][nkt][d] chunk (max, min) of V
  uint16_t* qm_hi;  // bf16 head of the block mean, in the Delta S MFMA operand order:
                    // [BH][ceil(nqb/32)][d/16][64 lanes][8] (lane 32 h + block % 32 holds
                    // channels 16 s + 8 h .. +7)
  uint16_t* qm_lo;  // the bf16 tail, q_mean - hi rounded to bf16, in the same order
  uint8_t* qsc;     // MX: [BH][Np][d/32] E8M0 of gamma(Q) blocks
  uint8_t* ksc;     // MX: [BH][nkt][64][4] E8M0 of gamma(K) blocks, MFMA A-operand lane order
  uint8_t* vsc;     // MX: [BH][nkt][64][4] E8M0 of V' blocks, MFMA A-operand lane order
};
constexpr int kWsSlices = 19;

// Bytes of each workspace slice, in carving order.
size_t workspace_layout(const Problem& p, size_t* sizes /* [kWsSlices] or null */);
void carve_workspace(const Problem& p, void* base, Workspace* w);

// The key a lane half h consumes at byte b of its 32-byte FP8 P fragment: the S^T
// accumulator of the two 32-key halves (T = b / 16) holds, for accumulator register
// r = b % 16, key 8*(r/4) + 4*h + r%4 of that half.
__host__ __device__ inline int kperm(int h, int b) {
  return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3);
}

// Scale group (0..3) of key t inside its 64-key tile: the lane half of the S^T accumulator
// that holds it, within its 32-key half.
// The key/value head (in [0, B*Hkv)) that query head bh (in [0, B*H)) reads.
__host__ __device__ inline int kv_head(int bh, int H, int Hkv, int G) { return (bh / H) * Hkv + (bh % H) / G; }

__host__ __device__ inline int kgroup(int t) {
  int u = t & 63;
  return 2 * (u >> 5) + ((u >> 2) & 1);
}

// MX: the key (inside its 64-key tile) that lane half h of the FP4 PV MFMA consumes at
// nibble j of its 32-nibble P fragment, once the two lane halves have swapped fragments so
// that half h holds the keys 32h..32h+31: the fragment's first 16 nibbles come from
// accumulator lane half 0 (keys 8*(r/4) + r%4), the last 16 from lane half 1 (+4).
__host__ __device__ inline int vperm_mx(int h, int j) {
  return 32 * h + 8 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3);
}

// E8M0 byte of an MX block with largest magnitude amax (FP32, >= 0, NaN excluded): the
// smallest e with amax <= 6 * 2^e, clamped to [-127, 127], biased by 127.  With
// amax = (1 + f) 2^(E - 127): e = E - 129 if f <= 1/2, else E - 128; a subnormal or zero
// amax gives e = -127; an infinite one e = 127.
__device__ inline uint32_t e8m0_code(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int E = (int)(u >> 23);
  if (E == 255) return 254u;
  const int c = E - 2 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
  return c > 0 ? (uint32_t)c : 0u;
}

__device__ inline float load_in(const uint16_t* p, size_t i, bool fp16) {
  uint16_t h = p[i];
  if (fp16) return static_cast<float>(__builtin_bit_cast(_Float16, h));
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// FP32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ inline uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// FP32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ inline uint32_t f32_to_fp16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

// |x| max that ignores NaN (a NaN element does not set a scale): IEEE maxNum of the magnitudes.
__device__ inline float amax_upd(float m, float x) { return fmaxf(m, fabsf(x)); }

// Lane value from a DPP pattern of the lane's row (16 lanes).
template <int CTRL>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max over aligned groups of G lanes (G = 2, 4, 8 or 16), every lane of a group receiving it,
// for values that are not NaN: lane swaps inside quads, then the half-row and row mirrors
// (each exchanges the two halves of the group reduced so far).  No LDS round trips.
template <int G>
__device__ inline float group_max(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2, 4, 8 or 16 lanes");
  v = fmaxf(v, dpp_f32<0xB1>(v));                     // quad_perm [1, 0, 3, 2]
  if constexpr (G >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  if constexpr (G >= 8) v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  if constexpr (G >= 16) v = fmaxf(v, dpp_f32<0x140>(v)); // row_mirror
  return v;
}

// Symmetric INT8 code: RNE of x / scale (IEEE FP32 division), clamped to +-127; NaN -> 0.
__device__ inline int8_t int8_code(float x, float scale) {
  float y = rintf(__fdiv_rn(x, scale));
  if (!(y == y)) return 0;
  y = y > 127.0f ? 127.0f : (y < -127.0f ? -127.0f : y);
  return static_cast<int8_t>(static_cast<int>(y));
}

// Max over the 64 lanes of a wave (values that are not NaN), every lane receiving it: the
// row maxima, then rows l and l ^ 16, then the wave halves (gfx950 lane-swap instructions).
__device__ inline float wave_max(float v) {
  v = group_max<16>(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Eight INT8 codes int8_code(x[e], scale), packed little-endian into two words, from the
// products with rcp = __fdiv_rn(1, scale).  |x / scale| <= 127.0001, and the exact product
// u = x * rcp is within |x / scale| * 2^-23 < 1.6e-5 of it; the IEEE quotient is within half
// an ulp (< 4e-6) of it too.  So the two round to the same integer unless a half-integer lies
// within 2e-5 of u.  t = fma(x, rcp, 1.5 * 2^23) rounds u to the nearest integer n (half to
// even) and holds n + 1.5 * 2^23 exactly, so n's two's-complement low byte is t's low byte;
// |x| <= amax keeps |n| <= 127.  A chunk with some |u - n| >= 0.4999 (about 1 in 5000), or a
// NaN (whose t lies above the integers' bit range), is coded again with the division: one
// branch per chunk, not per element.
__device__ inline uint2 int8_pack8_rcp(const float (&x)[8], float scale, float rcp) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: floats in [2^23, 2^24) step by 1
  uint32_t t[8];
  float rmax = 0.0f;
  uint32_t tmax = 0u;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float tf = fmaf(x[e], rcp, kMagic);
    const float n = tf - kMagic;
    rmax = fmaxf(rmax, fabsf(fmaf(x[e], rcp, -n)));  // a NaN residual is caught by tmax
    t[e] = __float_as_uint(tf);
    tmax = max(tmax, t[e]);
  }
  uint32_t w[2];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    // low bytes of t[4k .. 4k + 3] -> bytes 0 .. 3 (v_perm_b32: selector byte i picks byte i
    // of {S0, S1} as bytes 7..4, 3..0; 0x0c gives zero)
    const uint32_t lo = __builtin_amdgcn_perm(t[4 * k + 1], t[4 * k], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(t[4 * k + 3], t[4 * k + 2], 0x04000c0cu);
    w[k] = lo | hi;
  }
  if (!(rmax < 0.4999f) || tmax > 0x4B40007Fu) {  // 0x4B40007F: the bits of 1.5 * 2^23 + 127
    w[0] = w[1] = 0u;
#pragma unroll
    for (int e = 0; e < 8; e++) w[e >> 2] |= (uint32_t)(uint8_t)int8_code(x[e], scale) << (8 * (e & 3));
  }
  return make_uint2(w[0], w[1]);
}

// The E4M3 inputs x[e] / scale[e] (IEEE division) saturated to +-448, in place, from the
// products with rcp[e] = __fdiv_rn(1, scale[e]).  A product is within 3 ulps of the quotient,
// so the two round to the same E4M3 value unless the 20 low mantissa bits (the ones E4M3
// drops from a normal value) lie within 16 ulps of the rounding midpoint 2^19, or the value
// is below the E4M3 normal range (2^-6), or NaN.  A chunk holding such an element is divided
// instead.
__device__ inline void e4m3_in8_rcp(float (&x)[8], const float* scale, const float* rcp) {
  float y[8];
  uint32_t near = 0u;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    y[e] = x[e] * rcp[e];
    const uint32_t mag = __float_as_uint(y[e]) & 0x7FFFFFFFu;
    // below 2^-6 (wraps) or NaN / Inf, as one unsigned range test; then the midpoint window
    near |= static_cast<uint32_t>(mag - 0x3C800000u >= 0x7F800000u - 0x3C800000u);
    near |= static_cast<uint32_t>((mag & 0xFFFFFu) - (0x80000u - 15u) < 31u);
  }
  if (near) {
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = __fdiv_rn(x[e], scale[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float c = fminf(fmaxf(y[e], -448.0f), 448.0f);
    x[e] = (y[e] == y[e]) ? c : y[e];  // NaN stays NaN
  }
}

__device__ inline float int8_scale(float amax) {
  float a = amax > 1e-8f ? amax : 1e-8f;
  return __fdiv_rn(a, 127.0f);
}

// Scale of the E4M3 form of Q^ / K^ (SAGE_QK_FP8): amax / 448 with the INT8 path's floor.
__device__ inline float e4m3_scale(float amax) {
  float a = amax > 1e-8f ? amax : 1e-8f;
  return __fdiv_rn(a, 448.0f);
}

// Eight E4M3 codes of x[e] / scale (the IEEE quotient, saturated to +-448), packed
// little-endian into two words, through the reciprocal product with its exact fallback.
__device__ inline uint2 e4m3_pack8_rcp(const float (&x)[8], float scale, float rcp) {
  float y[8];
  float sc[8], rc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    y[e] = x[e];
    sc[e] = scale;
    rc[e] = rcp;
  }
  e4m3_in8_rcp(y, sc, rc);
  uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return make_uint2(w0, w1);
}

// bf16 bits of an FP32 value, round to nearest even (hardware conversion).
__device__ inline uint16_t bf16_rn(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ inline float bf16_val(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Launchers; each returns hipSuccess or the launch error.
// The Q blocks (q_hat, dq or the MX scales, q_mean and its bf16 head/tail; skipped when q is null)
// and the K / V chunk statistics, in one launch.
hipError_t launch_stats(const Problem& p, const void* q, const void* k, const void* v, const Workspace& w,
                        hipStream_t s);
// Chunk statistics -> K mean, V_m and the V scale.
hipError_t launch_kv_finalize(const Problem& p, const Workspace& w, hipStream_t s);
// K^, Delta S (into ds_out scaled by ds_scale; skipped when ds_out is null) and V^.
hipError_t launch_kv_quant(const Problem& p, const void* k, const void* v, const Workspace& w,
                           float ds_scale, float* ds_out, hipStream_t s);
// The fused kernels.  e0 / e1 (may be null): events that take the kernel's start and end
// times from its own dispatch (no separate event records on the stream).
hipError_t launch_attn_fwd(const Problem& p, const Workspace& w, void* out, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1);
hipError_t launch_attn_fwd_mx(const Problem& p, const Workspace& w, void* out, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1);

}  // namespace sage
