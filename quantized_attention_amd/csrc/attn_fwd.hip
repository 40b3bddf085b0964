// attn_fwd.hip -- fused quantized attention forward, INT8 QK / FP8 PV (gfx950).
//
// "SageAttention2 Technical Report" summary, 3.4 "The Complete Algorithm (Algorithm 1)",
// per 128-query block i and 64-key tile j:
//   S   = dequant(Q^_i K^_j^T) + Delta S_ij                    ("Smoothing Q", per-thread dQ dK)
//   m   = max(m, rowmax S);  P~ = exp(S - m);  l = e^{m_old - m} l + rowsum P~   (FP32)
//   P^  = E4M3(448 P~)                                           ("FP8 Quantization for P~V")
//   R   = P^ V^_j  over this tile only;  O = e^{m_old - m} O + R in FP32
//                                                                ("Two-Level Accumulation")
//   out = O / l / 448 * dV (+ V_m)                                (epilogue)
//
// Mapping on CDNA4.  A work-group of 4 wave64s owns one query block; wave w owns queries
// 32w..32w+31.  Scores are produced transposed, S^T = K^ Q^T, with v_mfma_i32_32x32x32_i8:
// the 32x32 accumulator gives each lane ONE query (lane % 32) and 16 keys of a 32-key half
// (rows 8b + 4h + k, h = lane / 32), so the row max and row sum are lane-local plus one
// exchange with lane ^ 32, the per-thread scale of a lane's fragment is dQ[query] * dK[group],
// and the same lane's 32 P^ bytes (two halves) are already the B operand of
// O^T = V^T P^T on v_mfma_f32_32x32x64_f8f6f4 -- V^ was stored with its keys permuted to
// that order, so P never moves between lanes.  The exponent works in base 2 with the
// factor sm_scale*log2(e) folded into the dequant multiplier and Delta S, and log2(448)
// folded into the running max, so exp2 yields 448 P~ directly.
#include "sage_common.hpp"

namespace sage {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448)

template <int D>
struct Tiles {
  static constexpr int KS = D + 16;   // padded K^ row (bytes)
  static constexpr int VS = kBK + 16; // padded V^ channel row (bytes)
};

struct AttnArgs {
  const int8_t* qhat;
  const int8_t* khat;
  const uint8_t* vhat;
  const float* dq;
  const float* dk;
  const float* dv;
  const float* vmean;
  const float* ds;   // Delta S * sm_scale * log2(e)
  void* out;
  int N, M, nqb, nkt, Np, Mp;
  float qk_scale;    // sm_scale * log2(e)
};

template <int D, bool CAUSAL, int OUT>  // OUT: 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = Tiles<D>::KS, VS = Tiles<D>::VS;
  constexpr int NKS = D / 32;  // k-steps of the QK MFMA; also channel sub-tiles of O
  __shared__ __attribute__((aligned(16))) int8_t sK[kBK * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sV[D * VS];
  __shared__ float sDS[kBK];
  __shared__ float sDK[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int bh = blockIdx.y;
  // heavy blocks first under the causal mask
  const int qb = CAUSAL ? (a.nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int q0 = qb * kBQ;
  const int qrow = q0 + 32 * w + col;  // this lane's query

  // Q^ fragments (B operand): query qrow, channels 32s + 16h .. +16
  v4i qf[NKS];
  {
    const int8_t* qp = a.qhat + ((size_t)bh * a.Np + qrow) * D + 16 * h;
#pragma unroll
    for (int s = 0; s < NKS; s++) qf[s] = *reinterpret_cast<const v4i*>(qp + 32 * s);
  }
  const float dql = a.dq[(size_t)bh * a.Np + qrow] * a.qk_scale;

  v16f O[NKS];
#pragma unroll
  for (int c = 0; c < NKS; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) O[c][r] = 0.0f;
  float m_run = -INFINITY;  // running max (base-2 units)
  float l_run = 0.0f;       // this lane's partial row sum of 448 P~

  int jend = a.nkt;
  if (CAUSAL) jend = min(a.nkt, (q0 + kBQ + kBK - 1) / kBK);

  const int8_t* kbase = a.khat + (size_t)bh * a.Mp * D;
  const uint8_t* vbase = a.vhat + (size_t)bh * a.nkt * D * kBK;
  const float* dsbase = a.ds + ((size_t)bh * a.nqb + qb) * a.Mp;
  const float* dkbase = a.dk + (size_t)bh * a.nkt * 4;

  for (int j = 0; j < jend; j++) {
    // ---- stage K^ (64 x D) and V^ (D x 64) of tile j in LDS ----
    {
      const int8_t* kt = kbase + (size_t)j * kBK * D;
      const uint8_t* vt = vbase + (size_t)j * D * kBK;
#pragma unroll
      for (int x = tid; x < kBK * D / 16; x += 256) {
        const int row = x / (D / 16), cc = (x % (D / 16)) * 16;
        *reinterpret_cast<v4i*>(&sK[row * KS + cc]) = *reinterpret_cast<const v4i*>(kt + row * D + cc);
      }
#pragma unroll
      for (int x = tid; x < D * kBK / 16; x += 256) {
        const int row = x / (kBK / 16), cc = (x % (kBK / 16)) * 16;
        *reinterpret_cast<v4i*>(&sV[row * VS + cc]) = *reinterpret_cast<const v4i*>(vt + row * kBK + cc);
      }
      if (tid < kBK) sDS[tid] = dsbase[(size_t)j * kBK + tid];
      if (tid < 4) sDK[tid] = dkbase[(size_t)j * 4 + tid];
    }
    __syncthreads();

    // ---- S^T = K^ Q^T on the INT8 MFMA (exact INT32) ----
    v16i acc[2];
#pragma unroll
    for (int T = 0; T < 2; T++) {
#pragma unroll
      for (int r = 0; r < 16; r++) acc[T][r] = 0;
#pragma unroll
      for (int s = 0; s < NKS; s++) {
        const v4i kf = *reinterpret_cast<const v4i*>(&sK[(32 * T + col) * KS + 32 * s + 16 * h]);
        acc[T] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[s], acc[T], 0, 0, 0);
      }
    }

    // ---- dequantize, add Delta S, mask; tile row max ----
    float sc[2][16];
    float mt = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; T++) {
      const float mul = dql * sDK[2 * T + h];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int kk = 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
        const int key = j * kBK + kk;
        float s = fmaf((float)acc[T][r], mul, sDS[kk]);
        const bool valid = (key < a.M) && (!CAUSAL || key <= qrow);
        s = valid ? s : -INFINITY;
        sc[T][r] = s;
        mt = fmaxf(mt, s);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    // base so that exp2(s - base) = 448 * exp(S - m); a row with nothing valid yet keeps 0s
    const float base = (m_new == -INFINITY) ? 0.0f : m_new - kLog2_448;
    const float alpha = exp2f(m_run - m_new);  // 0 on the first tile (m_run = -inf)
    m_run = m_new;

    // ---- P = 448 P~ (FP32), row sum, FP8 pack in the PV B-operand order ----
    float psum = 0.0f;
    v8i pf;
#pragma unroll
    for (int T = 0; T < 2; T++) {
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        float p0 = exp2f(sc[T][4 * q4 + 0] - base);
        float p1 = exp2f(sc[T][4 * q4 + 1] - base);
        float p2 = exp2f(sc[T][4 * q4 + 2] - base);
        float p3 = exp2f(sc[T][4 * q4 + 3] - base);
        psum += (p0 + p1) + (p2 + p3);
        int wd = 0;
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, wd, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
        pf[4 * T + q4] = wd;
      }
    }
    l_run = fmaf(l_run, alpha, psum);

    // ---- R = P^ V^ per 32-channel sub-tile (fresh FP32 accumulator), O = alpha O + R ----
#pragma unroll
    for (int c = 0; c < NKS; c++) {
      const uint8_t* vp = &sV[(32 * c + col) * VS + 32 * h];
      v8i vf;
      const v4i lo = *reinterpret_cast<const v4i*>(vp);
      const v4i hi = *reinterpret_cast<const v4i*>(vp + 16);
      vf[0] = lo[0]; vf[1] = lo[1]; vf[2] = lo[2]; vf[3] = lo[3];
      vf[4] = hi[0]; vf[5] = hi[1]; vf[6] = hi[2]; vf[7] = hi[3];
      v16f R;
#pragma unroll
      for (int r = 0; r < 16; r++) R[r] = 0.0f;
      R = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, R, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; r++) O[c][r] = fmaf(O[c][r], alpha, R[r]);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l (l holds 448 * sum P~) * dV (+ V_m) ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow >= a.N) return;
  const float inv = 1.0f / l_tot;
  const float* dvp = a.dv + (size_t)bh * D;
  const float* vmp = a.vmean + (size_t)bh * D;
  const size_t orow = ((size_t)bh * a.N + qrow) * D;
#pragma unroll
  for (int c = 0; c < NKS; c++) {
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ch = 32 * c + 8 * b + 4 * h;
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; k++) o[k] = fmaf(O[c][4 * b + k] * inv, dvp[ch + k], vmp[ch + k]);
      if (OUT == 2) {
        float4 v4 = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + ch) = v4;
      } else if (OUT == 1) {
        uint2 u;
        u.x = f32_to_fp16_bits(o[0]) | (f32_to_fp16_bits(o[1]) << 16);
        u.y = f32_to_fp16_bits(o[2]) | (f32_to_fp16_bits(o[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + ch) = u;
      } else {
        uint2 u;
        u.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
        u.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + ch) = u;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const Problem& p, const AttnArgs& a, hipStream_t s) {
  dim3 grid(p.nqb, p.BH);
  const int out = p.out_fp32 ? 2 : (p.fp16 ? 1 : 0);
  if (out == 2)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 2>), grid, dim3(256), 0, s, a);
  else if (out == 1)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Problem& p, const Workspace& w, void* out, hipStream_t s) {
  AttnArgs a;
  a.qhat = w.qhat; a.khat = w.khat; a.vhat = w.vhat; a.dq = w.dq; a.dk = w.dk; a.dv = w.dv;
  a.vmean = w.vmean; a.ds = w.ds; a.out = out;
  a.N = p.N; a.M = p.M; a.nqb = p.nqb; a.nkt = p.nkt; a.Np = p.Np; a.Mp = p.Mp;
  a.qk_scale = p.sm_scale * kLog2e;
  if (p.d == 128) return p.causal ? launch_d<128, true>(p, a, s) : launch_d<128, false>(p, a, s);
  return p.causal ? launch_d<64, true>(p, a, s) : launch_d<64, false>(p, a, s);
}

}  // namespace sage
