// attn_fwd.hip -- fused quantized attention forward, INT8 QK / FP8 PV (gfx950).
//
// "SageAttention2 Technical Report" summary, 3.4 "The Complete Algorithm (Algorithm 1)",
// per 128-query block i and 64-key tile j:
//   S   = dequant(Q^_i K^_j^T) + Delta S_ij                    ("Smoothing Q", per-thread dQ dK)
//   m   = max(m, rowmax S);  P~ = exp(S - m);  l = e^{m_old - m} l + rowsum P~   (FP32)
//   P^  = E4M3(448 P~)                                           ("FP8 Quantization for P~V")
//   O   = e^{m_old - m} O + P^ V^_j, the tile's products summed before they meet the FP32
//         buffer O                                               ("Two-Level Accumulation")
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
//
// Two-level accumulation on this hardware: the FP8 MFMA sums one tile's 64 products in its
// own internal accumulator (whose precision is below FP32, like the accumulator the pages
// found on their GPUs) and then adds that per-tile sum to the C operand with one FP32
// rounding -- a probe of v_mfma_f32_32x32x64_f8f6f4 shows C passes through at full FP32
// precision.  So the default path keeps O in the MFMA's C/D registers: level one is the
// MFMA-internal tile sum, level two the FP32 buffer O, and the online-softmax rescale
// O *= e^{m_old - m} runs only when some row of the wave raised its maximum.  The literal
// form (R = P^ V^ from a zero accumulator, then O = alpha O + R with one VALU FMA per element)
// is kept as a variant for comparison.
//
// Work-group order: heavy query blocks first under the causal mask, and blocks of one head
// kept on one XCD (work-groups are dealt to the 8 XCDs round-robin), so a head's K^/V^
// tiles are shared through that XCD's L2.  K^/V^ tiles are double-buffered in LDS; the
// next tile's global loads are in flight while the current one is computed.
#include "sage_common.hpp"

namespace sage {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448)
constexpr int kXCD = 8;

template <int D>
struct Tiles {
  static constexpr int KS = D + 16;    // padded K^ row (bytes): conflict-free 16-lane b128 reads
  static constexpr int VS = kBK + 16;  // padded V^ channel row (bytes)
  static constexpr int KBYTES = kBK * KS;
  static constexpr int VBYTES = D * VS;
  static constexpr int KLD = kBK * D / 16 / 256;  // 16-byte loads per thread per tile
  static constexpr int VLD = D * kBK / 16 / 256;
};

struct AttnArgs {
  const int8_t* qhat;
  const int8_t* khat;
  const uint8_t* vhat;
  const float* dq;
  const float* dk;
  const float* dv;
  const float* vmean;
  const float* ds;  // Delta S * sm_scale * log2(e)
  void* out;
  int N, M, BH, nqb, nkt, Np, Mp;
  float qk_scale;   // sm_scale * log2(e)
  int xcd_map;      // 1: heads grouped per XCD
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max over the two lanes that share a query (l and l ^ 32), on the VALU
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 64-key tile for one wave: scores, online softmax, P^ V^ into O.  `masked` (wave-
// uniform) selects the causal / ragged-tail mask; interior tiles skip it.
template <int D, bool CAUSAL, bool ACC_VALU>
__device__ __forceinline__ void tile_step(const int8_t* __restrict__ sK, const uint8_t* __restrict__ sV,
                                          const float* __restrict__ sDS, const float* __restrict__ sDK,
                                          const v4i (&qf)[D / 32], float dql, int h, int col, int key0,
                                          int qrow, int M, bool masked, v16f (&O)[D / 32], float& m_run,
                                          float& l_run) {
  constexpr int KS = Tiles<D>::KS, VS = Tiles<D>::VS, NKS = D / 32;
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
  // ---- dequantize (dQ dK sm_scale log2e) and add Delta S ----
  float sc[2][16];
#pragma unroll
  for (int T = 0; T < 2; T++) {
    const float mul = dql * sDK[2 * T + h];
#pragma unroll
    for (int r = 0; r < 16; r++)
      sc[T][r] = fmaf((float)acc[T][r], mul, sDS[32 * T + 8 * (r >> 2) + 4 * h + (r & 3)]);
  }
  if (masked) {
    // Keys past M, and keys after the query under the causal mask.  Tile-local key
    // kk = c(T, r) + 4h is valid iff kk <= lim, i.e. c(T, r) <= lim - 4h, one compare per score.
    asm volatile("" ::: "memory");  // keep this a real branch (interior tiles skip it)
    int lim = M - 1 - key0;
    if (CAUSAL) lim = min(lim, qrow - key0);
    lim -= 4 * h;
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        sc[T][r] = (32 * T + 8 * (r >> 2) + (r & 3) <= lim) ? sc[T][r] : -INFINITY;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int T = 0; T < 2; T++)
#pragma unroll
    for (int r = 0; r < 16; r++) mt = fmaxf(mt, sc[T][r]);
  mt = pair_max(mt);
  const float m_new = fmaxf(m_run, mt);
  const float base = (m_new == -INFINITY) ? 0.0f : m_new - kLog2_448;
  const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile, exactly 1 if m is unchanged
  m_run = m_new;
  // ---- P = 448 P~ (FP32), row sum, E4M3 pack in the PV B-operand order ----
  float psum = 0.0f;
  v8i pf;
#pragma unroll
  for (int T = 0; T < 2; T++) {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const float p0 = fast_exp2(sc[T][4 * q4 + 0] - base);
      const float p1 = fast_exp2(sc[T][4 * q4 + 1] - base);
      const float p2 = fast_exp2(sc[T][4 * q4 + 2] - base);
      const float p3 = fast_exp2(sc[T][4 * q4 + 3] - base);
      psum += (p0 + p1) + (p2 + p3);
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
      pf[4 * T + q4] = wd;
    }
  }
  l_run = fmaf(l_run, alpha, psum);
  // ---- O^T += V^T P^T per 32-channel sub-tile ----
  if (!ACC_VALU) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < NKS; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) O[c][r] *= alpha;
    }
  }
#pragma unroll
  for (int c = 0; c < NKS; c++) {
    const uint8_t* vp = &sV[(32 * c + col) * VS + 32 * h];
    const v4i lo = *reinterpret_cast<const v4i*>(vp);
    const v4i hi = *reinterpret_cast<const v4i*>(vp + 16);
    const v8i vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (ACC_VALU) {
      v16f R;
#pragma unroll
      for (int r = 0; r < 16; r++) R[r] = 0.0f;
      R = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, R, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; r++) O[c][r] = fmaf(O[c][r], alpha, R[r]);
    } else {
      O[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, O[c], 0, 0, 0, 0, 0, 0);
    }
  }
}

template <int D, bool CAUSAL, int OUT, bool ACC_VALU>  // OUT: 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  using TL = Tiles<D>;
  constexpr int KS = TL::KS, VS = TL::VS, NKS = D / 32;
  __shared__ __attribute__((aligned(16))) int8_t sK[2][TL::KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][TL::VBYTES];
  __shared__ float sDS[2][kBK];
  __shared__ float sDK[2][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  // ---- work-group -> (head, query block) ----
  int bh, qi;
  {
    const int L = blockIdx.x;
    if (a.xcd_map) {  // XCD x gets heads x, x+8, ...; a head's blocks stay together
      const int x = L % kXCD, r = L / kXCD;
      bh = x + kXCD * (r / a.nqb);
      qi = r % a.nqb;
    } else {
      bh = L / a.nqb;
      qi = L % a.nqb;
    }
  }
  const int qb = CAUSAL ? (a.nqb - 1 - qi) : qi;  // heavy blocks first
  const int q0 = qb * kBQ;
  const int wq0 = q0 + 32 * w;       // first query of this wave
  const int qrow = wq0 + col;        // this lane's query

  // ---- Q^ fragments (B operand): query qrow, channels 32s + 16h .. +16 ----
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
  float m_run = -INFINITY, l_run = 0.0f;

  const int jend = CAUSAL ? min(a.nkt, (q0 + kBQ + kBK - 1) / kBK) : a.nkt;
  const int8_t* kbase = a.khat + (size_t)bh * a.Mp * D;
  const uint8_t* vbase = a.vhat + (size_t)bh * a.nkt * D * kBK;
  const float* dsbase = a.ds + ((size_t)bh * a.nqb + qb) * a.Mp;
  const float* dkbase = a.dk + (size_t)bh * a.nkt * 4;

  // ---- staging: global -> registers (next tile) -> LDS ----
  v4i kreg[TL::KLD], vreg[TL::VLD];
  float dsreg = 0.0f, dkreg = 0.0f;
  auto gload = [&](int j) {
    const int8_t* kt = kbase + (size_t)j * kBK * D;
    const uint8_t* vt = vbase + (size_t)j * D * kBK;
#pragma unroll
    for (int i = 0; i < TL::KLD; i++) kreg[i] = *reinterpret_cast<const v4i*>(kt + (tid + 256 * i) * 16);
#pragma unroll
    for (int i = 0; i < TL::VLD; i++) vreg[i] = *reinterpret_cast<const v4i*>(vt + (tid + 256 * i) * 16);
    if (tid < kBK) dsreg = dsbase[(size_t)j * kBK + tid];
    if (tid < 4) dkreg = dkbase[(size_t)j * 4 + tid];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TL::KLD; i++) {
      const int x = tid + 256 * i, row = x / (D / 16), cc = (x % (D / 16)) * 16;
      *reinterpret_cast<v4i*>(&sK[buf][row * KS + cc]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < TL::VLD; i++) {
      const int x = tid + 256 * i, row = x / (kBK / 16), cc = (x % (kBK / 16)) * 16;
      *reinterpret_cast<v4i*>(&sV[buf][row * VS + cc]) = vreg[i];
    }
    if (tid < kBK) sDS[buf][tid] = dsreg;
    if (tid < 4) sDK[buf][tid] = dkreg;
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int j = 0; j < jend; j++) {
    const int buf = j & 1;
    if (j + 1 < jend) gload(j + 1);
    const int key0 = j * kBK;
    // wave-uniform tile class: fully masked (skip), boundary (masked) or interior
    const bool skip = CAUSAL && key0 > wq0 + 31;
    const bool masked = (CAUSAL && key0 + kBK - 1 > wq0) || (key0 + kBK > a.M);
    if (!skip)
      tile_step<D, CAUSAL, ACC_VALU>(sK[buf], sV[buf], sDS[buf], sDK[buf], qf, dql, h, col, key0, qrow, a.M,
                                     masked, O, m_run, l_run);
    if (j + 1 < jend) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l (l holds 448 * sum P~) * dV (+ V_m) ----
  const float l_tot = pair_sum(l_run);
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
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + ch) = make_float4(o[0], o[1], o[2], o[3]);
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

template <int D, bool CAUSAL, bool ACC_VALU>
hipError_t launch_d(const Problem& p, const AttnArgs& a, hipStream_t s) {
  dim3 grid(p.nqb * p.BH);
  const int out = p.out_fp32 ? 2 : (p.fp16 ? 1 : 0);
  if (out == 2)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 2, ACC_VALU>), grid, dim3(256), 0, s, a);
  else if (out == 1)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 1, ACC_VALU>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 0, ACC_VALU>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool ACC_VALU>
hipError_t launch_c(const Problem& p, const AttnArgs& a, hipStream_t s) {
  return p.causal ? launch_d<D, true, ACC_VALU>(p, a, s) : launch_d<D, false, ACC_VALU>(p, a, s);
}

}  // namespace

hipError_t launch_attn_fwd(const Problem& p, const Workspace& w, void* out, hipStream_t s) {
  AttnArgs a;
  a.qhat = w.qhat; a.khat = w.khat; a.vhat = w.vhat; a.dq = w.dq; a.dk = w.dk; a.dv = w.dv;
  a.vmean = w.vmean; a.ds = w.ds; a.out = out;
  a.N = p.N; a.M = p.M; a.BH = p.BH; a.nqb = p.nqb; a.nkt = p.nkt; a.Np = p.Np; a.Mp = p.Mp;
  a.qk_scale = p.sm_scale * kLog2e;
  a.xcd_map = (p.BH % kXCD == 0) ? 1 : 0;
  const bool valu = (p.variant & SAGE_ACC_VALU) != 0;
  if (p.d == 128) return valu ? launch_c<128, true>(p, a, s) : launch_c<128, false>(p, a, s);
  return valu ? launch_c<64, true>(p, a, s) : launch_c<64, false>(p, a, s);
}

}  // namespace sage
