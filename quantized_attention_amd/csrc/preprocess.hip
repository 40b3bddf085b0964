// preprocess.hip -- smoothing and quantization of Q, K, V (gfx950).
//
// "SageAttention2 Technical Report" summary, 3.4:
//   * "Smoothing Q": k = mean(K) over all tokens of the head, gamma(K) = K - k; for each
//     128-query block q_i = mean(Q_i), gamma(Q_i) = Q_i - q_i.
//   * "Per-Thread INT4 Quantization" (here INT8): one scale per thread fragment of the
//     S^T = K^ Q^T MFMA -- per query token for Q, per 16-key group for K.
//   * "FP8 Quantization for P~V": dV[c] = max_t |V[t,c]| / 448, V^ = E4M3(V / dV).
//   * "Optional Smoothing of V": V' = V - V_m before the V quantizer.
// "Quantization for Attention, in depth", "Failure modes": means and scales cover valid
// tokens only.
//
// The values are pinned: FP64 sums in a fixed order (64-token chunks in token order, chunk
// sums in chunk order, one FP64 division, one rounding to FP32), IEEE FP32 division for
// every scale and code, round-half-even, so Q^, K^, V^, the scales and the means have
// exactly one correct value.  Every kernel here is HBM-bound; none needs MFMA.
#include "sage_common.hpp"

namespace sage {
namespace {

// ---- K (and V) chunk statistics: one thread per channel, 64 tokens in order ----
__global__ void k_stats_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                               double* __restrict__ kpart, double* __restrict__ vpart,
                               float* __restrict__ vamax, int M, int d, int nkt, bool fp16,
                               bool smooth_v) {
  const int u = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  if (c >= d) return;
  const size_t base = (size_t)bh * M * d;
  const int t0 = u * kBK, t1 = min(t0 + kBK, M);
  double ks = 0.0, vs = 0.0;
  float va = 0.0f;
  for (int t = t0; t < t1; t++) {
    ks += (double)load_in(K, base + (size_t)t * d + c, fp16);
    float x = load_in(V, base + (size_t)t * d + c, fp16);
    if (smooth_v)
      vs += (double)x;
    else
      va = amax_upd(va, x);
  }
  const size_t o = ((size_t)bh * nkt + u) * d + c;
  kpart[o] = ks;
  if (smooth_v)
    vpart[o] = vs;
  else
    vamax[o] = va;
}

// ---- chunk sums -> means (and the V scale when V is not smoothed) ----
__global__ void k_finalize_kernel(const double* __restrict__ kpart, const double* __restrict__ vpart,
                                  const float* __restrict__ vamax, float* __restrict__ kmean,
                                  float* __restrict__ vmean, float* __restrict__ dv, int M, int d,
                                  int nkt, bool smooth_v) {
  const int bh = blockIdx.x, c = threadIdx.x;
  if (c >= d) return;
  double ks = 0.0, vs = 0.0;
  float va = 0.0f;
  for (int u = 0; u < nkt; u++) {
    const size_t o = ((size_t)bh * nkt + u) * d + c;
    ks += kpart[o];
    if (smooth_v)
      vs += vpart[o];
    else
      va = va > vamax[o] ? va : vamax[o];
  }
  kmean[(size_t)bh * d + c] = (float)(ks / (double)M);
  if (smooth_v) {
    vmean[(size_t)bh * d + c] = (float)(vs / (double)M);
  } else {
    vmean[(size_t)bh * d + c] = 0.0f;
    float a = va > 1e-8f ? va : 1e-8f;
    dv[(size_t)bh * d + c] = __fdiv_rn(a, 448.0f);
  }
}

// ---- K: gamma(K), per-group scale, INT8 codes; V' chunk max when V is smoothed ----
// 256 threads, one 64-key tile.  Each thread owns 4 consecutive channels of a key.
template <int D>
__global__ __launch_bounds__(256) void k_quant_kernel(const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const float* __restrict__ kmean,
                                                      const float* __restrict__ vmean,
                                                      int8_t* __restrict__ khat, float* __restrict__ dk,
                                                      float* __restrict__ vamax, int M, int Mp, int nkt,
                                                      bool fp16, bool smooth_v) {
  constexpr int QUADS = kBK * D / 4;          // 4-channel groups in the tile
  constexpr int PER = QUADS / 256;            // per thread
  __shared__ float gmax[4][4];                // [group][wave]
  __shared__ float sdk[4];
  const int u = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t in_base = (size_t)bh * M * D;
  const float* km = kmean + (size_t)bh * D;
  float g[PER][4];
  float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int qd = tid + 256 * i;
    const int t = qd / (D / 4), c0 = (qd % (D / 4)) * 4;
    const int key = u * kBK + t;
    const int grp = kgroup(t);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float x = 0.0f;
      if (key < M) x = load_in(K, in_base + (size_t)key * D + c0 + e, fp16) - km[c0 + e];
      g[i][e] = x;
      // group index is a runtime value; update all four under a select
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (q == grp) am[q] = amax_upd(am[q], x);
    }
  }
  // wave reduction of the four maxima, then across the four waves (max is exact)
#pragma unroll
  for (int q = 0; q < 4; q++) {
    float m = am[q];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float o = __shfl_xor(m, off);
      m = o > m ? o : m;
    }
    if (lane == 0) gmax[q][wave] = m;
  }
  __syncthreads();
  if (tid < 4) {
    float m = gmax[tid][0];
    for (int w = 1; w < 4; w++) m = gmax[tid][w] > m ? gmax[tid][w] : m;
    const float s = int8_scale(m);
    sdk[tid] = s;
    dk[((size_t)bh * nkt + u) * 4 + tid] = s;
  }
  __syncthreads();
  int8_t* kout = khat + ((size_t)bh * Mp + (size_t)u * kBK) * D;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int qd = tid + 256 * i;
    const int t = qd / (D / 4), c0 = (qd % (D / 4)) * 4;
    const int key = u * kBK + t;
    const float s = sdk[kgroup(t)];
    uint32_t word = 0;
    if (key < M) {
#pragma unroll
      for (int e = 0; e < 4; e++) word |= (uint32_t)(uint8_t)int8_code(g[i][e], s) << (8 * e);
    }
    *reinterpret_cast<uint32_t*>(kout + (size_t)t * D + c0) = word;
  }
  if (smooth_v && tid < D) {
    const float vm = vmean[(size_t)bh * D + tid];
    float va = 0.0f;
    for (int t = u * kBK; t < min(u * kBK + kBK, M); t++)
      va = amax_upd(va, load_in(V, in_base + (size_t)t * D + tid, fp16) - vm);
    vamax[((size_t)bh * nkt + u) * D + tid] = va;
  }
}

// ---- V scale after smoothing: max over the chunk maxima ----
__global__ void v_scale_kernel(const float* __restrict__ vamax, float* __restrict__ dv, int d, int nkt) {
  const int bh = blockIdx.x, c = threadIdx.x;
  if (c >= d) return;
  float va = 0.0f;
  for (int u = 0; u < nkt; u++) {
    const float x = vamax[((size_t)bh * nkt + u) * d + c];
    va = va > x ? va : x;
  }
  const float a = va > 1e-8f ? va : 1e-8f;
  dv[(size_t)bh * d + c] = __fdiv_rn(a, 448.0f);
}

// ---- V: E4M3 codes, transposed per tile with the P-fragment key order ----
template <int D>
__global__ __launch_bounds__(256) void v_quant_kernel(const uint16_t* __restrict__ V,
                                                      const float* __restrict__ vmean,
                                                      const float* __restrict__ dv,
                                                      uint8_t* __restrict__ vhat, int M, int nkt,
                                                      bool fp16) {
  __shared__ float sv[kBK][D + 1];
  const int u = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const size_t in_base = (size_t)bh * M * D;
  const float* vm = vmean + (size_t)bh * D;
  const float* sc = dv + (size_t)bh * D;
  // coalesced load of the tile: V' = V - V_m (FP32), then V' / dV (IEEE division)
  for (int x = tid; x < kBK * D; x += 256) {
    const int t = x / D, c = x % D;
    const int key = u * kBK + t;
    float y = 0.0f;
    if (key < M) {
      const float vp = load_in(V, in_base + (size_t)key * D + c, fp16) - vm[c];
      y = __fdiv_rn(vp, sc[c]);
      // saturate to the E4M3 range (the conversion itself does not); NaN stays NaN
      y = y > 448.0f ? 448.0f : (y < -448.0f ? -448.0f : y);
    }
    sv[t][c] = y;
  }
  __syncthreads();
  // each thread writes 4-byte words: channel c, bytes p0..p0+3 of its 64-byte row
  uint8_t* vout = vhat + ((size_t)bh * nkt + u) * (size_t)D * kBK;
  for (int x = tid; x < D * (kBK / 4); x += 256) {
    const int c = x / (kBK / 4), p0 = (x % (kBK / 4)) * 4;
    const int h = p0 >> 5, b0 = p0 & 31;
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sv[kperm(h, b0)][c], sv[kperm(h, b0 + 1)][c], w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sv[kperm(h, b0 + 2)][c], sv[kperm(h, b0 + 3)][c], w, true);
    *reinterpret_cast<int*>(vout + (size_t)c * kBK + p0) = w;
  }
}

// ---- Q: block mean, gamma(Q), per-token scale, INT8 codes ----
template <int D>
__global__ __launch_bounds__(256) void q_prep_kernel(const uint16_t* __restrict__ Q,
                                                     int8_t* __restrict__ qhat, float* __restrict__ dq,
                                                     float* __restrict__ qmean, int N, int Np, int nqb,
                                                     bool fp16) {
  __shared__ uint16_t sq[kBQ][D + 2];  // raw 16-bit inputs of the block
  __shared__ float sm[D];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r0 = i * kBQ, n = min(kBQ, N - r0);
  const size_t in_base = (size_t)bh * N * D;
  for (int x = tid; x < kBQ * D; x += 256) {
    const int r = x / D, c = x % D;
    sq[r][c] = (r < n) ? Q[in_base + (size_t)(r0 + r) * D + c] : (uint16_t)0;
  }
  __syncthreads();
  if (tid < D) {
    double s = 0.0;  // rows in order, FP64
    for (int r = 0; r < n; r++) s += (double)load_in(&sq[r][0], tid, fp16);
    const float m = (float)(s / (double)n);
    sm[tid] = m;
    qmean[((size_t)bh * nqb + i) * D + tid] = m;
  }
  __syncthreads();
  // each wave takes 32 rows; a lane holds D/64 channels of the row
  constexpr int CPL = D / 64;
  for (int rr = 0; rr < kBQ / 4; rr++) {
    const int r = wave * (kBQ / 4) + rr;
    float g[CPL];
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL; e++) {
      const int c = lane * CPL + e;
      g[e] = (r < n) ? load_in(&sq[r][0], c, fp16) - sm[c] : 0.0f;
      am = amax_upd(am, g[e]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o = __shfl_xor(am, off);
      am = o > am ? o : am;
    }
    const float s = (r < n) ? int8_scale(am) : 1.0f;
    const size_t row = (size_t)bh * Np + r0 + r;
    if (lane == 0) dq[row] = s;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < CPL; e++)
      word |= (uint32_t)(uint8_t)((r < n) ? int8_code(g[e], s) : 0) << (8 * e);
    if (CPL == 2)
      *reinterpret_cast<uint16_t*>(qhat + row * D + lane * CPL) = (uint16_t)word;
    else
      qhat[row * D + lane] = (int8_t)word;
  }
}

}  // namespace

hipError_t launch_k_stats(const Problem& p, const void* k, const void* v, const Workspace& w, hipStream_t s) {
  hipLaunchKernelGGL(k_stats_kernel, dim3(p.nkt, p.BH), dim3(p.d), 0, s,
                     (const uint16_t*)k, (const uint16_t*)v, w.kpart, w.vpart, w.vamax, p.M, p.d,
                     p.nkt, p.fp16, p.smooth_v);
  return hipGetLastError();
}

hipError_t launch_k_finalize(const Problem& p, const Workspace& w, hipStream_t s) {
  hipLaunchKernelGGL(k_finalize_kernel, dim3(p.BH), dim3(p.d), 0, s, w.kpart, w.vpart, w.vamax,
                     w.kmean, w.vmean, w.dv, p.M, p.d, p.nkt, p.smooth_v);
  return hipGetLastError();
}

hipError_t launch_k_quant(const Problem& p, const void* k, const void* v, const Workspace& w, hipStream_t s) {
  if (p.d == 128)
    hipLaunchKernelGGL(k_quant_kernel<128>, dim3(p.nkt, p.BH), dim3(256), 0, s, (const uint16_t*)k,
                       (const uint16_t*)v, w.kmean, w.vmean, w.khat, w.dk, w.vamax, p.M, p.Mp, p.nkt,
                       p.fp16, p.smooth_v);
  else
    hipLaunchKernelGGL(k_quant_kernel<64>, dim3(p.nkt, p.BH), dim3(256), 0, s, (const uint16_t*)k,
                       (const uint16_t*)v, w.kmean, w.vmean, w.khat, w.dk, w.vamax, p.M, p.Mp, p.nkt,
                       p.fp16, p.smooth_v);
  return hipGetLastError();
}

hipError_t launch_v_scale(const Problem& p, const Workspace& w, hipStream_t s) {
  hipLaunchKernelGGL(v_scale_kernel, dim3(p.BH), dim3(p.d), 0, s, w.vamax, w.dv, p.d, p.nkt);
  return hipGetLastError();
}

hipError_t launch_v_quant(const Problem& p, const void* v, const Workspace& w, hipStream_t s) {
  if (p.d == 128)
    hipLaunchKernelGGL(v_quant_kernel<128>, dim3(p.nkt, p.BH), dim3(256), 0, s, (const uint16_t*)v,
                       w.vmean, w.dv, w.vhat, p.M, p.nkt, p.fp16);
  else
    hipLaunchKernelGGL(v_quant_kernel<64>, dim3(p.nkt, p.BH), dim3(256), 0, s, (const uint16_t*)v,
                       w.vmean, w.dv, w.vhat, p.M, p.nkt, p.fp16);
  return hipGetLastError();
}

hipError_t launch_q_prep(const Problem& p, const void* q, const Workspace& w, hipStream_t s) {
  if (p.d == 128)
    hipLaunchKernelGGL(q_prep_kernel<128>, dim3(p.nqb, p.BH), dim3(256), 0, s, (const uint16_t*)q,
                       w.qhat, w.dq, w.qmean, p.N, p.Np, p.nqb, p.fp16);
  else
    hipLaunchKernelGGL(q_prep_kernel<64>, dim3(p.nqb, p.BH), dim3(256), 0, s, (const uint16_t*)q,
                       w.qhat, w.dq, w.qmean, p.N, p.Np, p.nqb, p.fp16);
  return hipGetLastError();
}

}  // namespace sage
