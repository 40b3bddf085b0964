// delta_s.hip -- the Q-smoothing correction Delta S_i[t] = q_i . gamma(K)[t] (gfx950).
//
// "SageAttention2 Technical Report" summary, 3.4 "Smoothing Q": after subtracting the
// block mean q_i from Q_i, S_ij = gamma(Q_i) gamma(K_j)^T + Delta S_ij with
// Delta S_ij = q_i gamma(K_j)^T, a 1 x b_k row per (i, j) shared by the block's rows,
// computed in higher precision than the quantized product and added after dequantization.
//
// Here it is one FP32 GEMM per head, [nqb x d] x [d x M], taken from the unquantized
// gamma(K) = fp32(K - mean(K)) so that the decomposition stays exact; summation is in channel
// order in FP32.  A work-group takes one 64-key tile and QB query blocks: gamma(K) of the
// tile and the QB means sit in LDS, each thread produces QB*64/256 outputs.  With causal
// masking only the tiles a block can see (t < 128 (i + 1)) are produced.
#include "sage_common.hpp"

namespace sage {
namespace {

constexpr int QB = 16;

template <int D>
__global__ __launch_bounds__(256) void delta_s_kernel(const uint16_t* __restrict__ K,
                                                      const float* __restrict__ kmean,
                                                      const float* __restrict__ qmean,
                                                      float* __restrict__ ds, int M, int Mp, int nqb,
                                                      int causal, bool fp16, float scale) {
  __shared__ float gk[kBK][D + 1];
  __shared__ float qm[QB][D];
  const int u = blockIdx.x, ib0 = blockIdx.y * QB, bh = blockIdx.z, tid = threadIdx.x;
  const int nib = min(QB, nqb - ib0);
  // causal: block i sees keys < 128 (i + 1); the tile is needed by blocks i >= u / 2
  if (causal && (ib0 + nib - 1) * kBQ + kBQ <= u * kBK) return;
  const size_t in_base = (size_t)bh * M * D;
  const float* km = kmean + (size_t)bh * D;
  for (int x = tid; x < kBK * D; x += 256) {
    const int t = x / D, c = x % D;
    const int key = u * kBK + t;
    gk[t][c] = (key < M) ? load_in(K, in_base + (size_t)key * D + c, fp16) - km[c] : 0.0f;
  }
  for (int x = tid; x < QB * D; x += 256) {
    const int ib = x / D, c = x % D;
    qm[ib][c] = (ib < nib) ? qmean[((size_t)bh * nqb + ib0 + ib) * D + c] : 0.0f;
  }
  __syncthreads();
  const int t = tid & 63, j0 = tid >> 6;
  for (int ib = j0; ib < nib; ib += 4) {
    const int i = ib0 + ib;
    if (causal && (i + 1) * kBQ <= u * kBK) continue;
    float s = 0.0f;
#pragma unroll 8
    for (int c = 0; c < D; c++) s = fmaf(qm[ib][c], gk[t][c], s);
    ds[((size_t)bh * nqb + i) * Mp + (size_t)u * kBK + t] = s * scale;
  }
}

}  // namespace

hipError_t launch_delta_s(const Problem& p, const void* k, const Workspace& w, float ds_scale,
                          float* ds_out, hipStream_t s) {
  dim3 grid(p.nkt, (p.nqb + QB - 1) / QB, p.BH);
  if (p.d == 128)
    hipLaunchKernelGGL(delta_s_kernel<128>, grid, dim3(256), 0, s, (const uint16_t*)k, w.kmean,
                       w.qmean, ds_out, p.M, p.Mp, p.nqb, p.causal, p.fp16, ds_scale);
  else
    hipLaunchKernelGGL(delta_s_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)k, w.kmean,
                       w.qmean, ds_out, p.M, p.Mp, p.nqb, p.causal, p.fp16, ds_scale);
  return hipGetLastError();
}

}  // namespace sage
