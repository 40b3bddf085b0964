// sagebwd.hip -- SageBwd, the trainable 8-bit attention (gfx950): preprocessing, the forward
// with the row log-sum-exp, and the backward.
//
// "SageAttention3: Microscaling FP4 Attention for Inference and An Exploration of 8-Bit
// Training" summary, "SageBwd Forward Pass: INT8 Quantization for Training" and "SageBwd
// Backward Pass and the Critical dOV^T Decision":
//   forward   K <- K - mean(K); Q (128 rows), K, V (64 keys) quantized per block to INT8;
//             S = Q^ K^T s_Q s_K sm; online softmax; P per (row, key block) to INT8 with
//             s_P = (the row's block max of P) / 127; O += P^ V^ s_P s_V;  L = m + ln l
//   backward  D = rowsum(dO o O); per (query block i, key block j): S again, P = exp(S - L),
//             P^ per block; dV_j += P^^T dO^_i;  dP = dO_i V_j^T on 16-bit inputs;
//             dS = P o (dP - D), dS^ per block;  dQ_i += dS^ K^_j;  dK_j += dS^^T Q^_i;
//             dQ += rowsum(dS) k (the smoothing term)
//
// Mapping.  Every score tile is computed transposed (S^T = K^ Q^T on v_mfma_i32_32x32x32_i8:
// a lane owns one query, 16 keys of each 32-key half), so row quantities (L, D, the running
// max) are per lane.  The P^ (forward) and dS^ (dQ kernel) bytes of a lane are then the B
// operand of an INT8 MFMA whose A operand (V^T, K^T) is stored with its keys permuted to the
// lane order (i8perm), as the FP8 P^ V^ product of the inference kernel.  The dK/dV kernel
// computes every pair's dS once: it writes P^ and dS^ key-major to LDS and contracts over the
// queries against transposed Q^ and dO^ (one 32-query step per MFMA), and leaves the pair's
// dS^ bytes (in the B-operand order of the dQ product), scale and row sums of dS in the
// workspace; the dQ kernel, launched after it, contracts those against K^ transposed.
// dP^T = V dO^T runs on the bf16 MFMA from the 16-bit inputs.
#include "attn_device.hpp"
#include "sagebwd.hpp"

namespace sage {
namespace {

using namespace attn;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_127 = 6.988684686772166f;

// Position p of a key-permuted 64-key row (i8perm) holds key 32T + 8(b/4) + 4h + b%4,
// T = p / 32, h = p / 16 % 2, b = p % 16: the key that byte b of lane half h feeds into the
// INT8 MFMA of key half T, when the B operand is a lane's 16 score-accumulator values.
__host__ __device__ inline int i8perm(int p) {
  const int T = p >> 5, h = (p >> 4) & 1, b = p & 15;
  return 32 * T + 8 * (b >> 2) + 4 * h + (b & 3);
}

// ---- per-block INT8 quantization of a [T][D] tensor of one head (Q, dO: 128 rows; K, V: 64):
// scale = max(amax, 1e-8) / 127 over the block's valid rows (K: after subtracting the mean),
// codes into the row layout [Tp][D] (rows >= T are 0) and / or the transposed layout
// [blocks][D][RB] (positions natural, or i8perm for 64-row blocks) ----
template <int D, int RB, bool PERM>
__global__ __launch_bounds__(256) void sb_quant_kernel(const uint16_t* __restrict__ src, const float* __restrict__ mean,
                                                       int8_t* __restrict__ rows, int8_t* __restrict__ trans,
                                                       float* __restrict__ scale, int T, int Tp, int nb, bool fp16) {
  constexpr int CH = RB * D / 8 / 256;  // 8-element chunks per thread
  constexpr int LS = D + 16;            // LDS code row stride (bytes)
  __shared__ __attribute__((aligned(16))) int8_t sc[RB * LS];
  __shared__ float wmax[4];
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blk * RB, n = min(RB, T - r0);
  const size_t base = ((size_t)bh * T + r0) * D;
  float x[CH][8];
  float am = 0.0f;
  v4i raws[CH];  // every chunk of the thread in flight at once (rows >= n re-read row n - 1, unused)
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int e = tid + 256 * i, r = e / (D / 8), c0 = (e % (D / 8)) * 8;
    raws[i] = *reinterpret_cast<const v4i*>(src + base + (size_t)min(r, n - 1) * D + c0);
  }
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int e = tid + 256 * i, r = e / (D / 8), c0 = (e % (D / 8)) * 8;
    if (r < n) {
      const v4i raw = raws[i];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const uint32_t u = static_cast<uint32_t>(raw[k]);
        const uint16_t lo = static_cast<uint16_t>(u & 0xffffu), hi = static_cast<uint16_t>(u >> 16);
        x[i][2 * k] = fp16 ? static_cast<float>(__builtin_bit_cast(_Float16, lo)) : __uint_as_float(u << 16);
        x[i][2 * k + 1] = fp16 ? static_cast<float>(__builtin_bit_cast(_Float16, hi)) : __uint_as_float(u & 0xffff0000u);
      }
      if (mean) {
#pragma unroll
        for (int k = 0; k < 8; k++) x[i][k] = x[i][k] - mean[(size_t)bh * D + c0 + k];
      }
#pragma unroll
      for (int k = 0; k < 8; k++) am = amax_upd(am, x[i][k]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; k++) x[i][k] = 0.0f;
    }
  }
  am = wave_max(am);
  if (lane == 0) wmax[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = int8_scale(am);
  if (tid == 0) scale[(size_t)bh * nb + blk] = s;
  const float rcp = __fdiv_rn(1.0f, s);
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int e = tid + 256 * i, r = e / (D / 8), c0 = (e % (D / 8)) * 8;
    const uint2 w = (r < n) ? int8_pack8_rcp(x[i], s, rcp) : make_uint2(0u, 0u);
    if (rows) *reinterpret_cast<uint2*>(rows + ((size_t)bh * Tp + r0 + r) * D + c0) = w;
    *reinterpret_cast<uint2*>(&sc[r * LS + c0]) = w;
  }
  if (!trans) return;
  __syncthreads();
  // transposed: 16 positions of one channel per thread step
  int8_t* tb = trans + ((size_t)bh * nb + blk) * (size_t)D * RB;
  for (int e = tid; e < D * (RB / 16); e += 256) {
    const int c = e / (RB / 16), p0 = (e % (RB / 16)) * 16;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      uint32_t v = 0;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int p = p0 + 4 * q + k;
        const int r = PERM ? i8perm(p) : p;
        v |= (uint32_t)(uint8_t)sc[r * LS + c] << (8 * k);
      }
      w[q] = v;
    }
    *reinterpret_cast<uint4*>(tb + (size_t)c * RB + p0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// An LDS tile of R rows of RB bytes, unpadded; the 16-byte chunks of a row are XOR-swizzled so
// that the 16 lanes one ds_read_b128 serves at once (16 consecutive rows, one chunk column)
// hit 16 distinct 16-byte bank groups.  Filled by LDS DMA: instruction i of wave w writes the
// tile's bytes [1024 (NPW w + i), +1024), lane l the 16-byte chunk 64 (NPW w + i) + l.
template <int R, int RB>
struct SbTile {
  static constexpr int BYTES = R * RB, CH = RB / 16, RPL = RB >= 256 ? 1 : 256 / RB, NPW = BYTES / 4096;
  static_assert(BYTES % 4096 == 0 && CH >= 4 && CH <= 16, "tile shape");
  __device__ static int swz(int r) { return (r / RPL) & (CH - 1); }
  __device__ static int off(int r, int c) { return r * RB + 16 * (c ^ swz(r)); }
  // the row and logical chunk that lane `lane` of wave w's instruction i fills
  __device__ static void src(int w, int i, int lane, int& r, int& c) {
    const int q = (NPW * w + i) * 64 + lane;
    r = q / CH;
    c = (q % CH) ^ swz(r);
  }
};

// The low bytes of four words, packed little-endian (v_perm_b32 byte selects).
__device__ __forceinline__ uint32_t sb_pack4(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
  return __builtin_amdgcn_perm(t1, t0, 0x0c0c0400u) | __builtin_amdgcn_perm(t3, t2, 0x04000c0cu);
}

struct FwdArgs {
  const int8_t* qh;  // [BH][Np][D]
  const float* sq;   // [BH][nqb]
  const int8_t* kh;  // [BH][Mp][D]
  const float* sk;   // [BH][nkt]
  const int8_t* vt;  // [BH][nkt][D][64], keys in i8perm order
  const float* sv;   // [BH][nkt]
  void* out;         // [BH][N][D]
  float* lse;        // [BH][N]
  int N, M, nqb, nkt, Np, Mp, coff;
  float qk_scale;    // sm_scale * log2(e)
};

// Work-group L of a grid of nblk blocks per head -> (head, block).  Work-groups are dealt to the
// 8 XCDs round-robin; XCD x takes whole heads x, x + 8, ... (in block order), so the operands a
// head's blocks share (its K/V tiles, or its query-side tiles) are read through one XCD's L2.
// Plain head-major order when the head count is not a multiple of 8.
__device__ __forceinline__ void sb_map(int nblk, int& bh, int& blk) {
  const int L = blockIdx.x, BH = gridDim.x / nblk;
  if (BH % kXCD == 0) {
    const int x = L % kXCD, r = L / kXCD;
    bh = x + kXCD * (r / nblk);
    blk = r % nblk;
  } else {
    bh = L / nblk;
    blk = L % nblk;
  }
}

// ---- forward: one work-group per (head, 128-query block), wave w owns queries 32w..; the key
// block's K^ rows and V^ transposed stream into a 2-slot LDS ring by DMA ----
template <int D, bool CAUSAL, int OUT>
__global__ __launch_bounds__(256, 2) void sb_fwd_kernel(FwdArgs a) {
  constexpr int NKS = D / 32;
  using TK = SbTile<kBK, D>;  // K^ rows
  using TV = SbTile<D, kBK>;  // V^ transposed, keys in i8perm order
  __shared__ __attribute__((aligned(1024))) int8_t sK[2][TK::BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sV[2][TV::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, qi;
  sb_map(a.nqb, bh, qi);
  const int qb = CAUSAL ? (a.nqb - 1 - qi) : qi;
  const int q0 = qb * kBQ, wq0 = q0 + 32 * w, qrow = wq0 + col;
  v4i qf[NKS];
  {
    const int8_t* qp = a.qh + ((size_t)bh * a.Np + qrow) * D + 16 * h;
#pragma unroll
    for (int s = 0; s < NKS; s++) qf[s] = *reinterpret_cast<const v4i*>(qp + 32 * s);
  }
  const float sqk = a.sq[(size_t)bh * a.nqb + qb] * a.qk_scale;
  v16f O[NKS];
#pragma unroll
  for (int c = 0; c < NKS; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) O[c][r] = 0.0f;
  // O and l are held relative to exp2(m_ref), a reference for the row's running max: a block's
  // contribution is scaled by exp2(rm - m_ref) / 127 instead of rescaling O whenever the max
  // rises.  m_ref moves (and O, l are rescaled) only when a block's max exceeds it by more than
  // kRefSlack, which keeps every scale below 2^kRefSlack / 127; a row's first visible block
  // always moves it.  The quotient O / l and the log-sum-exp m_ref + log2 l do not depend on it.
  constexpr float kRefSlack = 16.0f;
  float m_ref = -FLT_MAX, l_run = 0.0f;
  const int jend = CAUSAL ? max(0, min(a.nkt, (q0 + kBQ + a.coff + kBK - 1) / kBK)) : a.nkt;
  int ko[TK::NPW], vo[TV::NPW];  // per-lane DMA source offsets inside a block
#pragma unroll
  for (int i = 0; i < TK::NPW; i++) {
    int r, c;
    TK::src(w, i, lane, r, c);
    ko[i] = r * D + 16 * c;
  }
#pragma unroll
  for (int i = 0; i < TV::NPW; i++) {
    int r, c;
    TV::src(w, i, lane, r, c);
    vo[i] = r * kBK + 16 * c;
  }
  auto dma = [&](int j, int b) {
    const int8_t* kt = a.kh + ((size_t)bh * a.Mp + (size_t)j * kBK) * D;
    const int8_t* vt = a.vt + ((size_t)bh * a.nkt + j) * (size_t)D * kBK;
#pragma unroll
    for (int i = 0; i < TK::NPW; i++) dma16(lds_addr(&sK[b][(TK::NPW * w + i) * 1024]), kt, ko[i]);
#pragma unroll
    for (int i = 0; i < TV::NPW; i++) dma16(lds_addr(&sV[b][(TV::NPW * w + i) * 1024]), vt, vo[i]);
  };
  // The blocks' K^ and V^ scales: loads that the kernel's own stores might alias, so the compiler
  // issues them as vector loads.  Each block's pair is loaded during the block before it; empty
  // uses put the compiler's waits for these (and for the Q^ rows) before the DMAs, so that no
  // wait of its own inside a block can also hold on the next block's DMA.
  float skn = 0.0f, svn = 0.0f;
  if (jend > 0) {
    skn = a.sk[(size_t)bh * a.nkt];
    svn = a.sv[(size_t)bh * a.nkt];
  }
#pragma unroll
  for (int s = 0; s < NKS; s++) asm volatile("" ::"v"(qf[s]));
  asm volatile("" ::"v"(sqk));
  if (jend > 0) dma(0, 0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // block 0 landed
  for (int j = 0; j < jend; j++) {
    const int b = j & 1;
    const float skj = skn, svj = svn;  // this block's scales
    asm volatile("" ::"v"(skj), "v"(svj));
    if (j + 1 < jend) dma(j + 1, b ^ 1);  // the slot block j-1 left (freed by the last barrier)
    {  // the next block's scales (the last block reloads its own)
      const int jn = j + 1 < jend ? j + 1 : j;
      skn = a.sk[(size_t)bh * a.nkt + jn];
      svn = a.sv[(size_t)bh * a.nkt + jn];
    }
    const int key0 = j * kBK;
    if (!(CAUSAL && key0 > wq0 + 31 + a.coff)) {  // else every key of the block is masked for this wave
      const int8_t* cK = sK[b];
      const int8_t* cV = sV[b];
      v16i acc[2];
#pragma unroll
      for (int T = 0; T < 2; T++) {
#pragma unroll
        for (int r = 0; r < 16; r++) acc[T][r] = 0;
#pragma unroll
        for (int s = 0; s < NKS; s++) {
          const v4i kf = *reinterpret_cast<const v4i*>(&cK[TK::off(32 * T + col, 2 * s + h)]);
          acc[T] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[s], acc[T], 0, 0, 0);
        }
      }
      const float mul = sqk * skj;
      float sc[2][16];
      int lim = a.M - 1 - key0;
      if (CAUSAL) lim = min(lim, qrow + a.coff - key0);
      lim -= 4 * h;
      float rm = -INFINITY;
      // boundary blocks only (keys past M, or after a query of the wave): the per-score test
      const bool masked = key0 + kBK > a.M || (CAUSAL && key0 + kBK - 1 > wq0 + a.coff);
      // sc holds the exact integer scores (|acc| < 2^24); S = sc * mul.  As mul > 0 and rounding
      // is monotonic, the row's max of the rounded products is the rounded product of its max,
      // and the exponent takes S - base in one FMA.
#pragma unroll
      for (int T = 0; T < 2; T++)
#pragma unroll
        for (int r = 0; r < 16; r++) sc[T][r] = (float)acc[T][r];
      if (masked) {
        asm volatile("" ::: "memory");  // keep this a real branch: interior blocks skip the test
#pragma unroll
        for (int T = 0; T < 2; T++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            sc[T][r] = (32 * T + 8 * (r >> 2) + (r & 3) <= lim) ? sc[T][r] : -INFINITY;
      }
#pragma unroll
      for (int T = 0; T < 2; T++)
#pragma unroll
        for (int r = 0; r < 16; r++) rm = fmaxf(rm, sc[T][r]);
      rm = pair_max(rm) * mul;  // the row's max of S over this tile
      if (__any(rm > m_ref + kRefSlack)) {  // some row of the wave moves its reference
        const float m_new = rm > m_ref + kRefSlack ? rm : m_ref;
        const float alpha = fast_exp2(m_ref - m_new);  // 1 for the rows that keep theirs
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < NKS; c++)
#pragma unroll
          for (int r = 0; r < 16; r++) O[c][r] *= alpha;
      }
      // e = 127 P / (the row's block max of P) = 127 exp2(S - rm); P^ = rne(e)
      const float base = (rm == -INFINITY) ? 0.0f : rm - kLog2_127;
      float esum = 0.0f;
      v4i pb[2];
#pragma unroll
      for (int T = 0; T < 2; T++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          // e in [0, 127]: the byte conversion rounds half to even and packs byte k of the word
          uint32_t wd = 0;
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const float e = fast_exp2(fmaf(sc[T][4 * q4 + k], mul, -base));
            esum += e;
            wd = __builtin_amdgcn_cvt_pk_u8_f32(e, k, wd);
          }
          pb[T][q4] = (int)wd;
        }
      esum = pair_sum(esum);
      // s_P = exp2(rm - m) / 127 against the running max m, here against m_ref
      const float sp = (rm == -INFINITY) ? 0.0f : fast_exp2(rm - m_ref) * (1.0f / 127.0f);
      l_run = fmaf(esum, sp, l_run);
      const float osc = sp * svj;
#pragma unroll
      for (int c = 0; c < NKS; c++) {
        v16i R;
#pragma unroll
        for (int r = 0; r < 16; r++) R[r] = 0;
#pragma unroll
        for (int T = 0; T < 2; T++) {
          const v4i vf = *reinterpret_cast<const v4i*>(&cV[TV::off(32 * c + col, 2 * T + h)]);
          R = __builtin_amdgcn_mfma_i32_32x32x32_i8(vf, pb[T], R, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) O[c][r] = fmaf((float)R[r], osc, O[c][r]);
      }
    }
    // block j+1 landed (this wave's DMAs, then everyone's); slot b may be refilled
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (qrow >= a.N) return;
  const float inv = 1.0f / l_run;
  if (h == 0) a.lse[(size_t)bh * a.N + qrow] = (m_ref + __log2f(l_run)) * kLn2;
  const size_t orow = ((size_t)bh * a.N + qrow) * D;
#pragma unroll
  for (int c = 0; c < NKS; c++)
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ch = 32 * c + 8 * b + 4 * h;
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; k++) o[k] = O[c][4 * b + k] * inv;
      store_out4<OUT>(a.out, orow + ch, o);
    }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// One 32x32x16 step of dP^T = V dO^T on the MFMA of the input type (bf16 or fp16).
template <bool FP16>
__device__ __forceinline__ v16f mfma16(const v4i& a, const v4i& b, const v16f& c) {
  if constexpr (FP16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                   0);
}

// 8 consecutive 16-bit inputs (bf16 or fp16) widened to FP32.
__device__ __forceinline__ void sb_widen8(const v4i& raw, bool fp16, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const uint32_t u = static_cast<uint32_t>(raw[e]);
    if (fp16) {
      x[2 * e] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
      x[2 * e + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
    } else {
      x[2 * e] = __uint_as_float(u << 16);
      x[2 * e + 1] = __uint_as_float(u & 0xffff0000u);
    }
  }
}

// ---- backward preprocessing: D = rowsum(dO o O) (FP64 sum), L2 = L log2(e); padded rows
// get D = 0 and L2 = +inf (their P is 0).  A row is spread over D/8 lanes holding 8
// consecutive channels each (16- or 32-byte loads); every load of the thread's rows is issued
// before any is used, and the lanes' FP64 partial sums meet in a butterfly. ----
template <int D, int OUT>
__global__ __launch_bounds__(256) void sb_dprep_kernel(const void* __restrict__ out, const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ Dr,
                                                       float* __restrict__ L2, int N, int Np, bool fp16) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPP = 256 / LPR;      // rows per pass
  constexpr int NP = kBQ / RPP;       // passes per 128-row block
  const int tid = threadIdx.x, bh = blockIdx.y, sub = tid / LPR, cl = tid % LPR;
  v4i rd[NP], ro[NP], ro2[NP];
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int row = min(blockIdx.x * kBQ + p * RPP + sub, N - 1);  // rows >= N: a valid row, not used
    const size_t base = ((size_t)bh * N + row) * D + 8 * cl;
    rd[p] = *reinterpret_cast<const v4i*>(dout + base);
    if constexpr (OUT == 2) {
      ro[p] = *reinterpret_cast<const v4i*>(reinterpret_cast<const float*>(out) + base);
      ro2[p] = *reinterpret_cast<const v4i*>(reinterpret_cast<const float*>(out) + base + 4);
    } else {
      ro[p] = *reinterpret_cast<const v4i*>(reinterpret_cast<const uint16_t*>(out) + base);
    }
  }
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int row = blockIdx.x * kBQ + p * RPP + sub;
    float dv[8], ov[8];
    sb_widen8(rd[p], fp16, dv);
    if constexpr (OUT == 2) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        ov[e] = __int_as_float(ro[p][e]);
        ov[4 + e] = __int_as_float(ro2[p][e]);
      }
    } else {
      sb_widen8(ro[p], OUT == 1, ov);
    }
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < 8; e++) s += (double)dv[e] * (double)ov[e];
#pragma unroll
    for (int x = 1; x < LPR; x <<= 1) s += __shfl_xor(s, x);
    if (cl == 0) {
      const size_t o = (size_t)bh * Np + row;
      Dr[o] = row < N ? (float)s : 0.0f;
      L2[o] = row < N ? lse[(size_t)bh * N + row] * kLog2e : INFINITY;
    }
  }
}

struct BwdArgs {
  const int8_t* qh;    // [BH][Np][D] Q^ rows
  const int8_t* qt;    // [BH][nqb][D][128] Q^ transposed
  const float* sq;     // [BH][nqb]
  const int8_t* kh;    // [BH][Mp][D] K^ rows
  const int8_t* kt;    // [BH][nkt][D][64] K^ transposed, keys in i8perm order
  const float* sk;     // [BH][nkt]
  const int8_t* dot;   // [BH][nqb][D][128] dO^ transposed
  const float* sdo;    // [BH][nqb]
  const float* Dr;     // [BH][Np]
  const float* L2;     // [BH][Np]
  const float* kmean;  // [BH][D] (null: K not smoothed)
  const uint16_t* V;   // [BH][M][D] 16-bit
  const uint16_t* dO;  // [BH][N][D] 16-bit
  float* dq;           // [BH][N][D]
  float* dk;           // [BH][M][D]
  float* dv;           // [BH][M][D]
  // dS^ of each (128-query block i, 64-key block j) pair, written by the dK/dV kernel and
  // contracted by the dQ kernel: pair (i, j) of head bh is p = (bh nqb + i) nkt + j, one
  // kSbRec-byte record per pair and wave (the wave's 32 queries)
  int8_t* dsh;         // [pairs][4 waves][kSbRec]
  int N, M, nqb, nkt, Np, Mp, coff;
  float qk_scale;      // sm_scale * log2(e)
  float sm;            // sm_scale
};

// The elementwise part shared by both backward kernels, for one wave's 32 queries (lane = query,
// 16 keys per 32-key half): S^T from K^ / Q^ fragments, P = exp2(S - L2), dP^T = V dO^T on the
// bf16 MFMA from the 16-bit V tile in LDS, dS = P (dP - D).  Masked pairs give P = dS = 0.
// vfrag(T, s): the lane's 16 bytes (8 values, channels 16 s + 8 h ..) of V row 32 T + col.
// masked (wave-uniform): some key of the block is past M or after a query of the wave (causal);
// otherwise every pair is visible and the per-pair test is skipped.
template <int D, bool FP16, typename VF>
__device__ __forceinline__ void sb_pair(const v4i (&kf)[2][D / 32], const v4i (&qf)[D / 32], const v4i (&of)[D / 16],
                                        VF&& vfrag, float mul, float l2, float dr, bool masked,
                                        int lim, int h, int col, float (&P)[2][16], float (&dS)[2][16]) {
#pragma unroll
  for (int T = 0; T < 2; T++) {
    v16i acc;
#pragma unroll
    for (int r = 0; r < 16; r++) acc[r] = 0;
#pragma unroll
    for (int s = 0; s < D / 32; s++) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[T][s], qf[s], acc, 0, 0, 0);
    v16f dp;
#pragma unroll
    for (int r = 0; r < 16; r++) dp[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
      dp = mfma16<FP16>(vfrag(T, s), of[s], dp);
    }
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const bool vis = 32 * T + 8 * (r >> 2) + (r & 3) <= lim;
        const float p = vis ? fast_exp2((float)acc[r] * mul - l2) : 0.0f;
        P[T][r] = p;
        dS[T][r] = vis ? p * (dp[r] - dr) : 0.0f;  // a masked key's V row may be a stand-in
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float p = fast_exp2((float)acc[r] * mul - l2);
        P[T][r] = p;
        dS[T][r] = p * (dp[r] - dr);
      }
    }
  }
}

// Block maxima of P and |dS| over the work-group's 128 x 64 block (4 waves; one barrier; xs is
// rewritten only after the caller's next barrier).
__device__ __forceinline__ void sb_block_max(float pm, float dm, float* xs, int lane, int w, float& pmax, float& dmax) {
  pm = wave_max(pm);
  dm = wave_max(dm);
  if (lane == 0) {
    xs[w] = pm;
    xs[4 + w] = dm;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // LDS only: tile DMAs stay in flight
  pmax = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3]));
  dmax = fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7]));
}

// The block maximum of |dS| alone (the dQ kernel quantizes only dS); same barrier and slots.
__device__ __forceinline__ float sb_block_max_ds(float dm, float* xs, int lane, int w) {
  dm = wave_max(dm);
  if (lane == 0) xs[4 + w] = dm;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // LDS only: tile DMAs stay in flight
  return fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7]));
}

// INT8 code of x against 127 / amax (inv = 0: the block is all zero), in the low byte of the
// result: the product plus 1.5 * 2^23 holds its round-half-even integer in the low mantissa bits
// (no convert).  Every caller quantizes a block against its own maximum, |x| <= amax, and
// inv = rn(127 / amax), so |x * inv| <= 127 (1 + 2^-24)^2, which rounds to 127: the clamp to
// [-127, 127] the codes are defined with never acts on finite values and is left out.
__device__ __forceinline__ uint32_t sb_code8(float x, float inv) {
  return __float_as_uint(fmaf(x, inv, 12582912.0f));
}

// The 16-bit rows of one 64-key V tile into LDS (rows >= M are 0).
template <int D>
__device__ __forceinline__ void sb_load_v(const uint16_t* __restrict__ V, int M, int t0, uint16_t* sVb, int vs, int tid) {
  for (int e = tid; e < kBK * D / 8; e += 256) {
    const int r = e / (D / 8), c = (e % (D / 8)) * 8;
    v4i x = {0, 0, 0, 0};
    if (t0 + r < M) x = *reinterpret_cast<const v4i*>(V + (size_t)(t0 + r) * D + c);
    *reinterpret_cast<v4i*>(sVb + r * vs + c) = x;
  }
}

// The fragments of one query row: Q^ (INT8 MFMA B operand) and dO (bf16 MFMA B operand).
template <int D>
__device__ __forceinline__ void sb_q_frags(const BwdArgs& a, int bh, int qrow, int h, v4i (&qf)[D / 32],
                                           v4i (&of)[D / 16]) {
  const int8_t* qp = a.qh + ((size_t)bh * a.Np + qrow) * D + 16 * h;
#pragma unroll
  for (int s = 0; s < D / 32; s++) qf[s] = *reinterpret_cast<const v4i*>(qp + 32 * s);
  // rows past N (the last block's padding) read row 0 instead: every lane issues the same loads,
  // and the loaded values cannot matter, since such a row's P is exactly 0 (its log-sum-exp is
  // stored as +inf) and its dS = P (dP - 0) with dP finite
  const uint16_t* op = a.dO + ((size_t)bh * a.N + (qrow < a.N ? qrow : 0)) * D + 8 * h;
#pragma unroll
  for (int s = 0; s < D / 16; s++) of[s] = *reinterpret_cast<const v4i*>(op + 16 * s);
}
// Vector memory loads of one query block's prefetch in the dK / dV kernel: sb_q_frags, the two
// row scalars and the block's two scales.  Its barrier waits for everything issued before them.
template <int D>
constexpr int kSbRowLoads = D / 32 + D / 16 + 4;

// dQ of one lane's query row (channels 32 c + 8 b + 4 h + k), with the K-mean term
// sm rowsum(dS) mean(K) when K was smoothed.  Each channel group's K-mean loads are issued
// before its stores (which the compiler must otherwise order after every possibly aliasing store).
template <int D>
__device__ __forceinline__ void sb_dq_store(const BwdArgs& a, int bh, int qrow, int h, float rs,
                                            const v16f (&dq)[D / 32]) {
  const size_t orow = ((size_t)bh * a.N + qrow) * D;
#pragma unroll
  for (int c = 0; c < D / 32; c++) {
    float4 km4[4] = {};
    if (a.kmean)
#pragma unroll
      for (int b = 0; b < 4; b++)
        km4[b] = *reinterpret_cast<const float4*>(a.kmean + (size_t)bh * D + 32 * c + 8 * b + 4 * h);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ch = 32 * c + 8 * b + 4 * h;
      const float kmv[4] = {km4[b].x, km4[b].y, km4[b].z, km4[b].w};
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; k++) o[k] = a.kmean ? fmaf(a.sm * rs, kmv[k], dq[c][4 * b + k]) : dq[c][4 * b + k];
      store_out4<2>(a.dq, orow + ch, o);
    }
  }
}

// ---- dQ with dS recomputed (SAGE_TRAIN_RECOMPUTE_DS, or a pair buffer beyond kSbPairLimit):
// one work-group per (head, 128-query block); loops over the key blocks.  The key block's K^
// rows, K^ transposed and 16-bit V rows stream into a 2-slot LDS ring by DMA: block j+1 is in
// flight while block j is computed, one barrier per block publishes the next.  S, P, dP and dS
// come from the same elementwise part as in the dK/dV kernel, so both see the same dS^ ----
template <int D, bool CAUSAL, bool FP16>
__global__ __launch_bounds__(256, 2) void sb_dq_recompute_kernel(BwdArgs a) {
  constexpr int NKS = D / 32;
  using TK = SbTile<kBK, D>;      // K^ rows
  using TT = SbTile<D, kBK>;      // K^ transposed, keys in i8perm order
  using TV = SbTile<kBK, 2 * D>;  // V rows, 16-bit
  __shared__ __attribute__((aligned(1024))) int8_t sK[2][TK::BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sKt[2][TT::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sVb[2][TV::BYTES];
  __shared__ float xs[8];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, qi;
  sb_map(a.nqb, bh, qi);
  const int qb = CAUSAL ? (a.nqb - 1 - qi) : qi;
  const int q0 = qb * kBQ, qrow = q0 + 32 * w + col;
  v4i qf[NKS];
  v4i of[D / 16];
  sb_q_frags<D>(a, bh, qrow, h, qf, of);
  const float l2 = a.L2[(size_t)bh * a.Np + qrow], dr = a.Dr[(size_t)bh * a.Np + qrow];
  const float sq = a.sq[(size_t)bh * a.nqb + qb];
  v16f dq[NKS];
#pragma unroll
  for (int c = 0; c < NKS; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) dq[c][r] = 0.0f;
  float rs = 0.0f;
  const int jend = CAUSAL ? max(0, min(a.nkt, (q0 + kBQ + a.coff + kBK - 1) / kBK)) : a.nkt;

  // per-lane DMA source offsets inside a block (V: row and byte column; its rows are clamped to
  // the last key, a stand-in for keys >= M, whose P and dS are 0)
  int ko[TK::NPW], to[TT::NPW], vr[TV::NPW], vc[TV::NPW];
#pragma unroll
  for (int i = 0; i < TK::NPW; i++) {
    int r, c;
    TK::src(w, i, lane, r, c);
    ko[i] = r * D + 16 * c;
  }
#pragma unroll
  for (int i = 0; i < TT::NPW; i++) {
    int r, c;
    TT::src(w, i, lane, r, c);
    to[i] = r * kBK + 16 * c;
  }
#pragma unroll
  for (int i = 0; i < TV::NPW; i++) {
    int r, c;
    TV::src(w, i, lane, r, c);
    vr[i] = r;
    vc[i] = 16 * c;
  }
  auto dma = [&](int j, int b) {
    const int8_t* kr = a.kh + ((size_t)bh * a.Mp + (size_t)j * kBK) * D;
    const int8_t* kt = a.kt + ((size_t)bh * a.nkt + j) * (size_t)D * kBK;
    const uint16_t* vb = a.V + ((size_t)bh * a.M + (size_t)j * kBK) * D;
    const int vlast = a.M - 1 - j * kBK;  // >= 0: block j holds a key
#pragma unroll
    for (int i = 0; i < TK::NPW; i++) dma16(lds_addr(&sK[b][(TK::NPW * w + i) * 1024]), kr, ko[i]);
#pragma unroll
    for (int i = 0; i < TT::NPW; i++) dma16(lds_addr(&sKt[b][(TT::NPW * w + i) * 1024]), kt, to[i]);
#pragma unroll
    for (int i = 0; i < TV::NPW; i++)
      dma16(lds_addr(&sVb[b][(TV::NPW * w + i) * 1024]), vb, min(vr[i], vlast) * (2 * D) + vc[i]);
  };
  if (jend > 0) dma(0, 0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // block 0 landed
  for (int j = 0; j < jend; j++) {
    const int b = j & 1;
    if (j + 1 < jend) dma(j + 1, b ^ 1);  // the slot block j-1 left (freed by the last barrier)
    const int8_t* cK = sK[b];
    const int8_t* cKt = sKt[b];
    const uint8_t* cV = sVb[b];
    v4i kf[2][NKS];
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int s = 0; s < NKS; s++) kf[T][s] = *reinterpret_cast<const v4i*>(&cK[TK::off(32 * T + col, 2 * s + h)]);
    const int key0 = j * kBK;
    int lim = a.M - 1 - key0;
    if (CAUSAL) lim = min(lim, qrow + a.coff - key0);
    lim -= 4 * h;
    float P[2][16], dS[2][16];
    auto vfrag = [&](int T, int s) {
      return *reinterpret_cast<const v4i*>(&cV[TV::off(32 * T + col, 2 * s + h)]);
    };
    const bool masked = key0 + kBK > a.M || (CAUSAL && key0 + kBK - 1 > q0 + 32 * w + a.coff);
    sb_pair<D, FP16>(kf, qf, of, vfrag, sq * a.sk[(size_t)bh * a.nkt + j] * a.qk_scale, l2, dr, masked, lim, h, col, P,
                     dS);
    float dm = 0.0f;
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        dm = fmaxf(dm, fabsf(dS[T][r]));
        rs += dS[T][r];
      }
    const float dmax = sb_block_max_ds(dm, xs, lane, w);
    const float inv = dmax > 0.0f ? __fdiv_rn(127.0f, dmax) : 0.0f;
    const float sds = __fdiv_rn(dmax, 127.0f);
    v4i db[2];
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        db[T][q4] = (int)sb_pack4(sb_code8(dS[T][4 * q4 + 0], inv), sb_code8(dS[T][4 * q4 + 1], inv),
                                  sb_code8(dS[T][4 * q4 + 2], inv), sb_code8(dS[T][4 * q4 + 3], inv));
      }
    const float osc = sds * a.sk[(size_t)bh * a.nkt + j] * a.sm;
#pragma unroll
    for (int c = 0; c < NKS; c++) {
      v16i R;
#pragma unroll
      for (int r = 0; r < 16; r++) R[r] = 0;
#pragma unroll
      for (int T = 0; T < 2; T++) {
        const v4i kt = *reinterpret_cast<const v4i*>(&cKt[TT::off(32 * c + col, 2 * T + h)]);
        R = __builtin_amdgcn_mfma_i32_32x32x32_i8(kt, db[T], R, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; r++) dq[c][r] = fmaf((float)R[r], osc, dq[c][r]);
    }
    // block j+1 landed (this wave's DMAs, then everyone's); slot b may be refilled
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  rs = pair_sum(rs);
  if (qrow >= a.N) return;
  sb_dq_store<D>(a, bh, qrow, h, rs, dq);
}

// ---- dQ: one work-group per (head, 128-query block); loops over the key blocks.  The dK/dV
// kernel (launched first) leaves, per pair and wave, a record of the dS^ codes in this kernel's
// B-operand order, the per-query sums of dS and the pair's multiplier; here
// dQ = sum_j dS^_j K^_j (max|dS_j| / 127) s_j sm_scale contracts them against the key block's K^
// transposed.  Both stream in by DMA: K^ transposed through a 2-slot LDS ring (block j+1 in
// flight while block j is used), the records through a 3-slot one (record j+2 in flight), one
// barrier per block; no wait inside a block holds on memory ----
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 3) void sb_dq_kernel(BwdArgs a) {
  constexpr int NKS = D / 32;
  using TT = SbTile<D, kBK>;  // K^ transposed, keys in i8perm order
  __shared__ __attribute__((aligned(1024))) int8_t sKt[2][TT::BYTES];
  // a 3-slot ring of the pairs' records, one kSbRecLds-byte slot per wave: the record of pair j+2
  // streams in while pair j is contracted (and pair j+1's, already landed, waits)
  __shared__ __attribute__((aligned(1024))) int8_t sRec[3][4][kSbRecLds];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, qi;
  sb_map(a.nqb, bh, qi);
  const int qb = CAUSAL ? (a.nqb - 1 - qi) : qi;
  const int q0 = qb * kBQ, qrow = q0 + 32 * w + col;
  v16f dq[NKS];
#pragma unroll
  for (int c = 0; c < NKS; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) dq[c][r] = 0.0f;
  float rs = 0.0f;
  // the key blocks this query block attends to (the pairs the dK/dV kernel wrote)
  const int jend = CAUSAL ? max(0, min(a.nkt, (q0 + kBQ + a.coff + kBK - 1) / kBK)) : a.nkt;
  int to[TT::NPW];  // per-lane DMA source offsets inside a block
#pragma unroll
  for (int i = 0; i < TT::NPW; i++) {
    int r, c;
    TT::src(w, i, lane, r, c);
    to[i] = r * kBK + 16 * c;
  }
  const uint32_t lds0 = lds_addr(&sKt[0][TT::NPW * w * 1024]), lds1 = lds_addr(&sKt[1][TT::NPW * w * 1024]);
  auto dma = [&](int j, int b) {
    const int8_t* kt = a.kt + ((size_t)bh * a.nkt + j) * (size_t)D * kBK;
    const uint32_t base = b ? lds1 : lds0;
#pragma unroll
    for (int i = 0; i < TT::NPW; i++) dma16(base + 1024 * i, kt, to[i]);
  };
  // this wave's record of pair (qb, jj) into ring slot r: the codes (two 1 KiB halves), then the
  // row sums (lanes 0-31) and the pair's multiplier (lanes 32-63 all fetch it): three DMAs
  const int8_t* rbase = a.dsh + (((size_t)bh * a.nqb + qb) * a.nkt * 4 + w) * kSbRec;
  const uint32_t rec0 = lds_addr(&sRec[0][w][0]);
  const uint32_t tail_off = lane < 32 ? 2048 + 4 * lane : 2048 + 4 * 32;
  auto fetch = [&](int jj, int r) {
    const int8_t* g = rbase + (size_t)jj * 4 * kSbRec;
    const uint32_t l = rec0 + (uint32_t)r * 4 * kSbRecLds;
    dma16(l, g, 16 * lane);
    dma16(l + 1024, g, 1024 + 16 * lane);
    dma4(l + 2048, g, tail_off);
  };
  if (jend > 0) {
    dma(0, 0);
    fetch(0, 0);
    fetch(min(1, jend - 1), 1);
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // block 0 and records 0, 1 landed
  int r = 0;  // ring slot of pair j's record
  for (int j = 0; j < jend; j++) {
    const int b = j & 1;
    if (j + 1 < jend) dma(j + 1, b ^ 1);  // the slot block j-1 left (freed by the last barrier)
    // pair j+2's record (the last pairs fetch pair jend-1 again, into a slot nobody reads) into the
    // slot pair j-1 left; always three DMAs, which the wait below leaves in flight
    fetch(min(j + 2, jend - 1), r == 0 ? 2 : r - 1);
    const int8_t* rec = &sRec[r][w][0];
    const v4i db0 = *reinterpret_cast<const v4i*>(rec + 16 * lane);
    const v4i db1 = *reinterpret_cast<const v4i*>(rec + 1024 + 16 * lane);
    const float* tail = reinterpret_cast<const float*>(rec + 2048);
    rs += tail[col];
    const float osc = tail[32];  // (max|dS| / 127) s_K sm_scale
    const int8_t* cKt = sKt[b];
#pragma unroll
    for (int c = 0; c < NKS; c++) {
      v16i R;
#pragma unroll
      for (int rr = 0; rr < 16; rr++) R[rr] = 0;
      const v4i kt0 = *reinterpret_cast<const v4i*>(&cKt[TT::off(32 * c + col, h)]);
      const v4i kt1 = *reinterpret_cast<const v4i*>(&cKt[TT::off(32 * c + col, 2 + h)]);
      R = __builtin_amdgcn_mfma_i32_32x32x32_i8(kt0, db0, R, 0, 0, 0);
      R = __builtin_amdgcn_mfma_i32_32x32x32_i8(kt1, db1, R, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 16; rr++) dq[c][rr] = fmaf((float)R[rr], osc, dq[c][rr]);
    }
    r = r == 2 ? 0 : r + 1;
    // block j+1 and record j+1 landed (this wave's DMAs, then everyone's; only the three of
    // record j+2, issued last, may still be in flight); slot b and record slot r-1 may be refilled
    asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // no DMA may still write this work-group's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (qrow >= a.N) return;
  sb_dq_store<D>(a, bh, qrow, h, rs, dq);
}

// ---- dK, dV: one work-group per (head, 64-key block); loops over the query blocks.  P^ and
// dS^ of a pair go to LDS key-major; wave w then owns key half w % 2 and half of the channel
// groups of both outputs, and contracts over the block's 128 queries ----
template <int D, bool CAUSAL, bool FP16, bool STORE>
__global__ __launch_bounds__(256, 2) void sb_dkv_kernel(BwdArgs a) {
  constexpr int NKS = D / 32, NG = NKS / 2, VS = D + 8, PS = kBQ + 16;
  using TQ = SbTile<D, kBQ>;  // dO^ and Q^ transposed: [channel][query] of one query block
  __shared__ __attribute__((aligned(16))) uint16_t sVb[kBK * VS];
  __shared__ __attribute__((aligned(16))) int8_t sP[kBK * PS];
  __shared__ __attribute__((aligned(16))) int8_t sD[kBK * PS];
  __shared__ __attribute__((aligned(1024))) int8_t sOt[TQ::BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sQt[TQ::BYTES];
  __shared__ float xs[8];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, j;
  sb_map(a.nkt, bh, j);
  const int key0 = j * kBK;
  sb_load_v<D>(a.V + (size_t)bh * a.M * D, a.M, key0, sVb, VS, tid);
  v4i kf[2][NKS];
  {
    const int8_t* kr = a.kh + ((size_t)bh * a.Mp + key0) * D;
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int s = 0; s < NKS; s++)
        kf[T][s] = *reinterpret_cast<const v4i*>(kr + (size_t)(32 * T + col) * D + 32 * s + 16 * h);
  }
  const float skj = a.sk[(size_t)bh * a.nkt + j];
  // this wave's output tiles, of both dV and dK: key half Tw, channel groups c0 .. c0 + NG - 1
  const int Tw = w & 1, c0 = (w >> 1) * NG;
  v16f accV[NG], accK[NG];
#pragma unroll
  for (int g = 0; g < NG; g++)
#pragma unroll
    for (int r = 0; r < 16; r++) accV[g][r] = accK[g][r] = 0.0f;
  int to[TQ::NPW];  // per-lane DMA source offsets inside a transposed block
#pragma unroll
  for (int x = 0; x < TQ::NPW; x++) {
    int r, c;
    TQ::src(w, x, lane, r, c);
    to[x] = r * kBQ + 16 * c;
  }
  // LDS addresses of this wave's DMA destinations (scalars)
  const uint32_t ot_lds = lds_addr(&sOt[TQ::NPW * w * 1024]), qt_lds = lds_addr(&sQt[TQ::NPW * w * 1024]);
  const int ilo = CAUSAL ? max(0, (key0 - a.coff) / kBQ) : 0;
  // this wave's query rows of the first block; each later block's rows are loaded while the
  // block before it is contracted into dV and dK
  // (with the block's Q^ and dO^ scales: loads that the kernel's own stores might alias, so the
  // compiler issues them as vector loads, which must not be waited for next to the DMAs)
  v4i qf[NKS];
  v4i of[D / 16];
  float l2 = 0.0f, dr = 0.0f, sqb = 0.0f, sdob = 0.0f;
  if (ilo < a.nqb) {
    const int qr = ilo * kBQ + 32 * w + col;
    sb_q_frags<D>(a, bh, qr, h, qf, of);
    l2 = a.L2[(size_t)bh * a.Np + qr];
    dr = a.Dr[(size_t)bh * a.Np + qr];
    sqb = a.sq[(size_t)bh * a.nqb + ilo];
    sdob = a.sdo[(size_t)bh * a.nqb + ilo];
  }
  for (int i = ilo; i < a.nqb; i++) {
    __syncthreads();  // the previous pair's LDS reads are done (and V is staged, i = ilo)
    // the block's rows and scales, loaded during the previous block: an empty use here puts the
    // compiler's wait for them before the DMAs below, so that the wait cannot also hold on those
#pragma unroll
    for (int s = 0; s < NKS; s++) asm volatile("" ::"v"(qf[s]));
#pragma unroll
    for (int s = 0; s < D / 16; s++) asm volatile("" ::"v"(of[s]));
    asm volatile("" ::"v"(l2), "v"(dr), "v"(sqb), "v"(sdob));
    const float sqi = sqb, sdoi = sdob;  // this block's Q^ and dO^ scales
    const int q0 = i * kBQ, qrow = q0 + 32 * w + col;
    {
      // the block's dO^ and Q^ transposed for the dV / dK products, by DMA: they land while the
      // scores and gradients of the block are computed (issued after this wave's row loads)
      const int8_t* dob = a.dot + ((size_t)bh * a.nqb + i) * (size_t)D * kBQ;
      const int8_t* qtb = a.qt + ((size_t)bh * a.nqb + i) * (size_t)D * kBQ;
#pragma unroll
      for (int x = 0; x < TQ::NPW; x++) dma16(ot_lds + 1024 * x, dob, to[x]);
#pragma unroll
      for (int x = 0; x < TQ::NPW; x++) dma16(qt_lds + 1024 * x, qtb, to[x]);
    }
    int lim = a.M - 1 - key0;
    if (CAUSAL) lim = min(lim, qrow + a.coff - key0);
    lim -= 4 * h;
    float P[2][16], dS[2][16];
    // the score multiplier in the dQ kernel's order, so that both kernels see the same P and dS
    auto vfrag = [&](int T, int s) {
      return *reinterpret_cast<const v4i*>(sVb + (32 * T + col) * VS + 16 * s + 8 * h);
    };
    const bool masked = key0 + kBK > a.M || (CAUSAL && key0 + kBK - 1 > q0 + 32 * w + a.coff);
    sb_pair<D, FP16>(kf, qf, of, vfrag, sqi * skj * a.qk_scale, l2, dr, masked, lim, h, col, P, dS);
    {  // the next block's rows and scales (the last block reloads its own), issued as soon as the
       // products above have read these: in flight through the block maxima, the codes and dV / dK
      const int in = i + 1 < a.nqb ? i + 1 : i;
      const int qn = in * kBQ + 32 * w + col;
      sb_q_frags<D>(a, bh, qn, h, qf, of);
      l2 = a.L2[(size_t)bh * a.Np + qn];
      dr = a.Dr[(size_t)bh * a.Np + qn];
      sqb = a.sq[(size_t)bh * a.nqb + in];
      sdob = a.sdo[(size_t)bh * a.nqb + in];
    }
    float pm = 0.0f, dm = 0.0f;
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        pm = fmaxf(pm, P[T][r]);
        dm = fmaxf(dm, fabsf(dS[T][r]));
      }
    float pmax, dmax;
    sb_block_max(pm, dm, xs, lane, w, pmax, dmax);
    const float pinv = pmax > 0.0f ? __fdiv_rn(127.0f, pmax) : 0.0f;
    const float dinv = dmax > 0.0f ? __fdiv_rn(127.0f, dmax) : 0.0f;
    // P^, dS^ key-major: byte [key][query]; dS^ also to the pair's buffer for the dQ kernel (the
    // lane's 32 codes as its B operand: 16 bytes per 32-key half), with the scale and the row sum
    const int qc = 32 * w + col;
    const size_t pr = ((size_t)bh * a.nqb + i) * a.nkt + j;
    float rsp = 0.0f;
    v4i db[2];
#pragma unroll
    for (int T = 0; T < 2; T++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        uint32_t dc[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int r = 4 * q4 + e;
          const int key = 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
          sP[key * PS + qc] = (int8_t)sb_code8(P[T][r], pinv);
          dc[e] = sb_code8(dS[T][r], dinv);
          sD[key * PS + qc] = (int8_t)dc[e];
          rsp += dS[T][r];
        }
        db[T][q4] = (int)sb_pack4(dc[0], dc[1], dc[2], dc[3]);
      }
    rsp = pair_sum(rsp);
    // P^ / dS^ visible, and this block's dO^ / Q^ transposed landed (every wave's DMAs): vector
    // memory operations complete in issue order, so waiting until only the next block's row
    // loads (the last ones issued) are outstanding covers everything before them
    if constexpr (kSbRowLoads<D> == 16)
      asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (kSbRowLoads<D> == 10)
      asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      static_assert(kSbRowLoads<D> == 16 || kSbRowLoads<D> == 10, "row load count");
    const float vsc = __fdiv_rn(pmax, 127.0f) * sdoi;
    const float ksc = __fdiv_rn(dmax, 127.0f) * sqi * a.sm;
    if (STORE) {  // the wave's record of the pair for the dQ kernel: stored after the barrier, so
                  // that its wait on this block's memory operations does not wait on the stores;
                  // non-temporal: read once, by another kernel, it need not displace this kernel's
                  // tiles in L2
      int8_t* rec = a.dsh + (pr * 4 + w) * kSbRec;
      __builtin_nontemporal_store(db[0], reinterpret_cast<v4i*>(rec + 16 * lane));
      __builtin_nontemporal_store(db[1], reinterpret_cast<v4i*>(rec + 1024 + 16 * lane));
      float* tail = reinterpret_cast<float*>(rec + 2048);
      if (lane < 32) __builtin_nontemporal_store(rsp, tail + lane);
      else if (lane == 32) __builtin_nontemporal_store(__fdiv_rn(dmax, 127.0f) * skj * a.sm, tail + 32);
    }
#pragma unroll
    for (int g = 0; g < NG; g++) {
      const int c = c0 + g;
      {
        v16i R;
#pragma unroll
        for (int r = 0; r < 16; r++) R[r] = 0;
#pragma unroll
        for (int qs = 0; qs < kBQ / 32; qs++) {
          const v4i pa = *reinterpret_cast<const v4i*>(&sP[(32 * Tw + col) * PS + 32 * qs + 16 * h]);
          const v4i ob = *reinterpret_cast<const v4i*>(&sOt[TQ::off(32 * c + col, 2 * qs + h)]);
          R = __builtin_amdgcn_mfma_i32_32x32x32_i8(pa, ob, R, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) accV[g][r] = fmaf((float)R[r], vsc, accV[g][r]);
      }
      {
        v16i R;
#pragma unroll
        for (int r = 0; r < 16; r++) R[r] = 0;
#pragma unroll
        for (int qs = 0; qs < kBQ / 32; qs++) {
          const v4i da = *reinterpret_cast<const v4i*>(&sD[(32 * Tw + col) * PS + 32 * qs + 16 * h]);
          const v4i qb = *reinterpret_cast<const v4i*>(&sQt[TQ::off(32 * c + col, 2 * qs + h)]);
          R = __builtin_amdgcn_mfma_i32_32x32x32_i8(da, qb, R, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) accK[g][r] = fmaf((float)R[r], ksc, accK[g][r]);
      }
    }
  }
  // C[i = key][j = channel]: lane = channel 32 c + col, rows = keys 32 Tw + 8 (r / 4) + 4 h + r % 4
#pragma unroll
  for (int g = 0; g < NG; g++) {
    const int c = c0 + g;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int key = key0 + 32 * Tw + 8 * (r >> 2) + 4 * h + (r & 3);
      if (key >= a.M) continue;
      const size_t o = ((size_t)bh * a.M + key) * D + 32 * c + col;
      a.dv[o] = accV[g][r];
      a.dk[o] = accK[g][r];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- host side

// Workspace slices of SageBwd (256-byte aligned).  The pair buffer comes last: the other slices
// sit at the same offsets with or without it, which lets a backward with SAGE_TRAIN_RECOMPUTE_DS
// take the quantized inputs a forward without it kept (SAGE_TRAIN_KEEP_QUANT).
enum SbSlice { kSbQh, kSbQt, kSbSq, kSbKh, kSbKt, kSbSk, kSbVt, kSbSv, kSbDot, kSbSdo, kSbD, kSbL2,
               kSbKpart, kSbVpart, kSbVmax, kSbVmin, kSbKmean, kSbVmean, kSbDv, kSbDsh, kSbSlices };
static_assert(kSbDsh == kSbSlices - 1, "the pair buffer is the last slice");

bool sb_store_ds(const Problem& p) {
  const size_t pairs = (size_t)p.BH * p.nqb * p.nkt;
  return !(p.variant & SAGE_TRAIN_RECOMPUTE_DS) && pairs * 4 * kSbRec <= kSbPairLimit;
}

size_t sb_layout(const Problem& p, bool bwd, size_t* s) {
  const size_t BH = (size_t)p.BH, d = (size_t)p.d;
  size_t z[kSbSlices];
  z[kSbQh] = BH * p.Np * d;
  z[kSbQt] = bwd ? BH * p.Np * d : 0;
  z[kSbSq] = BH * p.nqb * 4;
  z[kSbKh] = BH * p.Mp * d;
  z[kSbKt] = bwd ? BH * p.Mp * d : 0;
  z[kSbSk] = BH * p.nkt * 4;
  z[kSbVt] = BH * p.Mp * d;
  z[kSbSv] = BH * p.nkt * 4;
  z[kSbDot] = bwd ? BH * p.Np * d : 0;
  z[kSbSdo] = bwd ? BH * p.nqb * 4 : 0;
  z[kSbD] = bwd ? BH * p.Np * 4 : 0;
  z[kSbL2] = bwd ? BH * p.Np * 4 : 0;
  z[kSbKpart] = BH * p.nkt * d * 8;
  z[kSbVpart] = BH * p.nkt * d * 8;
  z[kSbVmax] = BH * p.nkt * d * 8;  // (max, min) pairs
  z[kSbVmin] = 0;
  z[kSbKmean] = BH * d * 4;
  z[kSbVmean] = BH * d * 4;
  z[kSbDv] = BH * d * 4;
  const bool pb = bwd && sb_store_ds(p);  // the pair buffer: dS^ of every (query, key) block pair
  const size_t pairs = BH * p.nqb * p.nkt;
  z[kSbDsh] = pb ? pairs * 4 * kSbRec : 0;
  size_t tot = 0;
  for (int i = 0; i < kSbSlices; i++) {
    if (s) s[i] = tot;
    tot += (z[i] + 255) & ~(size_t)255;
  }
  return tot;
}

// K mean (the inference path's kernels, pinned order) and the per-block codes of Q, K, V.
hipError_t sb_prep_fwd(const Problem& p, const void* q, const void* k, const void* v, char* ws, bool bwd,
                       bool smooth_k, hipStream_t st) {
  size_t o[kSbSlices];
  sb_layout(p, bwd, o);
  Workspace w{};
  w.kpart = (double*)(ws + o[kSbKpart]);
  w.vpart = (double*)(ws + o[kSbVpart]);
  w.vmm = (float2*)(ws + o[kSbVmax]);
  w.kmean = (float*)(ws + o[kSbKmean]);
  w.vmean = (float*)(ws + o[kSbVmean]);
  w.dv = (float*)(ws + o[kSbDv]);
  hipError_t e;
  if (smooth_k) {
    // K's mean only: V is quantized per block, with no statistics over all tokens
    if ((e = launch_stats(p, nullptr, k, nullptr, w, st)) != hipSuccess) return e;
    if ((e = launch_kv_finalize_k_only(p, w, st)) != hipSuccess) return e;
  }
  const float* km = smooth_k ? w.kmean : nullptr;
  const dim3 gq(p.nqb, p.BH), gk(p.nkt, p.BH);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  int8_t* qh = (int8_t*)(ws + o[kSbQh]);
  int8_t* qt = bwd ? (int8_t*)(ws + o[kSbQt]) : nullptr;
  int8_t* kh = (int8_t*)(ws + o[kSbKh]);
  int8_t* kt = bwd ? (int8_t*)(ws + o[kSbKt]) : nullptr;
  int8_t* vt = (int8_t*)(ws + o[kSbVt]);
  float* sq = (float*)(ws + o[kSbSq]);
  float* sk = (float*)(ws + o[kSbSk]);
  float* sv = (float*)(ws + o[kSbSv]);
  if (p.d == 128) {
    hipLaunchKernelGGL((sb_quant_kernel<128, 128, false>), gq, dim3(256), 0, st, Q, nullptr, qh, qt, sq, p.N, p.Np,
                       p.nqb, p.fp16);
    hipLaunchKernelGGL((sb_quant_kernel<128, 64, true>), gk, dim3(256), 0, st, K, km, kh, kt, sk, p.M, p.Mp, p.nkt,
                       p.fp16);
    hipLaunchKernelGGL((sb_quant_kernel<128, 64, true>), gk, dim3(256), 0, st, V, nullptr, nullptr, vt, sv, p.M,
                       p.Mp, p.nkt, p.fp16);
  } else {
    hipLaunchKernelGGL((sb_quant_kernel<64, 128, false>), gq, dim3(256), 0, st, Q, nullptr, qh, qt, sq, p.N, p.Np,
                       p.nqb, p.fp16);
    hipLaunchKernelGGL((sb_quant_kernel<64, 64, true>), gk, dim3(256), 0, st, K, km, kh, kt, sk, p.M, p.Mp, p.nkt,
                       p.fp16);
    hipLaunchKernelGGL((sb_quant_kernel<64, 64, true>), gk, dim3(256), 0, st, V, nullptr, nullptr, vt, sv, p.M,
                       p.Mp, p.nkt, p.fp16);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
void sb_fwd_launch(const Problem& p, const FwdArgs& a, hipStream_t st) {
  const dim3 grid(p.nqb * p.BH);
  if (p.out_fp32) hipLaunchKernelGGL((sb_fwd_kernel<D, CAUSAL, 2>), grid, dim3(256), 0, st, a);
  else if (p.fp16) hipLaunchKernelGGL((sb_fwd_kernel<D, CAUSAL, 1>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((sb_fwd_kernel<D, CAUSAL, 0>), grid, dim3(256), 0, st, a);
}

hipError_t sb_forward(const Problem& p, char* ws, bool bwd, void* out, float* lse, hipStream_t st) {
  size_t o[kSbSlices];
  sb_layout(p, bwd, o);
  FwdArgs a;
  a.qh = (const int8_t*)(ws + o[kSbQh]);
  a.sq = (const float*)(ws + o[kSbSq]);
  a.kh = (const int8_t*)(ws + o[kSbKh]);
  a.sk = (const float*)(ws + o[kSbSk]);
  a.vt = (const int8_t*)(ws + o[kSbVt]);
  a.sv = (const float*)(ws + o[kSbSv]);
  a.out = out;
  a.lse = lse;
  a.N = p.N; a.M = p.M; a.nqb = p.nqb; a.nkt = p.nkt; a.Np = p.Np; a.Mp = p.Mp;
  a.coff = p.causal == 2 ? p.M - p.N : 0;
  a.qk_scale = p.sm_scale * kLog2e;
  if (p.d == 128) p.causal ? sb_fwd_launch<128, true>(p, a, st) : sb_fwd_launch<128, false>(p, a, st);
  else p.causal ? sb_fwd_launch<64, true>(p, a, st) : sb_fwd_launch<64, false>(p, a, st);
  return hipGetLastError();
}

// The backward's own preprocessing: dO^ transposed per 128 rows, D, L2.
hipError_t sb_prep_bwd(const Problem& p, const void* out, const void* dout, const float* lse, char* ws,
                       hipStream_t st) {
  size_t o[kSbSlices];
  sb_layout(p, true, o);
  int8_t* dot = (int8_t*)(ws + o[kSbDot]);
  float* sdo = (float*)(ws + o[kSbSdo]);
  float* Dr = (float*)(ws + o[kSbD]);
  float* L2 = (float*)(ws + o[kSbL2]);
  const dim3 gq(p.nqb, p.BH);
  auto dO = (const uint16_t*)dout;
  const int outk = p.out_fp32 ? 2 : (p.fp16 ? 1 : 0);
  if (p.d == 128) {
    hipLaunchKernelGGL((sb_quant_kernel<128, 128, false>), gq, dim3(256), 0, st, dO, nullptr, nullptr, dot, sdo, p.N,
                       p.Np, p.nqb, p.fp16);
    if (outk == 2) hipLaunchKernelGGL((sb_dprep_kernel<128, 2>), gq, dim3(256), 0, st, out, dO, lse, Dr, L2, p.N, p.Np, p.fp16);
    else if (outk == 1) hipLaunchKernelGGL((sb_dprep_kernel<128, 1>), gq, dim3(256), 0, st, out, dO, lse, Dr, L2, p.N, p.Np, p.fp16);
    else hipLaunchKernelGGL((sb_dprep_kernel<128, 0>), gq, dim3(256), 0, st, out, dO, lse, Dr, L2, p.N, p.Np, p.fp16);
  } else {
    hipLaunchKernelGGL((sb_quant_kernel<64, 128, false>), gq, dim3(256), 0, st, dO, nullptr, nullptr, dot, sdo, p.N,
                       p.Np, p.nqb, p.fp16);
    if (outk == 2) hipLaunchKernelGGL((sb_dprep_kernel<64, 2>), gq, dim3(256), 0, st, out, dO, lse, Dr, L2, p.N, p.Np, p.fp16);
    else if (outk == 1) hipLaunchKernelGGL((sb_dprep_kernel<64, 1>), gq, dim3(256), 0, st, out, dO, lse, Dr, L2, p.N, p.Np, p.fp16);
    else hipLaunchKernelGGL((sb_dprep_kernel<64, 0>), gq, dim3(256), 0, st, out, dO, lse, Dr, L2, p.N, p.Np, p.fp16);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool FP16>
void sb_bwd_launch(const Problem& p, const BwdArgs& a, hipStream_t st) {
  if (sb_store_ds(p)) {
    // dK/dV first: it leaves every pair's dS^ for the dQ contraction
    hipLaunchKernelGGL((sb_dkv_kernel<D, CAUSAL, FP16, true>), dim3(p.nkt * p.BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL((sb_dq_kernel<D, CAUSAL>), dim3(p.nqb * p.BH), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((sb_dq_recompute_kernel<D, CAUSAL, FP16>), dim3(p.nqb * p.BH), dim3(256), 0, st, a);
    hipLaunchKernelGGL((sb_dkv_kernel<D, CAUSAL, FP16, false>), dim3(p.nkt * p.BH), dim3(256), 0, st, a);
  }
}

template <int D>
void sb_bwd_d(const Problem& p, const BwdArgs& a, hipStream_t st) {
  if (p.causal) p.fp16 ? sb_bwd_launch<D, true, true>(p, a, st) : sb_bwd_launch<D, true, false>(p, a, st);
  else p.fp16 ? sb_bwd_launch<D, false, true>(p, a, st) : sb_bwd_launch<D, false, false>(p, a, st);
}

hipError_t sb_backward(const Problem& p, char* ws, bool smooth_k, const void* v, const void* dout, float* dq,
                       float* dk, float* dv, hipStream_t st) {
  size_t o[kSbSlices];
  sb_layout(p, true, o);
  BwdArgs a;
  a.qh = (const int8_t*)(ws + o[kSbQh]);
  a.qt = (const int8_t*)(ws + o[kSbQt]);
  a.sq = (const float*)(ws + o[kSbSq]);
  a.kh = (const int8_t*)(ws + o[kSbKh]);
  a.kt = (const int8_t*)(ws + o[kSbKt]);
  a.sk = (const float*)(ws + o[kSbSk]);
  a.dot = (const int8_t*)(ws + o[kSbDot]);
  a.sdo = (const float*)(ws + o[kSbSdo]);
  a.Dr = (const float*)(ws + o[kSbD]);
  a.L2 = (const float*)(ws + o[kSbL2]);
  a.kmean = smooth_k ? (const float*)(ws + o[kSbKmean]) : nullptr;
  a.V = (const uint16_t*)v;
  a.dO = (const uint16_t*)dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsh = (int8_t*)(ws + o[kSbDsh]);
  a.N = p.N; a.M = p.M; a.nqb = p.nqb; a.nkt = p.nkt; a.Np = p.Np; a.Mp = p.Mp;
  a.coff = p.causal == 2 ? p.M - p.N : 0;
  a.qk_scale = p.sm_scale * kLog2e;
  a.sm = p.sm_scale;
  if (p.d == 128) sb_bwd_d<128>(p, a, st);
  else sb_bwd_d<64>(p, a, st);
  return hipGetLastError();
}

}  // namespace sage
