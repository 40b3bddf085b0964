// attn_fwd_mx.hip -- fused quantized attention forward, MXFP4 variant (gfx950).
//
// "SageAttention3" summary, 3.4 "The NVFP4 Microscaling Format and Quantization Operator":
// each operand of the two products is E2M1 with one power-of-two (E8M0) scale per 32
// elements along the product's reduction dimension, and a product is the sum over blocks of
// X_a X_b (a^ . b^)_blk.  With the smoothing of "SageAttention2 Technical Report" 3.4, per
// 128-query block i and 64-key tile j:
//   S   = sum_blk X_Q X_K (Q^ K^T)_blk + Delta S_ij
//   m   = max(m, rowmax S);  P~ = exp(S - m);  l = e^{m_old - m} l + rowsum P~   (FP32)
//   P^  = E2M1(P~ / X_P), X_P per 32 keys of the row (the smallest 2^e with max <= 6 * 2^e)
//   O   = e^{m_old - m} O + sum_blk X_P X_V (P^ V^)_blk
//   out = O / l (+ V_m)
//
// Mapping.  As in the INT8/FP8 kernel, S^T = K^ Q^T on the 32x32 MFMA gives each lane one
// query and 16 keys of each 32-key half (keys 8b + 4h + k, h = lane / 32); here the MFMA is
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 (64 channels per instruction,
// each lane half a 32-channel block whose E8M0 scale the lane supplies: byte-selected from
// one scale word per tile for K, per kernel for Q).  The block scales are applied inside
// the MFMA, and so is Delta S: the QK accumulator starts from the tile's (unscaled) Delta S,
// which the matrix core adds at FP32.  The FP32 score then needs no dequant, and the factor
// sm_scale log2 e and the running max meet in the exponent's one FMA: exp2(s c - base).
// The P~ block of a row is 32 contiguous keys: its maximum is exp2 of the block's largest
// score (the same exp2 the element gets), which sets the E8M0 scale; the hardware
// conversion takes that scale directly (v_cvt_scalef32_pk_fp4_f32 divides by the power of
// two of the scale's exponent field and rounds to nearest even).  The FP4 PV MFMA consumes
// 32 keys per lane half, so the two lane halves swap their packed fragments once
// (v_permlane32_swap): afterwards half h holds the keys 32h..32h+31, the P block h and its
// scale, and V^ was stored with its keys in that order (vperm_mx).  O^T = V^T P^T then
// accumulates through the MFMA's FP32 C operand (lazy rescale when a row's maximum rises),
// or, as a variant, from a zero accumulator with one VALU FMA into O.
//
// Two-level P (knob; "SageAttention3" summary, 3.4 "Two-Level Quantization for the Attention
// Map P"): level one divides each row of the tile's P~ by s1 = rowmax(P~) / 6, so the row's
// largest value is exactly 6; level two is the block quantizer above; the tile's product is
// multiplied back by s1.  The row maximum of P~ comes from the softmax's maximum of S (the
// pages' reuse): P2 = P~ / s1 = exp2(S - (rowmax S - log2 6)), one exp2 per element as before,
// with the block scales from 6 exp2(block max S - rowmax S).  The factor s1 is not applied to
// the product: O is kept divided by the current s1 (O_true = s1 O), so a tile multiplies O by
// s1_old alpha / s1_new = exp2(b_old - b_new) (b = rowmax S - log2 6, the level-one base)
// before its product accumulates through the C operand, and the epilogue multiplies by
// s1 = exp2(b - m).
#include <hip/hip_ext.h>

#include "attn_device.hpp"

namespace sage {
namespace {

using namespace attn;

// LDS tiles, unpadded, 16-byte chunks XOR-swizzled within a row so that the 16 lanes a
// ds_read_b128 serves at once (16 consecutive rows, one chunk column) hit 16 distinct
// 16-byte bank groups.
template <int D>
struct MxTiles {
  static constexpr int KROW = D / 2;          // bytes per K^ row (two E2M1 codes per byte)
  static constexpr int KCH = KROW / 16;       // 16-byte chunks per K^ row
  static constexpr int KRPL = 256 / KROW;     // K^ rows per 256-byte bank line
  static constexpr int KBYTES = kBK * KROW;
  static constexpr int VROW = kBK / 2;        // V^ rows are channels: 64 keys, 32 bytes
  static constexpr int VBYTES = D * VROW;
  static constexpr int KDMA = KBYTES / 1024;  // 1 KiB LDS-DMA wave instructions per tile
  static constexpr int VDMA = VBYTES / 1024;
  __device__ static int kswz(int r) { return (r / KRPL) & (KCH - 1); }
  __device__ static int vswz(int r) { return (r >> 3) & 1; }
  __device__ static int koff(int r, int c) { return r * KROW + 16 * (c ^ kswz(r)); }
  __device__ static int voff(int r, int c) { return r * VROW + 16 * (c ^ vswz(r)); }
};

struct MxArgs {
  const uint8_t* qhat;  // [BH][Np][D/2]
  const uint8_t* khat;  // [BH][Mp][D/2]
  const uint8_t* vhat;  // [BH][nkt][D][32]
  const uint8_t* qsc;   // [BH][Np][D/32]
  const uint8_t* ksc;   // [BH][nkt][64][4]
  const uint8_t* vsc;   // [BH][nkt][64][4]
  const float* vmean;
  const float* ds;      // Delta S (unscaled)
  void* out;
  int BH, nqb, nkt, Np, Mp;  // bounds: padded workspace strides
  int causal2;      // causal = 2: key t visible to query r iff t <= r + M - N (else t <= r)
  SeqLayout ql, kl; // rows of q / out and of k, v per sequence (dense or packed)
  int H, Hkv, G;    // query heads, key/value heads, query heads per key/value head
  float qk_scale;       // sm_scale * log2(e)
  int xcd_map;
};

// One block-scaled FP4 MFMA: 32x32 output, 64-deep reduction; a and b carry 32 E2M1 codes
// per lane (the operand's upper half is not read for FP4), sa / sb the lanes' scale words
// with the E8M0 byte selected by OA / OB.
template <int OA, int OB>
__device__ __forceinline__ v16f mfma_fp4(const v4i& a, const v4i& b, const v16f& c, uint32_t sa, uint32_t sb) {
  const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
  const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OA, (int)sa, OB, (int)sb);
}

// S^T = Delta S + sum_blk X_K X_Q (K^ Q^T)_blk of one 64-key tile (before sm_scale): two 32-key
// halves, D/64 MFMAs each; the accumulator starts from the tile's Delta S (unscaled), which the
// matrix core adds at FP32.  The K scale word of lane l holds byte 2T + c for key 32T + l%32,
// channel block 2c + l/32; the Q scale word byte c for channel block 2c + l/32.
template <int D>
__device__ __forceinline__ void qk_tile_mx(const uint8_t* __restrict__ sK, const float* __restrict__ sDS,
                                           const v4i (&qf)[D / 64], uint32_t ks, uint32_t qs, int h, int col,
                                           v16f (&acc)[2]) {
  static_for<0, 2>([&](auto Tc) {
    constexpr int T = decltype(Tc)::value;
#pragma unroll
    for (int r = 0; r < 16; r++) acc[T][r] = sDS[32 * T + 8 * (r >> 2) + 4 * h + (r & 3)];
    static_for<0, D / 64>([&](auto Cc) {
      constexpr int C = decltype(Cc)::value;
      const v4i kf = *reinterpret_cast<const v4i*>(&sK[MxTiles<D>::koff(32 * T + col, 2 * C + h)]);
      acc[T] = mfma_fp4<2 * T + C, C>(kf, qf[C], acc[T], ks, qs);
    });
  });
}

constexpr float kLog2_6 = 2.5849625007211562f;  // log2(6)
constexpr float kP2Span = 64.0f;  // two-level P: level-one reference at most this far (log2) below the max

// max of two values that are not signalling NaNs (scores and their maxima), without the quieting
// step fmaxf asks the compiler for when an input comes out of a lane exchange
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// E8M0 code (biased exponent) of an MX block whose largest magnitude is 6 * 2^y, from yb = y + 127:
// the smallest e with 6 * 2^y <= 6 * 2^e is ceil(y), clamped to [-127, 127] and biased by 127, so
// the code is ceil(yb) clamped to [0, 254]; y = -inf (a fully masked block) gives code 0.
// Computed on the score arithmetic itself, so the block maximum needs no exp2 of its own; yb
// carries the FP32 rounding of the score arithmetic and of the bias, a relative 2^-16 at most in
// 6 * 2^y, the margin within which either exponent is a correct rounding of the method's value.
__device__ __forceinline__ uint32_t e8m0_code_log2(float yb) {
  return (uint32_t)__builtin_amdgcn_fmed3f(ceilf(yb), 0.0f, 254.0f);
}
constexpr float kBias6 = 127.0f - kLog2_6;  // the bias of e8m0_code_log2 less log2(6)

template <int D, bool CAUSAL, bool ACC_VALU, bool P2L>
__device__ __forceinline__ void softmax_pv_mx(const v16f (&acc)[2], const uint8_t* __restrict__ sV,
                                              uint32_t vs, float qk_scale, int h,
                                              int col, int key0, int qrow, int M, bool masked, v16f (&O)[D / 32],
                                              float& m_run, float& l_run, float& b_run) {
  static_assert(!(P2L && ACC_VALU), "two-level P accumulates through the C operand");
  // ---- scores before sm_scale log2(e): the block scales and Delta S are in the MFMA's sums;
  // the factor joins the base in one FMA per score (exp2 argument = sc * qk_scale - base) ----
  float sc[2][16];
#pragma unroll
  for (int T = 0; T < 2; T++)
#pragma unroll
    for (int r = 0; r < 16; r++) sc[T][r] = acc[T][r];
  if (masked) {
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
  // ---- running max; each 32-key half's maximum is also its P block's ----
  // One lane swap of the two halves' partial maxima leaves lane half h with block h's maximum
  // (its lane pair's), a second one hands it the other block's; no NaN canonicalization is
  // needed on these values (max3 / med3 below).
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    m0 = fmaxf(m0, sc[0][r]);
    m1 = fmaxf(m1, sc[1][r]);
  }
  const auto x1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
  const float mraw = max2(__uint_as_float(x1[0]), __uint_as_float(x1[1]));  // block h
  const auto x2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw), __float_as_uint(mraw), false, false);
  // the two blocks' maxima in log2 units (rounded products, so that the tile maximum equals
  // its block's maximum exactly)
  const float mown = mraw * qk_scale;                                                  // block h
  const float moth = (h ? __uint_as_float(x2[0]) : __uint_as_float(x2[1])) * qk_scale;  // block 1 - h
  const float m_tile = max2(mown, moth);
  const float m_new = fmaxf(m_run, m_tile);  // finite: m_run starts at -FLT_MAX
  const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile, exactly 1 if m is unchanged
  m_run = m_new;
  float base, resc = alpha;  // exponent base of the quantized values; factor on O before the MFMA
  // E8M0 codes of the P blocks from the log2 of their largest values, this lane's own block and
  // the other one (code 0 for a fully masked block)
  uint32_t pc_own, pc_oth;
  if constexpr (P2L) {
    // Level one: the row's largest P~ of this tile maps to 6.  A row with no visible key in the
    // tile keeps its base (its P2 are 0 and O stays as it is).  The reference of level one is
    // kept within kP2Span octaves of the running maximum: a tile whose maximum lies further
    // below contributes less than 2^-kP2Span of the row's sum (invisible in FP32), and the
    // rescale exp2(b_old - b_new) of O stays below 2^kP2Span, so O never leaves the FP32 range.
    const bool vis = m_tile > -INFINITY;
    const float bref = max2(m_tile, m_new - kP2Span);
    base = vis ? bref - kLog2_6 : b_run;
    resc = fast_exp2(b_run - base);
    b_run = base;
    // a block's largest P2 is 6 exp2(block max - bref): exactly 6 (code 127) for the block that
    // holds the tile's row maximum (bref = m_tile unless clamped)
    pc_own = vis ? e8m0_code_log2((mown - bref) + 127.0f) : 0u;
    pc_oth = vis ? e8m0_code_log2((moth - bref) + 127.0f) : 0u;
  } else {
    base = m_new;
    // a block's largest P~ is exp2(block max - base)
    pc_own = e8m0_code_log2((mown - base) + kBias6);
    pc_oth = e8m0_code_log2((moth - base) + kBias6);
  }
  const uint32_t pc0 = h ? pc_oth : pc_own, pc1 = h ? pc_own : pc_oth;
  // ---- P~ (FP32), row sum of the unquantized values, E2M1 pack ----
  float psum;
  uint32_t pk[2][2];
#pragma unroll
  for (int T = 0; T < 2; T++) {
    const float scl = __uint_as_float((T ? pc1 : pc0) << 23);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; e++) p[e] = fast_exp2(fmaf(sc[T][8 * q + e], qk_scale, -base));
      const float g = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      psum = (T == 0 && q == 0) ? g : psum + g;
      // each conversion writes one byte of its destination: seed it with a dead register (the
      // score the first value came from) so that no zeroing move is needed
      uint32_t wd = __float_as_uint(sc[T][8 * q]);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, p[0], p[1], scl, 0);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, p[2], p[3], scl, 1);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, p[4], p[5], scl, 2);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, p[6], p[7], scl, 3);
      pk[T][q] = wd;
    }
  }
  // l sums the unquantized P~ = s1 P2 in the two-level form, s1 = exp2(base - m_new)
  l_run = fmaf(l_run, alpha, P2L ? psum * fast_exp2(base - m_new) : psum);
  // ---- regroup: lane half h takes the whole 32-key half T = h (half 0's keys first) ----
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const auto r = __builtin_amdgcn_permlane32_swap(pk[0][q], pk[1][q], false, false);
    pk[0][q] = r[0];
    pk[1][q] = r[1];
  }
  const v4i pf = {(int)pk[0][0], (int)pk[0][1], (int)pk[1][0], (int)pk[1][1]};
  const uint32_t pcode = pc_own;
  // ---- O^T += sum_blk X_V X_P (V^T P^T)_blk per 32-channel sub-tile ----
  if (!ACC_VALU) {
    if (__any(resc != 1.0f)) {
#pragma unroll
      for (int c = 0; c < D / 32; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) O[c][r] *= resc;
    }
  }
  static_for<0, D / 32>([&](auto gc) {
    constexpr int g = decltype(gc)::value;
    const v4i vf = *reinterpret_cast<const v4i*>(&sV[MxTiles<D>::voff(32 * g + col, h)]);
    if (ACC_VALU) {
      v16f R;
#pragma unroll
      for (int r = 0; r < 16; r++) R[r] = 0.0f;
      R = mfma_fp4<g, 0>(vf, pf, R, vs, pcode);
#pragma unroll
      for (int r = 0; r < 16; r++) O[g][r] = fmaf(O[g][r], alpha, R[r]);
    } else {
      O[g] = mfma_fp4<g, 0>(vf, pf, O[g], vs, pcode);
    }
  });
}

// Registers are budgeted for OCC work-groups per CU (three waves per SIMD at d = 128, four at
// d = 64), which overlap one another's matrix and vector work; the K/V tiles use a 2-slot
// ring: tile j+1 streams in while tile j is computed.
template <int D, bool CAUSAL, int OUT, bool ACC_VALU, bool P2L>  // OUT: 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256, D == 64 ? 4 : 3) void attn_fwd_mx_kernel(MxArgs a) {
  using TL = MxTiles<D>;
  constexpr int NG = D / 32;  // 32-channel sub-tiles of O
  constexpr int NB = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t sK[NB][TL::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[NB][TL::VBYTES];
  __shared__ __attribute__((aligned(256))) float sDS[NB][kBK];
  __shared__ __attribute__((aligned(256))) uint32_t sKS[NB][64];
  __shared__ __attribute__((aligned(256))) uint32_t sVS[NB][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  int bh, qi;
  {
    const int L = blockIdx.x;
    if (a.xcd_map) {
      // XCD x (work-groups are dealt to the XCDs round-robin) takes whole groups of query heads
      // that share a key/value head: groups x, x+8, ...; a head's blocks stay together, so a
      // key/value head's tiles are read through one XCD's L2.
      const int x = L % kXCD, r = L / kXCD, k = r / a.nqb;
      bh = (x + kXCD * (k / a.G)) * a.G + k % a.G;
      qi = r % a.nqb;
    } else {
      bh = L / a.nqb;
      qi = L % a.nqb;
    }
  }
  const int kvh = kv_head(bh, a.H, a.Hkv, a.G);  // the key/value head this query head reads
  // this sequence's queries and keys (every sequence of a dense batch has N and M)
  const int bseq = bh / a.H;
  const int nseq = seq_rows(a.ql, bseq, 0, a.H, D).len, mseq = seq_rows(a.kl, bseq, 0, a.Hkv, D).len;
  const int coff = a.causal2 ? mseq - nseq : 0;  // key t visible to query r iff t <= r + coff
  const int nqbs = (nseq + kBQ - 1) / kBQ, nkts = (mseq + kBK - 1) / kBK;
  if (qi >= nqbs) return;  // a block past this sequence's queries (variable-length batches)
  const int qb = CAUSAL ? (nqbs - 1 - qi) : qi;  // heavy blocks first
  const int q0 = qb * kBQ;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + col;

  // ---- Q^ fragments (B operand): query qrow, channels 64c + 32h .. +32; scale bytes ----
  v4i qf[D / 64];
  uint32_t qs = 0;
  {
    const size_t row = (size_t)bh * a.Np + qrow;
    const uint8_t* qp = a.qhat + row * (D / 2) + 16 * h;
#pragma unroll
    for (int c = 0; c < D / 64; c++) qf[c] = *reinterpret_cast<const v4i*>(qp + 32 * c);
    const uint8_t* sp = a.qsc + row * (D / 32);
#pragma unroll
    for (int c = 0; c < D / 64; c++) qs |= (uint32_t)sp[2 * c + h] << (8 * c);
  }

  v16f O[NG];
#pragma unroll
  for (int c = 0; c < NG; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) O[c][r] = 0.0f;
  // -FLT_MAX, not -inf: a row that sees no key (variable-length batches) keeps l = 0 and O = 0
  // instead of NaN; a row's first visible tile still gets alpha = 0 exactly.
  float m_run = -FLT_MAX, l_run = 0.0f;
  float b_run = -FLT_MAX;  // two-level P: the level-one base of O (O_true = exp2(b_run - m_run) O)

  const int jend = CAUSAL ? max(0, min(nkts, (q0 + kBQ + coff + kBK - 1) / kBK)) : nkts;
  const uint8_t* kbase = a.khat + (size_t)kvh * a.Mp * (D / 2);
  const uint8_t* vbase = a.vhat + (size_t)kvh * a.nkt * TL::VBYTES;
  const float* dsbase = a.ds + ((size_t)bh * a.nqb + qb) * a.Mp;
  const uint8_t* ksbase = a.ksc + (size_t)kvh * a.nkt * 256;
  const uint8_t* vsbase = a.vsc + (size_t)kvh * a.nkt * 256;

  // ---- staging by LDS DMA.  D = 128: wave w moves K^ KiB w and V^ KiB w; D = 64: waves 0-1
  // move K^, waves 2-3 move V^.  Waves 0, 1, 2 also move Delta S, the K scales, the V scales.
  static_assert(TL::KDMA == TL::VDMA && (TL::KDMA == 4 || TL::KDMA == 2), "tile size");
  const bool movesK = TL::KDMA == 4 || w < 2, movesV = TL::VDMA == 4 || w >= 2;
  const int kchunk = movesK ? w : 0, vchunk = movesV ? (TL::VDMA == 4 ? w : w - 2) : 0;
  int koffs = 0, voffs = 0;
  {
    const int q = kchunk * 64 + lane;  // 16-byte LDS chunk this lane fills
    const int r = q / TL::KCH;
    koffs = r * TL::KROW + 16 * ((q % TL::KCH) ^ TL::kswz(r));
    const int qv = vchunk * 64 + lane;
    const int rv = qv / 2;
    voffs = rv * TL::VROW + 16 * ((qv & 1) ^ TL::vswz(rv));
  }
  auto dma = [&](int j, int slot) {
    if (movesK) dma16(lds_addr(&sK[slot][kchunk * 1024]), kbase + (size_t)j * TL::KBYTES, koffs);
    if (movesV) dma16(lds_addr(&sV[slot][vchunk * 1024]), vbase + (size_t)j * TL::VBYTES, voffs);
    if (w == 0) dma4(lds_addr(&sDS[slot][0]), dsbase + (size_t)j * kBK, 4 * lane);
    if (w == 1) dma4(lds_addr(&sKS[slot][0]), ksbase + (size_t)j * 256, 4 * lane);
    if (w == 2) dma4(lds_addr(&sVS[slot][0]), vsbase + (size_t)j * 256, 4 * lane);
  };
  // The slot of tile j+1 was last read in iteration j-1, which every wave left at the barrier
  // that closed it; at the end of iteration j, tile j+1 must have landed for all waves.
  auto publish = [&]() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  auto skip_t = [&](int j) { return CAUSAL && j * kBK > wq0 + 31 + coff; };  // fully masked for this wave
  if (jend > 0) dma(0, 0);
  publish();
  // One iteration; the slot is a compile-time constant so LDS addresses are immediates.
  auto iter = [&](int j, auto slotc) {
    constexpr int b = decltype(slotc)::value;
    if (j + 1 < jend) dma(j + 1, 1 - b);
    if (!skip_t(j)) {
      const int key0 = j * kBK;
      const bool masked = (CAUSAL && key0 + kBK - 1 > wq0 + coff) || (key0 + kBK > mseq);
      v16f acc[2];
      qk_tile_mx<D>(sK[b], sDS[b], qf, sKS[b][lane], qs, h, col, acc);
      softmax_pv_mx<D, CAUSAL, ACC_VALU, P2L>(acc, sV[b], sVS[b][lane], a.qk_scale, h, col, key0,
                                              qrow + coff, mseq, masked, O, m_run, l_run, b_run);
    }
    publish();
  };
  for (int j0 = 0; j0 < jend; j0 += NB) {
    static_for<0, NB>([&](auto slotc) {
      const int j = j0 + decltype(slotc)::value;
      if (j < jend) iter(j, slotc);
    });
  }

  // ---- epilogue: O / l (+ V_m); 0 for a row that saw no key ----
  const float l_tot = pair_sum(l_run);
  if (qrow >= nseq) return;
  const float inv = (P2L ? fast_exp2(b_run - m_run) : 1.0f) / l_tot;
  const bool none = l_tot == 0.0f;
  const float* vmp = a.vmean + (size_t)kvh * D;
  const SeqRows ro = seq_rows(a.ql, bseq, bh % a.H, a.H, D);
  const size_t orow = ro.base + (size_t)qrow * ro.stride;
  // per 32-channel group: its V_m loads all issued before its stores (the stores may alias them
  // as far as the compiler knows, which would otherwise serialize every load)
#pragma unroll
  for (int c = 0; c < NG; c++) {
    float4 vm4[4];
#pragma unroll
    for (int b = 0; b < 4; b++) vm4[b] = *reinterpret_cast<const float4*>(vmp + 32 * c + 8 * b + 4 * h);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ch = 32 * c + 8 * b + 4 * h;
      const float vmv[4] = {vm4[b].x, vm4[b].y, vm4[b].z, vm4[b].w};
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; k++) o[k] = none ? 0.0f : fmaf(O[c][4 * b + k], inv, vmv[k]);
      store_out4<OUT>(a.out, orow + ch, o);
    }
  }
}

struct LaunchEv {
  hipEvent_t e0, e1;
};

template <int D, bool CAUSAL, bool ACC_VALU, bool P2L>
hipError_t launch_d(const Problem& p, const MxArgs& a, hipStream_t s, LaunchEv ev) {
  dim3 grid(p.nqb * p.BH);
  const int out = p.out_fp32 ? 2 : (p.fp16 ? 1 : 0);
  if (out == 2)
    hipExtLaunchKernelGGL((attn_fwd_mx_kernel<D, CAUSAL, 2, ACC_VALU, P2L>), grid, dim3(256), 0, s, ev.e0, ev.e1, 0, a);
  else if (out == 1)
    hipExtLaunchKernelGGL((attn_fwd_mx_kernel<D, CAUSAL, 1, ACC_VALU, P2L>), grid, dim3(256), 0, s, ev.e0, ev.e1, 0, a);
  else
    hipExtLaunchKernelGGL((attn_fwd_mx_kernel<D, CAUSAL, 0, ACC_VALU, P2L>), grid, dim3(256), 0, s, ev.e0, ev.e1, 0, a);
  return hipGetLastError();
}

template <int D, bool ACC_VALU, bool P2L = false>
hipError_t launch_c(const Problem& p, const MxArgs& a, hipStream_t s, LaunchEv ev) {
  return p.causal ? launch_d<D, true, ACC_VALU, P2L>(p, a, s, ev) : launch_d<D, false, ACC_VALU, P2L>(p, a, s, ev);
}

}  // namespace

hipError_t launch_attn_fwd_mx(const Problem& p, const Workspace& w, void* out, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  MxArgs a;
  a.qhat = reinterpret_cast<const uint8_t*>(w.qhat);
  a.khat = reinterpret_cast<const uint8_t*>(w.khat);
  a.vhat = w.vhat;
  a.qsc = w.qsc; a.ksc = w.ksc; a.vsc = w.vsc;
  a.vmean = w.vmean; a.ds = w.ds; a.out = out;
  a.BH = p.BH; a.nqb = p.nqb; a.nkt = p.nkt; a.Np = p.Np; a.Mp = p.Mp;
  a.causal2 = p.causal == 2 ? 1 : 0;
  a.ql = p.ql; a.kl = p.kl;
  a.qk_scale = p.sm_scale * kLog2e;
  a.H = p.H; a.Hkv = p.Hkv; a.G = p.G;
  a.xcd_map = (p.BH % (kXCD * p.G) == 0) ? 1 : 0;
  const bool valu = (p.variant & SAGE_ACC_VALU) != 0;
  const LaunchEv ev{e0, e1};
  if (p.variant & SAGE_MX_P_TWO_LEVEL)  // the host check keeps SAGE_ACC_VALU out of this form
    return p.d == 128 ? launch_c<128, false, true>(p, a, s, ev) : launch_c<64, false, true>(p, a, s, ev);
  if (p.d == 128) return valu ? launch_c<128, true>(p, a, s, ev) : launch_c<128, false>(p, a, s, ev);
  return valu ? launch_c<64, true>(p, a, s, ev) : launch_c<64, false>(p, a, s, ev);
}

}  // namespace sage
