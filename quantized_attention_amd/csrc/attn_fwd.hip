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
#include <hip/hip_ext.h>

#include "attn_device.hpp"

namespace sage {
namespace {

using namespace attn;

constexpr float kLog2_448 = 8.807354922057604f;  // log2(448)

// LDS tiles are unpadded; 16-byte chunks are XOR-swizzled within a row so that the 16
// lanes a ds_read_b128 serves at once (16 consecutive rows, one chunk column) hit 16
// distinct 16-byte bank groups.  Rows sharing a 256-byte bank line differ in the low row
// bits, rows that alias differ in the swizzle.
template <int D>
struct Tiles {
  static constexpr int KROW = D;                   // bytes per K^ row
  static constexpr int KCH = D / 16;               // 16-byte chunks per K^ row
  static constexpr int KRPL = 256 / D;             // K^ rows per 256-byte bank line
  static constexpr int KBYTES = kBK * D;
  static constexpr int VBYTES = D * kBK;           // V^ rows are channels, 64 bytes each
  static constexpr int KDMA = KBYTES / 1024 / 4;   // 1 KiB LDS-DMA wave instructions per wave
  static constexpr int VDMA = VBYTES / 1024 / 4;
  __device__ static int kswz(int r) { return (r / KRPL) & (KCH - 1); }
  __device__ static int vswz(int r) { return (r >> 2) & 3; }
  __device__ static int koff(int r, int c) { return r * D + 16 * (c ^ kswz(r)); }
  __device__ static int voff(int r, int c) { return r * kBK + 16 * (c ^ vswz(r)); }
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
  int BH, nqb, nkt, Np, Mp;  // bounds: padded workspace strides
  int causal2;      // causal = 2: key t visible to query r iff t <= r + M - N (else t <= r)
  SeqLayout ql, kl; // rows of q / out and of k, v per sequence (dense or packed)
  int H, Hkv, G;    // query heads, key/value heads, query heads per key/value head
  float qk_scale;   // sm_scale * log2(e)
  int xcd_map;      // 1: heads grouped per XCD
};

// Score accumulator of one 32-key half: exact INT32 (INT8 Q^, K^) or FP32 (E4M3 Q^, K^).
template <bool QF8>
using acc_t = std::conditional_t<QF8, v16f, v16i>;

// S^T = K^ Q^T of one 64-key tile: two 32-key halves.  INT8: four 32-channel MFMAs
// (v_mfma_i32_32x32x32_i8).  E4M3 (QF8): two 64-channel MFMAs (v_mfma_f32_32x32x64_f8f6f4)
// over the same register bytes -- the A and B operands share one lane/byte -> k mapping, so
// pairing the K^ and Q^ chunks of two INT8 steps sums the same 64 channels.
template <int D, bool QF8>
__device__ __forceinline__ void qk_tile(const int8_t* __restrict__ sK, const v4i (&qf)[D / 32], int h, int col,
                                        acc_t<QF8> (&acc)[2]) {
  constexpr int NKS = D / 32;
#pragma unroll
  for (int T = 0; T < 2; T++) {
#pragma unroll
    for (int r = 0; r < 16; r++) acc[T][r] = 0;
    if constexpr (QF8) {
#pragma unroll
      for (int s = 0; s < NKS; s += 2) {
        const v4i k0 = *reinterpret_cast<const v4i*>(&sK[Tiles<D>::koff(32 * T + col, 2 * s + h)]);
        const v4i k1 = *reinterpret_cast<const v4i*>(&sK[Tiles<D>::koff(32 * T + col, 2 * s + 2 + h)]);
        const v8i kf = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        const v8i qq = {qf[s][0], qf[s][1], qf[s][2], qf[s][3], qf[s + 1][0], qf[s + 1][1], qf[s + 1][2], qf[s + 1][3]};
        acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qq, acc[T], 0, 0, 0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NKS; s++) {
        const v4i kf = *reinterpret_cast<const v4i*>(&sK[Tiles<D>::koff(32 * T + col, 2 * s + h)]);
        acc[T] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[s], acc[T], 0, 0, 0);
      }
    }
  }
}

// The rest of one tile for one wave, from its INT32 (or FP32) scores: dequantize, online
// softmax, P^ V^ into O.  `masked` (wave-uniform) selects the causal / ragged-tail mask;
// interior tiles skip it.
// vlo / vhi: this lane's byte offsets of its two 16-byte V^ chunks in a slot's first 32-channel
// sub-tile (the sub-tiles follow at 32 * kBK bytes).
template <int D, bool CAUSAL, bool ACC_VALU, typename ACC>
__device__ __forceinline__ void softmax_pv(const ACC (&acc)[2], const uint8_t* __restrict__ sV,
                                           const float* __restrict__ sDS, const float* __restrict__ sDK,
                                           float dql, int h, int col, int vlo, int vhi, int key0, int qrow, int M,
                                           bool masked, v16f (&O)[D / 32], float& m_run, float& l_run) {
  constexpr int NKS = D / 32;
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
  const float m_new = fmaxf(m_run, mt);  // finite: m_run starts at -FLT_MAX
  const float base = m_new - kLog2_448;
  const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile, exactly 1 if m is unchanged
  m_run = m_new;
  // ---- P = 448 P~ (FP32), row sum, E4M3 pack in the PV B-operand order ----
  // l = alpha l + rowsum P, as one chain that starts from alpha l
  float lsum;
  v8i pf;
#pragma unroll
  for (int T = 0; T < 2; T++) {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const float p0 = fast_exp2(sc[T][4 * q4 + 0] - base);
      const float p1 = fast_exp2(sc[T][4 * q4 + 1] - base);
      const float p2 = fast_exp2(sc[T][4 * q4 + 2] - base);
      const float p3 = fast_exp2(sc[T][4 * q4 + 3] - base);
      const float g = (p0 + p1) + (p2 + p3);
      lsum = (T == 0 && q4 == 0) ? fmaf(l_run, alpha, g) : lsum + g;
      // the instruction keeps the other half-word of its destination: seed it with a dead
      // register (the score p0 came from) so that no copy is needed
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(sc[T][4 * q4 + 0]), false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
      pf[4 * T + q4] = wd;
    }
  }
  l_run = lsum;
  // The packed P^ must exist before the rescale branch below: otherwise the exp work is sunk
  // past it and a rescale waits on the previous tile's PV MFMAs instead of overlapping them.
  asm volatile("" : "+v"(pf));
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
    const v4i lo = *reinterpret_cast<const v4i*>(&sV[vlo + 32 * kBK * c]);
    const v4i hi = *reinterpret_cast<const v4i*>(&sV[vhi + 32 * kBK * c]);
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

// PIPE: the QK MFMAs of tile j+1 are issued before the softmax of tile j (one wave overlaps
// its own matrix and vector work); otherwise the waves of other work-groups provide the
// overlap.  NB: LDS ring slots.  OCC: work-groups per CU the register budget is sized for.
template <int D, bool CAUSAL, int OUT, bool ACC_VALU, bool QF8, bool PIPE, int NB, int OCC>  // OUT: 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256, OCC) void attn_fwd_kernel(AttnArgs a) {
  using TL = Tiles<D>;
  constexpr int NKS = D / 32;
  static_assert(!PIPE || NB == 4, "the pipelined loop uses a 4-slot ring");
  static_assert(NB >= 2 && NB <= 4, "ring size");
  __shared__ __attribute__((aligned(1024))) int8_t sK[NB][TL::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[NB][TL::VBYTES];
  __shared__ __attribute__((aligned(256))) float sDS[NB][kBK];
  __shared__ __attribute__((aligned(16))) float sDK[NB][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  // ---- work-group -> (head, query block) ----
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
  // V^ fragment offsets (the swizzle of rows 32 c + col does not depend on c); kept in two
  // registers rather than recomputed per tile
  int vlo = TL::voff(col, 2 * h), vhi = TL::voff(col, 2 * h + 1);
  asm volatile("" : "+v"(vlo), "+v"(vhi));

  v16f O[NKS];
#pragma unroll
  for (int c = 0; c < NKS; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) O[c][r] = 0.0f;
  // The running max starts at -FLT_MAX, not -inf: a row that sees no key in a tile (only
  // possible in a variable-length batch) then keeps alpha = 1, l = 0 and O = 0 instead of NaN,
  // and the epilogue writes it as 0.  Any visible score exceeds -FLT_MAX, so alpha on a row's
  // first visible tile is exactly 0, as with -inf.
  float m_run = -FLT_MAX, l_run = 0.0f;

  const int jend = CAUSAL ? max(0, min(nkts, (q0 + kBQ + coff + kBK - 1) / kBK)) : nkts;
  const int8_t* kbase = a.khat + (size_t)kvh * a.Mp * D;
  const uint8_t* vbase = a.vhat + (size_t)kvh * a.nkt * D * kBK;
  const float* dsbase = a.ds + ((size_t)bh * a.nqb + qb) * a.Mp;
  const float* dkbase = a.dk + (size_t)kvh * a.nkt * 4;

  // ---- staging: global -> LDS by DMA (global_load_lds), no registers, no LDS stores ----
  // Per-lane source offsets inside a tile (the swizzle is the same for every tile).
  int koffs[TL::KDMA], voffs[TL::VDMA];
#pragma unroll
  for (int i = 0; i < TL::KDMA; i++) {
    const int q = (TL::KDMA * w + i) * 64 + lane;  // 16-byte LDS chunk this lane fills
    const int r = q / TL::KCH;
    koffs[i] = r * D + 16 * ((q % TL::KCH) ^ TL::kswz(r));
  }
#pragma unroll
  for (int i = 0; i < TL::VDMA; i++) {
    const int q = (TL::VDMA * w + i) * 64 + lane;
    const int r = q >> 2;
    voffs[i] = r * kBK + 16 * ((q & 3) ^ TL::vswz(r));
  }
  auto dma = [&](int j, int slot) {
    const int8_t* kt = kbase + (size_t)j * kBK * D;
    const uint8_t* vt = vbase + (size_t)j * D * kBK;
#pragma unroll
    for (int i = 0; i < TL::KDMA; i++) dma16(lds_addr(&sK[slot][(TL::KDMA * w + i) * 1024]), kt, koffs[i]);
#pragma unroll
    for (int i = 0; i < TL::VDMA; i++) dma16(lds_addr(&sV[slot][(TL::VDMA * w + i) * 1024]), vt, voffs[i]);
    if (w == 0) dma4(lds_addr(&sDS[slot][0]), dsbase + (size_t)j * kBK, 4 * lane);
    if (w == 1 && lane < 4) dma4(lds_addr(&sDK[slot][0]), dkbase + (size_t)j * 4, 4 * lane);
  };
  // Wait until this wave's DMAs of all tiles but the newest one have landed (the newest
  // tile's instructions may stay in flight) and its own LDS reads are done, then barrier:
  // the next tile is visible to all and the slot read last iteration may be refilled.
  constexpr int kPerTile = TL::KDMA + TL::VDMA;  // DMA instructions per tile, waves 2 and 3
  auto publish = [&](bool newest_in_flight) {
    if (!newest_in_flight)
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (w < 2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPerTile + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPerTile) : "memory");
  };

  auto skip_t = [&](int j) { return CAUSAL && j * kBK > wq0 + 31 + coff; };  // fully masked for this wave
  if constexpr (PIPE) {
    // Software pipeline per wave: the QK MFMAs of tile j+1 are issued before the softmax of
    // tile j, so the matrix core works on j+1 while the VALU works on j.  Tile j+3 streams into
    // the ring slot last read in the previous iteration; two tiles are always in flight, and one
    // barrier per tile publishes the next.
    auto body = [&](int j, acc_t<QF8> (&cur)[2], acc_t<QF8> (&nxt)[2]) {
      if (j + 3 < jend) dma(j + 3, (j + 3) % NB);
      if (j + 1 < jend && !skip_t(j + 1)) qk_tile<D, QF8>(sK[(j + 1) % NB], qf, h, col, nxt);
      if (!skip_t(j)) {
        const int key0 = j * kBK;
        const bool masked = (CAUSAL && key0 + kBK - 1 > wq0 + coff) || (key0 + kBK > mseq);
        const int b = j % NB;
        softmax_pv<D, CAUSAL, ACC_VALU, acc_t<QF8>>(cur, sV[b], sDS[b], sDK[b], dql, h, col, vlo, vhi, key0, qrow + coff, mseq, masked, O,
                                        m_run, l_run);
      }
      publish(j + 3 < jend);  // tile j+2 must be complete; j+3 may still be arriving
    };

    if (jend > 0) dma(0, 0);
    if (jend > 1) dma(1, 1);
    if (jend > 2) dma(2, 2);
    publish(jend > 2);  // tiles 0 and 1 landed; tile 2 may be arriving
    acc_t<QF8> accA[2], accB[2];
    if (jend > 0) qk_tile<D, QF8>(sK[0], qf, h, col, accA);  // tile 0 is never masked away
    for (int j = 0; j < jend; j += 2) {
      body(j, accA, accB);
      if (j + 1 < jend) body(j + 1, accB, accA);
    }
  } else {
    // Ring of NB slots: tile j is computed from slot j % NB while tiles j+1 .. j+NB-1 stream
    // in; at the end of iteration j, tile j+1 must have landed and up to NB-2 newer tiles may
    // still be in flight (n tiles -> n times this wave's DMA instructions per tile).
    auto publish_n = [&](int n) {
      if (n <= 0)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (n == 1) {
        if (w < 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPerTile + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPerTile) : "memory");
      } else {
        if (w < 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kPerTile + 2) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kPerTile) : "memory");
      }
    };
    for (int t = 0; t < NB - 1 && t < jend; t++) dma(t, t);
    publish_n(min(NB - 2, jend - 1));  // tile 0 landed
    // One iteration; the slot is a compile-time constant so LDS addresses are immediates.
    auto iter = [&](int j, auto slotc) {
      constexpr int b = decltype(slotc)::value;
      if (j + NB - 1 < jend) dma(j + NB - 1, (b + NB - 1) % NB);  // the slot tile j-1 left
      if (!skip_t(j)) {
        const int key0 = j * kBK;
        const bool masked = (CAUSAL && key0 + kBK - 1 > wq0 + coff) || (key0 + kBK > mseq);
        acc_t<QF8> acc[2];
        qk_tile<D, QF8>(sK[b], qf, h, col, acc);
        softmax_pv<D, CAUSAL, ACC_VALU, acc_t<QF8>>(acc, sV[b], sDS[b], sDK[b], dql, h, col, vlo, vhi, key0, qrow + coff, mseq, masked, O,
                                        m_run, l_run);
      }
      publish_n(min(NB - 2, jend - j - 2));
    };
    for (int j0 = 0; j0 < jend; j0 += NB) {
      static_for<0, NB>([&](auto slotc) {
        const int j = j0 + decltype(slotc)::value;
        if (j < jend) iter(j, slotc);
      });
    }
  }

  // ---- epilogue: O / l (l holds 448 * sum P~) * dV (+ V_m); 0 for a row that saw no key ----
  const float l_tot = pair_sum(l_run);
  if (qrow >= nseq) return;
  const float inv = 1.0f / l_tot;
  const bool none = l_tot == 0.0f;
  const float* dvp = a.dv + (size_t)kvh * D;
  const float* vmp = a.vmean + (size_t)kvh * D;
  const SeqRows ro = seq_rows(a.ql, bseq, bh % a.H, a.H, D);
  const size_t orow = ro.base + (size_t)qrow * ro.stride;
  // per 32-channel group: its dV and V_m loads all issued before its stores (the stores may
  // alias them as far as the compiler knows, which would otherwise serialize every load)
#pragma unroll
  for (int c = 0; c < NKS; c++) {
    float4 dv4[4], vm4[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ch = 32 * c + 8 * b + 4 * h;
      dv4[b] = *reinterpret_cast<const float4*>(dvp + ch);
      vm4[b] = *reinterpret_cast<const float4*>(vmp + ch);
    }
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ch = 32 * c + 8 * b + 4 * h;
      const float dvv[4] = {dv4[b].x, dv4[b].y, dv4[b].z, dv4[b].w};
      const float vmv[4] = {vm4[b].x, vm4[b].y, vm4[b].z, vm4[b].w};
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; k++) o[k] = none ? 0.0f : fmaf(O[c][4 * b + k] * inv, dvv[k], vmv[k]);
      store_out4<OUT>(a.out, orow + ch, o);
    }
  }
}

// Loop shape of the fused kernel.  Default (measured fastest at prefill 32k): the plain loop
// with a 2-slot ring and registers budgeted for three work-groups per CU, so that three
// waves per SIMD overlap one another's matrix and vector work.  The software-pipelined
// 4-slot form (two work-groups per CU) stays selectable for comparison.
#ifndef SAGE_ATTN_PIPE
#define SAGE_ATTN_PIPE 0
#endif
#ifndef SAGE_ATTN_OCC
#define SAGE_ATTN_OCC 0  // 0: per head dimension (d = 64 fits four work-groups per CU, d = 128 three)
#endif
#ifndef SAGE_ATTN_RING
#define SAGE_ATTN_RING 2
#endif
constexpr bool kPipe = SAGE_ATTN_PIPE != 0;
constexpr int kRing = kPipe ? 4 : SAGE_ATTN_RING;
template <int D>
constexpr int occ_for() {
  return kPipe ? 2 : (SAGE_ATTN_OCC ? SAGE_ATTN_OCC : (D == 64 ? 4 : 3));
}

struct LaunchEv {
  hipEvent_t e0, e1;
};

template <int D, bool CAUSAL, bool ACC_VALU, bool QF8>
hipError_t launch_d(const Problem& p, const AttnArgs& a, hipStream_t s, LaunchEv ev) {
  dim3 grid(p.nqb * p.BH);
  const int out = p.out_fp32 ? 2 : (p.fp16 ? 1 : 0);
  if (out == 2)
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 2, ACC_VALU, QF8, kPipe, kRing, occ_for<D>()>), grid, dim3(256), 0,
                          s, ev.e0, ev.e1, 0, a);
  else if (out == 1)
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 1, ACC_VALU, QF8, kPipe, kRing, occ_for<D>()>), grid, dim3(256), 0,
                          s, ev.e0, ev.e1, 0, a);
  else
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, 0, ACC_VALU, QF8, kPipe, kRing, occ_for<D>()>), grid, dim3(256), 0,
                          s, ev.e0, ev.e1, 0, a);
  return hipGetLastError();
}

template <int D, bool ACC_VALU, bool QF8>
hipError_t launch_c(const Problem& p, const AttnArgs& a, hipStream_t s, LaunchEv ev) {
  return p.causal ? launch_d<D, true, ACC_VALU, QF8>(p, a, s, ev) : launch_d<D, false, ACC_VALU, QF8>(p, a, s, ev);
}

template <int D, bool ACC_VALU>
hipError_t launch_q(const Problem& p, const AttnArgs& a, hipStream_t s, LaunchEv ev) {
  return p.qf8 ? launch_c<D, ACC_VALU, true>(p, a, s, ev) : launch_c<D, ACC_VALU, false>(p, a, s, ev);
}

}  // namespace

hipError_t launch_attn_fwd(const Problem& p, const Workspace& w, void* out, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  AttnArgs a;
  a.qhat = w.qhat; a.khat = w.khat; a.vhat = w.vhat; a.dq = w.dq; a.dk = w.dk; a.dv = w.dv;
  a.vmean = w.vmean; a.ds = w.ds; a.out = out;
  a.BH = p.BH; a.nqb = p.nqb; a.nkt = p.nkt; a.Np = p.Np; a.Mp = p.Mp;
  a.causal2 = p.causal == 2 ? 1 : 0;
  a.ql = p.ql; a.kl = p.kl;
  a.qk_scale = p.sm_scale * kLog2e;
  a.H = p.H; a.Hkv = p.Hkv; a.G = p.G;
  a.xcd_map = (p.BH % (kXCD * p.G) == 0) ? 1 : 0;
  const bool valu = (p.variant & SAGE_ACC_VALU) != 0;
  const LaunchEv ev{e0, e1};
  if (p.d == 128) return valu ? launch_q<128, true>(p, a, s, ev) : launch_q<128, false>(p, a, s, ev);
  return valu ? launch_q<64, true>(p, a, s, ev) : launch_q<64, false>(p, a, s, ev);
}

}  // namespace sage
