// preprocess.hip -- smoothing, quantization and the Delta S correction (gfx950).
//
// "SageAttention2 Technical Report" summary, 3.4:
//   * "Smoothing Q": k = mean(K) over all tokens of the head, gamma(K) = K - k; for each
//     128-query block q_i = mean(Q_i), gamma(Q_i) = Q_i - q_i, and the GEMV correction
//     Delta S_ij = q_i gamma(K_j)^T added back after dequantization.
//   * "Per-Thread INT4 Quantization" (here INT8): one scale per thread fragment of the
//     S^T = K^ Q^T MFMA -- per query token for Q, per 16-key group for K.
//   * "FP8 Quantization for P~V": dV[c] = max_t |V[t,c]| / 448, V^ = E4M3(V / dV).
//   * "Optional Smoothing of V": V' = V - V_m before the V quantizer.
// "Quantization for Attention, in depth", "Failure modes": means and scales cover valid
// tokens only.
//
// Pinned values: FP64 sums in a fixed order (64-token chunks in token order, chunk sums in
// chunk order, one FP64 division, one rounding to FP32), IEEE FP32 division for every scale
// and code, round-half-even -- so Q^, K^, V^, the scales and the means have exactly one
// correct value.  max_t |V' [t,c]| comes from the per-channel max and min of V: FP32
// subtraction of a fixed V_m is monotone, so max |fp32(V - V_m)| = max(fp32(max V - V_m),
// fp32(V_m - min V)) exactly, and V is read twice, not three times.
//
// Launches, in order on the caller's stream: stats (one grid: the Q blocks first, then the
// K / V chunk statistics) reads the inputs once; kv_finalize turns chunk statistics into means
// and the V scale; kv_quant reads K and V once more and writes K^, V^ and Delta S.  Delta S_i[t] = q_i . gamma(K)[t] for one
// 64-key tile against every query block is a small GEMM done on the bf16 MFMA with both
// operands split into a bf16 head and tail (x = hi + lo, exact to 2^-16 relative), three
// products accumulated in FP32 -- FP32-class accuracy at matrix-core speed.
#include "sage_common.hpp"

namespace sage {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// 8 consecutive 16-bit inputs widened to FP32.
__device__ __forceinline__ void widen8(const v4i& raw, bool fp16, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const uint32_t u = static_cast<uint32_t>(raw[e]);
    const uint16_t lo = static_cast<uint16_t>(u & 0xffffu), hi = static_cast<uint16_t>(u >> 16);
    if (fp16) {
      x[2 * e] = static_cast<float>(__builtin_bit_cast(_Float16, lo));
      x[2 * e + 1] = static_cast<float>(__builtin_bit_cast(_Float16, hi));
    } else {
      x[2 * e] = __uint_as_float(u << 16);
      x[2 * e + 1] = __uint_as_float(u & 0xffff0000u);
    }
  }
}

// ---- K and V chunk statistics.  A wave takes one 64-token chunk of K or of V; lane l owns
// channels D/64 l .. +D/64-1 and loads the chunk's rows straight into registers, all 64
// loads in flight (one wave load reads a row's 128 or 256 contiguous bytes), then adds them in
// token order (FP64); for V also the max / min (one float2 per channel), and the sum when
// smoothing.  Work-group u2 of key/value head bh: waves 0, 1 take chunk 2 u2 (K, V), waves
// 2, 3 chunk 2 u2 + 1; with K only (SageBwd needs no V statistics), wave w takes chunk 4 u2 + w ----
struct StatsArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  // Q side (q_prep)
  int8_t* qhat;
  float* dq;
  uint8_t* qsc;
  float* qmean;
  uint16_t* qm_hi;
  uint16_t* qm_lo;
  // K / V side
  double* kpart;
  double* vpart;
  float2* vmm;
  SeqLayout ql, kl;
  int H, Hkv, Np, nqb, nkt;
  int nq_blocks;  // work-groups of the Q side (0: statistics only), interleaved with the K / V side
  int nkv_x;      // work-groups of the K / V side per key/value head
  int nkv_total;  // work-groups of the K / V side
  bool fp16, smooth_v;
  bool k_only;    // K's chunks only (no V statistics): every wave takes a chunk of K
};

template <int D>
__device__ __forceinline__ void kv_stats_block(const StatsArgs& a, int u2, int bh) {
  constexpr int CPL = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = a.k_only ? 4 * u2 + w : 2 * u2 + (w >> 1);
  const bool isv = !a.k_only && (w & 1) != 0;
  if (u >= a.nkt) return;
  const SeqRows R = seq_rows(a.kl, bh / a.Hkv, bh % a.Hkv, a.Hkv, D);
  const int t0 = u * kBK;
  if (t0 >= R.len) return;  // past this sequence's keys: no chunk
  const int n = min(kBK, R.len - t0);
  const uint16_t* src = (isv ? a.V : a.K) + R.base + (size_t)t0 * R.stride + CPL * lane;
  uint32_t raw[kBK];  // row t (clamped to the chunk's last valid row), this lane's channels
#pragma unroll
  for (int t = 0; t < kBK; t++) {
    const size_t off = (size_t)min(t, n - 1) * R.stride;
    raw[t] = CPL == 2 ? *reinterpret_cast<const uint32_t*>(src + off) : (uint32_t)src[off];
  }
  auto val = [&](int t, int j) {
    const uint32_t hbits = CPL == 2 ? (j ? raw[t] >> 16 : raw[t] & 0xffffu) : raw[t];
    return a.fp16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hbits)))
                  : __uint_as_float(hbits << 16);
  };
  const size_t o = ((size_t)bh * a.nkt + u) * D + CPL * lane;
  double sm[CPL];
  float mx[CPL], mn[CPL];
#pragma unroll
  for (int j = 0; j < CPL; j++) {
    sm[j] = 0.0;
    mx[j] = -INFINITY;
    mn[j] = INFINITY;
  }
  if (!isv) {
#pragma unroll
    for (int t = 0; t < kBK; t++)
      if (t < n)
#pragma unroll
        for (int j = 0; j < CPL; j++) sm[j] += (double)val(t, j);
#pragma unroll
    for (int j = 0; j < CPL; j++) a.kpart[o + j] = sm[j];
  } else {
#pragma unroll
    for (int t = 0; t < kBK; t++)
      if (t < n)
#pragma unroll
        for (int j = 0; j < CPL; j++) {
          const float x = val(t, j);
          if (a.smooth_v) sm[j] += (double)x;
          mx[j] = x > mx[j] ? x : mx[j];  // NaN ignored
          mn[j] = x < mn[j] ? x : mn[j];
        }
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      if (a.smooth_v) a.vpart[o + j] = sm[j];
      a.vmm[o + j] = make_float2(mx[j], mn[j]);
    }
  }
}

// ---- chunk statistics -> K mean, V_m (when smoothing) and the V scale ----
// One work-group per key/value head, 3 d threads in three roles: thread c < d adds channel c's K
// chunk sums, thread d + c takes channel c's V max / min, thread 2 d + c adds its V sums (when
// smoothing); each in chunk order, as the pinned order requires.  A chunk's partials of one array
// are d contiguous values, so the d threads of a role read each chunk row as one contiguous
// piece (1 KiB for the FP64 sums at d = 128), a batch of rows at a time, two batches in flight
// while a third is added.
struct FinArgs {
  const double* kpart;
  const double* vpart;
  const float2* vmm;
  float* kmean;
  float* vmean;
  float* dv;
  SeqLayout kl;
  int Hkv, d, nkt;
  bool smooth_v;
  bool k_only;  // the K mean only (no V statistics were taken)
};

// In-order reduction of one channel's nk chunk values (stride `stride` elements apart): the sum
// (T = double) or the max / min pair (T = float2).  Three batches of B loads rotate, so that two
// are in flight while the third is combined.
template <int B, typename T, typename F>
__device__ __forceinline__ void fin_chain(const T* __restrict__ p, size_t stride, int nk, F&& take) {
  T a[B], b[B], c[B];
  // rows past the last chunk re-read it (always in bounds; not combined): every batch issues the
  // same loads, so the compiler's waits keep the other two batches in flight
  auto load = [&](T (&x)[B], int u0) {
#pragma unroll
    for (int e = 0; e < B; e++) x[e] = p[(size_t)min(u0 + e, nk - 1) * stride];
  };
  auto use = [&](const T (&x)[B], int u0) {
    if (u0 + B <= nk) {  // a whole batch: the plain chain
#pragma unroll
      for (int e = 0; e < B; e++) take(x[e]);
    } else {
#pragma unroll
      for (int e = 0; e < B; e++)
        if (u0 + e < nk) take(x[e]);
    }
  };
  if (nk <= 0) return;
  load(a, 0);
  load(b, B);
  for (int u0 = 0; u0 < nk; u0 += 3 * B) {
    load(c, u0 + 2 * B);
    use(a, u0);
    if (u0 + B >= nk) break;
    load(a, u0 + 3 * B);
    use(b, u0 + B);
    if (u0 + 2 * B >= nk) break;
    load(b, u0 + 4 * B);
    use(c, u0 + 2 * B);
  }
}

// B: chunk rows per batch of loads (32 for long sequences, 8 for short ones, whose last batches
// would otherwise mostly re-read the last chunk)
template <int B>
__global__ __launch_bounds__(384) void kv_finalize_kernel(FinArgs f) {
  __shared__ float svm[128];  // V_m per channel, from the V-sum role to the max / min role
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int role = tid / f.d, c = tid % f.d;
  const int M = seq_rows(f.kl, bh / f.Hkv, bh % f.Hkv, f.Hkv, f.d).len;  // this sequence's keys
  const int nk = (M + kBK - 1) / kBK;                                    // its chunks
  const size_t o = (size_t)bh * f.nkt * f.d + c;  // channel c of chunk 0; chunk u at o + u d
  if (role == 0) {
    double ks = 0.0;
    fin_chain<B>(f.kpart + o, (size_t)f.d, nk, [&](double x) { ks += x; });
    // a sequence without keys (variable-length batches only) gets zero means and the floor scale
    f.kmean[(size_t)bh * f.d + c] = M > 0 ? (float)(ks / (double)M) : 0.0f;
  } else if (role == 2) {
    double vs = 0.0;
    if (f.smooth_v && !f.k_only) fin_chain<B>(f.vpart + o, (size_t)f.d, nk, [&](double x) { vs += x; });
    svm[c] = (f.smooth_v && M > 0) ? (float)(vs / (double)M) : 0.0f;
  }
  __syncthreads();
  if (role == 1 && !f.k_only) {
    float mx = -INFINITY, mn = INFINITY;
    fin_chain<B>(f.vmm + o, (size_t)f.d, nk, [&](float2 m) {
      mx = m.x > mx ? m.x : mx;  // NaN ignored
      mn = m.y < mn ? m.y : mn;
    });
    const float vm = svm[c];
    f.vmean[(size_t)bh * f.d + c] = vm;
    const float a1 = mx - vm, a2 = vm - mn;  // max |fp32(V - V_m)| over the tokens
    const float am = a1 > a2 ? a1 : a2;
    const float a = am > 1e-8f ? am : 1e-8f;
    f.dv[(size_t)bh * f.d + c] = __fdiv_rn(a, 448.0f);
  }
}

// ---- Q: block mean (and its bf16 head/tail), gamma(Q), per-token scale, INT8 (F8: E4M3) codes;
// query block i of query head bh ----
template <int D, bool MX, bool F8>
__device__ __forceinline__ void q_prep_block(const StatsArgs& a, int i, int bh) {
  const uint16_t* __restrict__ Q = a.Q;
  int8_t* __restrict__ qhat = a.qhat;
  float* __restrict__ dq = a.dq;
  uint8_t* __restrict__ qsc = a.qsc;
  const int H = a.H, Np = a.Np, nqb = a.nqb;
  const bool fp16 = a.fp16;
  constexpr int RS = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sq[kBQ * RS];
  __shared__ float sm[D];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const SeqRows R = seq_rows(a.ql, bh / H, bh % H, H, D);
  const int r0 = i * kBQ;
  if (r0 >= R.len) return;  // past this sequence's queries: the block is never read
  const int n = min(kBQ, R.len - r0);
  const size_t in_base = R.base + (size_t)r0 * R.stride;
  {
    // all of this thread's row chunks in flight at once (rows past the block's last valid row
    // re-read that row and are not stored; nothing reads them), then into LDS
    constexpr int NCH = kBQ * D / 8 / 256;
    v4i raw[NCH];
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const int x = tid + 256 * k, r = x / (D / 8), c0 = (x % (D / 8)) * 8;
      raw[k] = *reinterpret_cast<const v4i*>(Q + in_base + (size_t)min(r, n - 1) * R.stride + c0);
    }
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const int x = tid + 256 * k, r = x / (D / 8), c0 = (x % (D / 8)) * 8;
      if (r < n) *reinterpret_cast<v4i*>(&sq[r * RS + c0]) = raw[k];
    }
  }
  __syncthreads();
  if (tid < D) {
    double s = 0.0;  // rows in order, FP64 (8 LDS reads in flight)
    for (int rb = 0; rb < n; rb += 8) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = load_in(sq, (size_t)min(rb + e, kBQ - 1) * RS + tid, fp16);
#pragma unroll
      for (int e = 0; e < 8; e++)
        if (rb + e < n) s += (double)x[e];
    }
    const float m = (float)(s / (double)n);
    sm[tid] = m;
    const size_t o = ((size_t)bh * nqb + i) * D + tid;
    a.qmean[o] = m;
    const uint16_t hb = bf16_rn(m);
    // head / tail in the Delta S MFMA's B-operand order: per group of 32 blocks, channel step
    // s = c / 16, lane 32 ((c % 16) / 8) + block % 32, 8 bf16 per lane
    const size_t sw = ((((size_t)bh * ((nqb + 31) / 32) + i / 32) * (D / 16) + tid / 16) * 64 +
                       32 * ((tid % 16) / 8) + i % 32) * 8 + tid % 8;
    a.qm_hi[sw] = hb;
    a.qm_lo[sw] = bf16_rn(m - bf16_val(hb));
  }
  __syncthreads();
  // Each wave takes 32 rows.  A row is spread over LPR = D/8 lanes holding 8 consecutive
  // channels each (one 16-byte LDS read); a wave quantizes 64/LPR rows per step, and the
  // row / block maxima are short reductions inside each lane group.
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPS = 64 / LPR;       // rows per wave step
  const int sub = lane / LPR, cl = lane % LPR, c0 = 8 * cl;
  float mch[8];
#pragma unroll
  for (int e = 0; e < 8; e++) mch[e] = sm[c0 + e];
  for (int rr = 0; rr < kBQ / 4; rr += RPS) {
    const int r = wave * (kBQ / 4) + rr + sub;
    const size_t row = (size_t)bh * Np + r0 + r;
    float g[8];
    if (r < n) {
      const v4i raw = *reinterpret_cast<const v4i*>(&sq[r * RS + c0]);
      widen8(raw, fp16, g);
#pragma unroll
      for (int e = 0; e < 8; e++) g[e] = g[e] - mch[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; e++) g[e] = 0.0f;
    }
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) am = amax_upd(am, g[e]);
    if constexpr (MX) {
      am = group_max<4>(am);  // one E8M0 scale per 32 channels: 4 lanes
      const uint32_t code = e8m0_code(am);  // padded rows: amax 0 -> code 0, values 0
      const float sc = __uint_as_float(code << 23);
      uint32_t wd = 0;
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[0], g[1], sc, 0);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[2], g[3], sc, 1);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[4], g[5], sc, 2);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[6], g[7], sc, 3);
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(qhat) + row * (D / 2) + c0 / 2) = wd;
      if ((cl & 3) == 0) qsc[row * (D / 32) + cl / 4] = (uint8_t)code;
    } else {
      am = group_max<LPR>(am);
      const float sc = (r < n) ? (F8 ? e4m3_scale(am) : int8_scale(am)) : 1.0f;
      if (cl == 0) dq[row] = sc;
      uint2 w = make_uint2(0u, 0u);
      if (r < n) w = F8 ? e4m3_pack8_rcp(g, sc, __fdiv_rn(1.0f, sc)) : int8_pack8_rcp(g, sc, __fdiv_rn(1.0f, sc));
      *reinterpret_cast<uint2*>(qhat + row * D + c0) = w;
    }
  }
}

// ---- the first preprocessing launch: the Q blocks and the K / V chunk statistics side by side.
// Neither needs the other; the two kinds are interleaved in the grid (alternately, while both
// last) so that the CUs run both at once: the Q blocks wait on their serial block-mean chains,
// the K / V blocks stream ----
template <int D, bool MX, bool F8>
__global__ __launch_bounds__(256) void stats_kernel(StatsArgs a) {
  const int x = blockIdx.x;
  const int nkv = a.nkv_total;
  const int both = 2 * min(a.nq_blocks, nkv);  // [0, both): even x a Q block, odd x a K / V block
  int qi = -1, kvi = -1;
  if (x < both) {
    if (x & 1) kvi = x >> 1;
    else qi = x >> 1;
  } else if (a.nq_blocks > nkv) {
    qi = x - nkv;
  } else {
    kvi = x - a.nq_blocks;
  }
  if (qi >= 0) q_prep_block<D, MX, F8>(a, qi % a.nqb, qi / a.nqb);
  else kv_stats_block<D>(a, kvi % a.nkv_x, kvi / a.nkv_x);
}

struct KVArgs {
  const uint16_t* K;
  const uint16_t* V;
  const float* kmean;
  const float* vmean;
  const float* dv;
  const uint16_t* qm_hi;
  const uint16_t* qm_lo;
  int8_t* khat;
  float* dk;
  uint8_t* vhat;
  float* ds;  // null: no Delta S
  uint8_t* ksc;  // MX: E8M0 of gamma(K) blocks, [BH][nkt][64][4]
  uint8_t* vsc;  // MX: E8M0 of V' blocks, [BH][nkt][64][4]
  float ds_scale;
  int Mp, nkt, nqb, causal;  // nkt, nqb, Mp: the bounds (padded workspace strides)
  int H, Hkv, G;  // query heads, key/value heads, query heads per key/value head
  SeqLayout ql, kl;  // rows of q and of k, v
  bool fp16;
};

// ---- one 64-key tile of one key/value head (blockIdx.y): gamma(K), group scales, K^;
// Delta S against every query block of every query head that reads this key/value head;
// V' / dV -> E4M3, transposed in the P-fragment key order.  MX: gamma(K) and V' in E2M1
// with an E8M0 scale per 32 channels of a key / per 32 tokens of a channel ----
template <int D, bool MX, bool F8>
__global__ __launch_bounds__(256, MX ? 3 : 4) void kv_quant_kernel(KVArgs a) {
  constexpr int RS = D + 8;                 // bf16 split of gamma(K), 16-byte aligned rows
  constexpr int CH = kBK * D / 8 / 256;     // 8-element chunks per thread
  // The bf16 split of gamma(K) (read by the Delta S MFMAs) and the staged V' (read by the
  // transposing V^ writer) are live one after the other: they share one LDS buffer, which
  // lets four work-groups share a CU.
  constexpr int kSplitBytes = 2 * kBK * RS * 2, kVBytes = kBK * (D + 1) * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSplitBytes > kVBytes ? kSplitBytes : kVBytes];
  uint16_t* sAh = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sAl = sAh + kBK * RS;
  float (*sv)[D + 1] = reinterpret_cast<float (*)[D + 1]>(smem);
  __shared__ float gmax[4][4];
  __shared__ float sdk[4], srk[4];  // K group scales and their reciprocals
  __shared__ float ssv[MX ? 1 : D], srv[MX ? 1 : D];  // dV and 1 / dV per channel (srv: d = 64)
  const int u = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int b = bh / a.Hkv;
  const SeqRows R = seq_rows(a.kl, b, bh % a.Hkv, a.Hkv, D);
  const int t0 = u * kBK;
  if (t0 >= R.len) return;  // past this sequence's keys: the tile is never read
  const int n = min(kBK, R.len - t0);
  const size_t in_base = R.base + (size_t)t0 * R.stride;
  const float* km = a.kmean + (size_t)bh * D;
  // dV of channel tid: loaded with the K/V chunks, inverted into srv once Delta S is done
  const float dv_t = (!MX && tid < D) ? a.dv[(size_t)bh * D + tid] : 1.0f;

  // ---- all of this thread's K and V chunks in flight at once ----
  v4i kraw[CH], vraw[CH];
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int x = tid + 256 * i, row = x / (D / 8), c0 = (x % (D / 8)) * 8;
    const size_t off = in_base + (size_t)min(row, n - 1) * R.stride + c0;  // rows >= n are not used
    kraw[i] = *reinterpret_cast<const v4i*>(a.K + off);
    vraw[i] = *reinterpret_cast<const v4i*>(a.V + off);
  }

  // ---- gamma(K) = K - k (FP32), its bf16 split into LDS, group maxima ----
  float g[CH][8];
  float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int x = tid + 256 * i, row = x / (D / 8), c0 = (x % (D / 8)) * 8;
    if (row < n) {
      float w[8];
      widen8(kraw[i], a.fp16, w);
#pragma unroll
      for (int e = 0; e < 8; e++) g[i][e] = w[e] - km[c0 + e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; e++) g[i][e] = 0.0f;
    }
    if constexpr (!MX) {
      const int grp = kgroup(row);
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; e++) m = amax_upd(m, g[i][e]);
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (q == grp) am[q] = m > am[q] ? m : am[q];
    }
    v4i hv, lv;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint16_t h0 = bf16_rn(g[i][2 * e]), h1 = bf16_rn(g[i][2 * e + 1]);
      const uint16_t l0 = bf16_rn(g[i][2 * e] - bf16_val(h0)), l1 = bf16_rn(g[i][2 * e + 1] - bf16_val(h1));
      hv[e] = (int)((uint32_t)h0 | ((uint32_t)h1 << 16));
      lv[e] = (int)((uint32_t)l0 | ((uint32_t)l1 << 16));
    }
    *reinterpret_cast<v4i*>(&sAh[row * RS + c0]) = hv;
    *reinterpret_cast<v4i*>(&sAl[row * RS + c0]) = lv;
  }
  if constexpr (MX) {
    // ---- K^ in E2M1: the 4 threads holding a key's 32-channel block are consecutive lanes ----
    uint8_t* kout = reinterpret_cast<uint8_t*>(a.khat) + ((size_t)bh * a.Mp + t0) * (D / 2);
    uint8_t* sco = a.ksc + ((size_t)bh * a.nkt + u) * 256;
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const int x = tid + 256 * i, row = x / (D / 8), c0 = (x % (D / 8)) * 8;
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; e++) m = amax_upd(m, g[i][e]);
      m = group_max<4>(m);
      const uint32_t code = e8m0_code(m);  // keys >= M: all zero -> code 0, codes 0
      const float sc = __uint_as_float(code << 23);
      uint32_t wd = 0;
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[i][0], g[i][1], sc, 0);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[i][2], g[i][3], sc, 1);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[i][4], g[i][5], sc, 2);
      wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, g[i][6], g[i][7], sc, 3);
      *reinterpret_cast<uint32_t*>(kout + (size_t)row * (D / 2) + c0 / 2) = wd;
      if ((x & 3) == 0) {
        // A-operand scale of MFMA lane 32*(b%2) + row%32 (b = channel block), byte 2T + b/2
        const int b = c0 >> 5, T = row >> 5, l = 32 * (b & 1) + (row & 31);
        if (D == 128)
          sco[4 * l + 2 * T + (b >> 1)] = (uint8_t)code;
        else
          *reinterpret_cast<uint16_t*>(sco + 4 * l + 2 * T) = (uint16_t)code;  // byte 2T+1 = 0
      }
    }
  } else {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const float m = wave_max(am[q]);
    if (lane == 0) gmax[q][wave] = m;
  }
  __syncthreads();
  if (tid < 4) {
    float m = gmax[tid][0];
    for (int w = 1; w < 4; w++) m = gmax[tid][w] > m ? gmax[tid][w] : m;
    const float s = F8 ? e4m3_scale(m) : int8_scale(m);
    sdk[tid] = s;
    srk[tid] = __fdiv_rn(1.0f, s);
    a.dk[((size_t)bh * a.nkt + u) * 4 + tid] = s;
  }
  __syncthreads();

  // ---- K^ codes (keys >= M stay 0) ----
  {
    int8_t* kout = a.khat + ((size_t)bh * a.Mp + t0) * D;
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const int x = tid + 256 * i, row = x / (D / 8), c0 = (x % (D / 8)) * 8;
      uint2 w = make_uint2(0u, 0u);
      if (row < n)
        w = F8 ? e4m3_pack8_rcp(g[i], sdk[kgroup(row)], srk[kgroup(row)])
               : int8_pack8_rcp(g[i], sdk[kgroup(row)], srk[kgroup(row)]);
      *reinterpret_cast<uint2*>(kout + (size_t)row * D + c0) = w;
    }
  }
  }
  __syncthreads();  // sAh / sAl complete before the Delta S MFMAs read them

  // ---- Delta S^T[key][block] = gamma(K) q^T on the bf16 MFMA, split operands ----
  // Work units are (query head of this key/value head, group of 32 query blocks); a wave
  // takes units wave, wave + 4, ..., loads the group's q-mean head/tail once and computes
  // both 32-key halves of the tile against them.
  if (a.ds) {
    const int h = lane >> 5, col = lane & 31;
    // this sequence's query blocks and causal offset (key t visible to query r iff t <= r + coff);
    // under the causal mask, block i needs keys t <= 128 (i + 1) - 1 + coff
    const int nq = seq_rows(a.ql, b, 0, a.H, D).len;
    const int nqb = (nq + kBQ - 1) / kBQ;
    const int coff = a.causal == 2 ? R.len - nq : 0;
    const int ilo = (a.causal && t0 > coff) ? (t0 - coff) / kBQ : 0;
    const int ngrp = (nqb + 31) / 32, ngrp_all = (a.nqb + 31) / 32;  // this sequence's / the bound's
    for (int unit = wave; unit < a.G * ngrp; unit += 4) {
      const int g = unit / ngrp, gidx = unit % ngrp;
      if (32 * gidx + 31 < ilo) continue;
      const int bhq = (bh / a.Hkv) * a.H + (bh % a.Hkv) * a.G + g;  // query head
      const int blk = 32 * gidx + col;
      const bool bv = blk < nqb;
      // the block's q-mean head/tail, stored in this operand order: each load reads 1 KiB
      // contiguously (64 lanes x 16 bytes); all loads in flight
      const size_t qo = ((size_t)bhq * ngrp_all + gidx) * (D / 16) * 512 + (size_t)lane * 8;
      v8bf bq[D / 16], bl[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; s++) {
        bq[s] = bv ? *reinterpret_cast<const v8bf*>(a.qm_hi + qo + 512 * s) : v8bf{};
        bl[s] = bv ? *reinterpret_cast<const v8bf*>(a.qm_lo + qo + 512 * s) : v8bf{};
      }
#pragma unroll
      for (int T = 0; T < 2; T++) {
        v16f acc;
#pragma unroll
        for (int r = 0; r < 16; r++) acc[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < D / 16; s++) {
          const v8bf ah = *reinterpret_cast<const v8bf*>(&sAh[(32 * T + col) * RS + 16 * s + 8 * h]);
          const v8bf al = *reinterpret_cast<const v8bf*>(&sAl[(32 * T + col) * RS + 16 * s + 8 * h]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bq[s], acc, 0, 0, 0);  // small terms first
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[s], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bq[s], acc, 0, 0, 0);
        }
        if (bv && blk >= ilo) {
          float* dst = a.ds + ((size_t)bhq * a.nqb + blk) * a.Mp + t0 + 32 * T + 4 * h;
#pragma unroll
          for (int b = 0; b < 4; b++)
            *reinterpret_cast<float4*>(dst + 8 * b) =
                make_float4(acc[4 * b] * a.ds_scale, acc[4 * b + 1] * a.ds_scale, acc[4 * b + 2] * a.ds_scale,
                            acc[4 * b + 3] * a.ds_scale);
        }
      }
    }
  }
  if constexpr (!MX)
    if (tid < D) {
      ssv[tid] = dv_t;
      if constexpr (D == 64) srv[tid] = __fdiv_rn(1.0f, dv_t);
    }
  __syncthreads();  // the split of gamma(K) is dead: its LDS now stages V'; ssv, srv are complete

  // ---- V: V' / dV (the IEEE quotient's E4M3 value), saturated to the E4M3 range, staged in LDS ----
  // (MX: V' itself; the block scale comes from the staged values)
  {
    const float* vm = a.vmean + (size_t)bh * D;
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const int x = tid + 256 * i, row = x / (D / 8), c0 = (x % (D / 8)) * 8;
      float w[8];
      if (row < n) {
        widen8(vraw[i], a.fp16, w);
#pragma unroll
        for (int e = 0; e < 8; e++) w[e] = w[e] - vm[c0 + e];
        if constexpr (!MX) {
          if constexpr (D == 64) {
            e4m3_in8_rcp(w, ssv + c0, srv + c0);
          } else {  // d = 128: the product shortcut measured no faster here than the division
#pragma unroll
            for (int e = 0; e < 8; e++) {
              const float y = __fdiv_rn(w[e], ssv[c0 + e]);
              const float c = fminf(fmaxf(y, -448.0f), 448.0f);
              w[e] = (y == y) ? c : y;  // NaN stays NaN
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) w[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; e++) sv[row][c0 + e] = w[e];
    }
  }
  __syncthreads();
  if constexpr (MX) {
    // one thread per (channel, 32-token half): scale, then 32 codes in the vperm_mx order
    if (tid < 2 * D) {
      const int c = tid % D, T = tid / D;
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 32; k++) m = amax_upd(m, sv[32 * T + k][c]);
      const uint32_t code = e8m0_code(m);
      const float scf = __uint_as_float(code << 23);
      v4i out;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        // byte e of word q holds nibbles j = 8q + 2e, j + 1: keys vperm_mx(T, j), + 1
        const int k0 = vperm_mx(T, 8 * q), k1 = vperm_mx(T, 8 * q + 2);
        const int k2 = vperm_mx(T, 8 * q + 4), k3 = vperm_mx(T, 8 * q + 6);
        uint32_t wd = 0;
        wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, sv[k0][c], sv[k0 + 1][c], scf, 0);
        wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, sv[k1][c], sv[k1 + 1][c], scf, 1);
        wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, sv[k2][c], sv[k2 + 1][c], scf, 2);
        wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, sv[k3][c], sv[k3 + 1][c], scf, 3);
        out[q] = (int)wd;
      }
      uint8_t* vout = a.vhat + (((size_t)bh * a.nkt + u) * D + c) * (kBK / 2) + 16 * T;
      *reinterpret_cast<v4i*>(vout) = out;
      uint8_t* sco = a.vsc + ((size_t)bh * a.nkt + u) * 256 + 4 * (32 * T + (c & 31));
      sco[c >> 5] = (uint8_t)code;
      if (D == 64 && (c >> 5) == 1) *reinterpret_cast<uint16_t*>(sco + 2) = 0;  // bytes g >= d/32
    }
  } else {
    uint8_t* vout = a.vhat + ((size_t)bh * a.nkt + u) * (size_t)D * kBK;
    for (int x = tid; x < D * (kBK / 4); x += 256) {
      const int c = x / (kBK / 4), p0 = (x % (kBK / 4)) * 4;
      const int h = p0 >> 5, b0 = p0 & 31;
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(sv[kperm(h, b0)][c], sv[kperm(h, b0 + 1)][c], 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(sv[kperm(h, b0 + 2)][c], sv[kperm(h, b0 + 3)][c], wd, true);
      *reinterpret_cast<int*>(vout + (size_t)c * kBK + p0) = wd;
    }
  }
}

}  // namespace

hipError_t launch_stats(const Problem& p, const void* q, const void* k, const void* v, const Workspace& w,
                        hipStream_t s) {
  StatsArgs a;
  a.Q = (const uint16_t*)q;
  a.K = (const uint16_t*)k;
  a.V = (const uint16_t*)v;
  a.qhat = w.qhat; a.dq = w.dq; a.qsc = w.qsc; a.qmean = w.qmean; a.qm_hi = w.qm_hi; a.qm_lo = w.qm_lo;
  a.kpart = w.kpart; a.vpart = w.vpart; a.vmm = w.vmm;
  a.ql = p.ql; a.kl = p.kl;
  a.H = p.H; a.Hkv = p.Hkv; a.Np = p.Np; a.nqb = p.nqb; a.nkt = p.nkt;
  a.nq_blocks = q ? p.nqb * p.BH : 0;
  a.k_only = v == nullptr;  // K's mean only
  a.nkv_x = a.k_only ? (p.nkt + 3) / 4 : (p.nkt + 1) / 2;
  a.fp16 = p.fp16;
  a.smooth_v = p.smooth_v;
  const long long blocks = (long long)a.nq_blocks + (long long)a.nkv_x * p.BHkv;
  if (blocks >= (1LL << 31)) return hipErrorInvalidConfiguration;
  a.nkv_total = a.nkv_x * p.BHkv;
  const dim3 grid((unsigned)blocks);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a); };
  if (p.d == 128)
    p.mx ? go(stats_kernel<128, true, false>)
         : (p.qf8 ? go(stats_kernel<128, false, true>) : go(stats_kernel<128, false, false>));
  else
    p.mx ? go(stats_kernel<64, true, false>)
         : (p.qf8 ? go(stats_kernel<64, false, true>) : go(stats_kernel<64, false, false>));
  return hipGetLastError();
}

namespace {
hipError_t kv_finalize(const Problem& p, const Workspace& w, hipStream_t s, bool k_only) {
  FinArgs f;
  f.kpart = w.kpart; f.vpart = w.vpart; f.vmm = w.vmm;
  f.kmean = w.kmean; f.vmean = w.vmean; f.dv = w.dv;
  f.kl = p.kl; f.Hkv = p.Hkv; f.d = p.d; f.nkt = p.nkt; f.smooth_v = p.smooth_v && !k_only;
  f.k_only = k_only;
  if (p.nkt >= 96) hipLaunchKernelGGL(kv_finalize_kernel<32>, dim3(p.BHkv), dim3(3 * p.d), 0, s, f);
  else hipLaunchKernelGGL(kv_finalize_kernel<8>, dim3(p.BHkv), dim3(3 * p.d), 0, s, f);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_kv_finalize(const Problem& p, const Workspace& w, hipStream_t s) {
  return kv_finalize(p, w, s, false);
}

hipError_t launch_kv_finalize_k_only(const Problem& p, const Workspace& w, hipStream_t s) {
  return kv_finalize(p, w, s, true);
}

hipError_t launch_kv_quant(const Problem& p, const void* k, const void* v, const Workspace& w,
                           float ds_scale, float* ds_out, hipStream_t s) {
  KVArgs a;
  a.K = (const uint16_t*)k;
  a.V = (const uint16_t*)v;
  a.kmean = w.kmean;
  a.vmean = w.vmean;
  a.dv = w.dv;
  a.qm_hi = w.qm_hi;
  a.qm_lo = w.qm_lo;
  a.khat = w.khat;
  a.dk = w.dk;
  a.vhat = w.vhat;
  a.ds = ds_out;
  a.ksc = w.ksc;
  a.vsc = w.vsc;
  a.ds_scale = ds_scale;
  a.Mp = p.Mp;
  a.nkt = p.nkt;
  a.nqb = p.nqb;
  a.causal = p.causal;
  a.ql = p.ql;
  a.kl = p.kl;
  a.H = p.H;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.fp16 = p.fp16;
  const dim3 grid(p.nkt, p.BHkv);
  if (p.d == 128) {
    if (p.mx) hipLaunchKernelGGL((kv_quant_kernel<128, true, false>), grid, dim3(256), 0, s, a);
    else if (p.qf8) hipLaunchKernelGGL((kv_quant_kernel<128, false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((kv_quant_kernel<128, false, false>), grid, dim3(256), 0, s, a);
  } else {
    if (p.mx) hipLaunchKernelGGL((kv_quant_kernel<64, true, false>), grid, dim3(256), 0, s, a);
    else if (p.qf8) hipLaunchKernelGGL((kv_quant_kernel<64, false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((kv_quant_kernel<64, false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sage
