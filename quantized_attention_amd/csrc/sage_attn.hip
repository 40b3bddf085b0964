// sage_attn.hip -- C ABI entry points: argument checks, workspace, launch sequence.
//
// The sequence is the pages' forward pass ("SageAttention2 Technical Report" summary,
// 3.4 "The Complete Algorithm (Algorithm 1)" and 3.2 "Big-Picture Architecture"):
// preprocessing (K mean and K^, V scale and V^, Q block means and Q^, Delta S) as separate
// launches writing a device workspace, then one fused attention kernel.  All argument
// checks run before anything is enqueued; nothing here synchronizes the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "sage_common.hpp"
#include "sagebwd.hpp"

namespace sage {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_layout(const Problem& p, size_t* sizes) {
  const size_t BH = (size_t)p.BH, BK = (size_t)p.BHkv, d = (size_t)p.d;
  const size_t qd = p.mx ? d / 2 : d;                // bytes per quantized row
  size_t s[kWsSlices];
  s[0] = BH * p.Np * qd;                             // qhat
  s[1] = BK * p.Mp * qd;                             // khat
  s[2] = BK * p.nkt * d * (p.mx ? kBK / 2 : kBK);    // vhat
  s[3] = p.mx ? 0 : BH * p.Np * sizeof(float);       // dq
  s[4] = p.mx ? 0 : BK * p.nkt * 4 * sizeof(float);  // dk
  s[5] = BK * d * sizeof(float);                     // dv
  s[6] = BK * d * sizeof(float);                     // kmean
  s[7] = BK * d * sizeof(float);                     // vmean
  s[8] = BH * p.nqb * d * sizeof(float);             // qmean
  s[9] = BH * p.nqb * (size_t)p.Mp * sizeof(float);  // ds
  s[10] = BK * p.nkt * d * sizeof(double);           // kpart
  s[11] = BK * p.nkt * d * sizeof(double);           // vpart
  s[12] = BK * p.nkt * d * sizeof(float2);           // vmm
  s[13] = 0;                                         // (unused)
  const size_t nqb32 = (size_t)(p.nqb + 31) / 32 * 32;  // q-mean head/tail: groups of 32 blocks
  s[14] = BH * nqb32 * d * sizeof(uint16_t);         // qm_hi
  s[15] = BH * nqb32 * d * sizeof(uint16_t);         // qm_lo
  s[16] = p.mx ? BH * p.Np * (d / 32) : 0;           // qsc
  s[17] = p.mx ? BK * p.nkt * 256 : 0;               // ksc
  s[18] = p.mx ? BK * p.nkt * 256 : 0;               // vsc
  size_t tot = 0;
  for (int i = 0; i < kWsSlices; i++) {
    if (sizes) sizes[i] = s[i];
    tot += align256(s[i]);
  }
  return tot;
}

void carve_workspace(const Problem& p, void* base, Workspace* w) {
  size_t s[kWsSlices];
  workspace_layout(p, s);
  char* b = static_cast<char*>(base);
  void* ptr[kWsSlices];
  for (int i = 0; i < kWsSlices; i++) {
    ptr[i] = b;
    b += align256(s[i]);
  }
  w->qhat = (int8_t*)ptr[0];
  w->khat = (int8_t*)ptr[1];
  w->vhat = (uint8_t*)ptr[2];
  w->dq = (float*)ptr[3];
  w->dk = (float*)ptr[4];
  w->dv = (float*)ptr[5];
  w->kmean = (float*)ptr[6];
  w->vmean = (float*)ptr[7];
  w->qmean = (float*)ptr[8];
  w->ds = (float*)ptr[9];
  w->kpart = (double*)ptr[10];
  w->vpart = (double*)ptr[11];
  w->vmm = (float2*)ptr[12];
  w->qm_hi = (uint16_t*)ptr[14];
  w->qm_lo = (uint16_t*)ptr[15];
  w->qsc = (uint8_t*)ptr[16];
  w->ksc = (uint8_t*)ptr[17];
  w->vsc = (uint8_t*)ptr[18];
}

namespace {

constexpr unsigned kKnownBits =
    SAGE_PATH_MXFP4 | SAGE_QK_FP8 | SAGE_MX_P_TWO_LEVEL | SAGE_SMOOTH_V | SAGE_IN_FP16 | SAGE_OUT_FP32 |
    SAGE_ACC_VALU;

// Per-device "is gfx950" cache, filled once per device under a mutex.
int device_check() {
  static std::mutex mu;
  static signed char ok[64];
  static bool init = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return SAGE_ERR_DEVICE;
  std::lock_guard<std::mutex> g(mu);
  if (!init) {
    std::memset(ok, -1, sizeof(ok));
    init = true;
  }
  if (ok[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SAGE_ERR_DEVICE;
    ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 0;
  }
  return ok[dev] ? SAGE_OK : SAGE_ERR_UNSUPPORTED;
}

int make_problem(int B, int H, int Hkv, int N, int M, int d, int causal, float sm_scale, unsigned variant,
                 Problem* p) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || M < 1) return SAGE_ERR_INVALID_ARG;
  if (H % Hkv) return SAGE_ERR_INVALID_ARG;
  if (variant & ~kKnownBits) return SAGE_ERR_INVALID_ARG;
  if ((variant & SAGE_PATH_MXFP4) && (variant & SAGE_QK_FP8)) return SAGE_ERR_INVALID_ARG;
  if ((variant & SAGE_MX_P_TWO_LEVEL) && (!(variant & SAGE_PATH_MXFP4) || (variant & SAGE_ACC_VALU)))
    return SAGE_ERR_INVALID_ARG;
  if (causal < 0 || causal > 2) return SAGE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (causal == 2 && N > M) return SAGE_ERR_UNSUPPORTED;  // some rows would see no key
  const double big = (double)B * H * (double)(N > M ? N : M) * d;
  if (big >= 1099511627776.0) return SAGE_ERR_INVALID_ARG;  // 2^40 elements
  if ((long long)B * H > (1LL << 30)) return SAGE_ERR_INVALID_ARG;
  p->B = B; p->H = H; p->Hkv = Hkv; p->G = H / Hkv; p->N = N; p->M = M; p->d = d;
  p->causal = causal;
  p->sm_scale = (sm_scale > 0.0f && std::isfinite(sm_scale)) ? sm_scale : 1.0f / std::sqrt((float)d);
  p->variant = variant;
  p->BH = B * H;
  p->BHkv = B * Hkv;
  p->nqb = (N + kBQ - 1) / kBQ;
  p->nkt = (M + kBK - 1) / kBK;
  p->Np = p->nqb * kBQ;
  p->Mp = p->nkt * kBK;
  p->fp16 = (variant & SAGE_IN_FP16) != 0;
  p->out_fp32 = (variant & SAGE_OUT_FP32) != 0;
  p->smooth_v = (variant & SAGE_SMOOTH_V) != 0;
  p->mx = (variant & SAGE_PATH_MXFP4) != 0;
  p->qf8 = (variant & SAGE_QK_FP8) != 0;
  p->ql = {nullptr, N, 0};
  p->kl = {nullptr, M, 0};
  // grid limits: y = B*H (or B*Hkv) for the preprocessing kernels, x = blocks/tiles; the
  // one-dimensional grids of the fused and SageBwd kernels (B*H times the query blocks or the
  // key tiles, 256 work-items each) must count fewer than 2^32 work-items
  if (p->BH > 65535 || p->nkt > (1 << 30)) return SAGE_ERR_INVALID_ARG;
  if ((long long)p->BH * (p->nqb > p->nkt ? p->nqb : p->nkt) >= (1LL << 24)) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

int make_problem(const sage_attn_shape* sh, Problem* p) {
  if (!sh) return SAGE_ERR_INVALID_ARG;
  return make_problem(sh->B, sh->Hq, sh->Hkv, sh->N, sh->M, sh->d, sh->causal, sh->sm_scale, sh->variant, p);
}

// A variable-length batch is the dense problem with B = batch and N, M = the length bounds
// (the workspace is laid out for them); the kernels read each sequence's rows and lengths
// through the offsets.  causal = 2 with N > M is allowed here: the rows of a sequence that see
// no key are written as 0.
int make_problem(const sage_attn_varlen_shape* sh, Problem* p) {
  if (!sh || !sh->cu_seqlens_q || !sh->cu_seqlens_k) return SAGE_ERR_INVALID_ARG;
  if (sh->total_q < 1 || sh->total_k < 1) return SAGE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(sh->cu_seqlens_q) | reinterpret_cast<uintptr_t>(sh->cu_seqlens_k)) & 3u)
    return SAGE_ERR_INVALID_ARG;
  const int causal_check = sh->causal == 2 ? 1 : sh->causal;  // N > M is not an error here
  int rc = make_problem(sh->batch, sh->Hq, sh->Hkv, sh->max_seqlen_q, sh->max_seqlen_k, sh->d, causal_check,
                        sh->sm_scale, sh->variant, p);
  if (rc != SAGE_OK) return rc;
  if ((double)sh->total_q * sh->Hq * sh->d >= 1099511627776.0 || (double)sh->total_k * sh->Hkv * sh->d >= 1099511627776.0)
    return SAGE_ERR_INVALID_ARG;
  p->causal = sh->causal;
  p->ql = {sh->cu_seqlens_q, sh->max_seqlen_q, sh->total_q};
  p->kl = {sh->cu_seqlens_k, sh->max_seqlen_k, sh->total_k};
  return SAGE_OK;
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

// The preprocessing launches, in order on s; ds goes to ds_out scaled by ds_scale.  The first
// launch covers the Q blocks and the K / V chunk statistics together (both HBM-bound, neither
// needs the other); the chunk statistics are then reduced to the K mean, V_m and the V scale,
// which kv_quant needs.
int run_preprocess(const Problem& p, const void* q, const void* k, const void* v, const Workspace& w,
                   float ds_scale, float* ds_out, hipStream_t s) {
  if (launch_stats(p, q, k, v, w, s) != hipSuccess) return SAGE_ERR_LAUNCH;
  if (launch_kv_finalize(p, w, s) != hipSuccess) return SAGE_ERR_LAUNCH;
  if (launch_kv_quant(p, k, v, w, ds_scale, ds_out, s) != hipSuccess) return SAGE_ERR_LAUNCH;
  return SAGE_OK;
}

// Events of the measurement hook (per thread, consumed by the next forward call).
thread_local hipEvent_t t_prof_start = nullptr, t_prof_stop = nullptr;

int fwd_impl(const void* q, const void* k, const void* v, void* out, const Problem& p, void* ws,
             hipStream_t s) {
  Workspace w;
  carve_workspace(p, ws, &w);
  hipEvent_t e0 = t_prof_start, e1 = t_prof_stop;
  t_prof_start = t_prof_stop = nullptr;
  // the MX kernel adds Delta S through its matrix core's accumulator, before sm_scale log2(e);
  // the INT8/FP8 kernel adds it in its dequantizing FMA, scaled
  int rc = run_preprocess(p, q, k, v, w, p.mx ? 1.0f : p.sm_scale * 1.4426950408889634f, w.ds, s);
  if (rc != SAGE_OK) return rc;
  // the measurement events (if any) take the fused kernel's own start and end times
  if ((p.mx ? launch_attn_fwd_mx(p, w, out, s, e0, e1) : launch_attn_fwd(p, w, out, s, e0, e1)) != hipSuccess)
    return SAGE_ERR_LAUNCH;
  return SAGE_OK;
}

int check_io(const void* q, const void* k, const void* v, const void* out) {
  if (!q || !k || !v || !out) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// The forward of a resolved problem: argument checks, then the caller's workspace or a
// stream-ordered one.
int fwd_checked(const Problem& p, const void* q, const void* k, const void* v, void* out, void* workspace,
                size_t ws_bytes, void* stream) {
  int rc = check_io(q, k, v, out);
  if (rc != SAGE_OK) return rc;
  if (workspace) {
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return SAGE_ERR_INVALID_ARG;
    if (ws_bytes < workspace_layout(p, nullptr)) return SAGE_ERR_NO_MEMORY;
  }
  if ((rc = device_check()) != SAGE_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (workspace) return fwd_impl(q, k, v, out, p, workspace, s);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, workspace_layout(p, nullptr), s) != hipSuccess || !ws) {
    (void)hipGetLastError();
    return SAGE_ERR_NO_MEMORY;
  }
  rc = fwd_impl(q, k, v, out, p, ws, s);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == SAGE_OK) rc = SAGE_ERR_LAUNCH;
  return rc;
}

// Workspace of the no-allocation entry point: one array per device, held while the library is
// loaded.  In host code `scratch` is a stand-in symbol, not a device address; the device address
// of each GPU's copy comes from hipGetSymbolAddress on that GPU (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_MAX_BYTES];

// The device address of this device's scratch array, looked up once per device (with that
// device current) and kept; null if the lookup fails.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* ptr[64];
  static bool looked[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!looked[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;  // not cached: a later call may succeed
    }
    ptr[dev] = a;
    looked[dev] = true;
  }
  return ptr[dev];
}

// SageBwd problems: the dense shape with Hkv = Hq; the variant carries the input and output
// dtypes and the K-smoothing ablation.
int make_train_problem(const sage_attn_shape* sh, Problem* p, bool* smooth_k) {
  if (!sh) return SAGE_ERR_INVALID_ARG;
  constexpr unsigned kTrainOnly = SAGE_TRAIN_NO_SMOOTH_K | SAGE_TRAIN_RECOMPUTE_DS | SAGE_TRAIN_KEEP_QUANT;
  if (sh->variant & ~(SAGE_IN_FP16 | SAGE_OUT_FP32 | kTrainOnly)) return SAGE_ERR_INVALID_ARG;
  const int rc = make_problem(sh->B, sh->Hq, sh->Hkv, sh->N, sh->M, sh->d, sh->causal, sh->sm_scale,
                              sh->variant & ~kTrainOnly, p);
  if (rc != SAGE_OK) return rc;
  // read by the backward's layout and launch, and by the keeping of the quantized inputs
  p->variant |= sh->variant & (SAGE_TRAIN_RECOMPUTE_DS | SAGE_TRAIN_KEEP_QUANT);
  if (sh->Hkv != sh->Hq) return SAGE_ERR_UNSUPPORTED;
  *smooth_k = (sh->variant & SAGE_TRAIN_NO_SMOOTH_K) == 0;
  return SAGE_OK;
}

// A caller's workspace, or a stream-ordered one for the duration of `body`.
template <typename F>
int with_workspace(size_t need, void* workspace, size_t ws_bytes, hipStream_t s, F&& body) {
  if (workspace) {
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return SAGE_ERR_INVALID_ARG;
    if (ws_bytes < need) return SAGE_ERR_NO_MEMORY;
    return body(static_cast<char*>(workspace));
  }
  void* ws = nullptr;
  if (hipMallocAsync(&ws, need, s) != hipSuccess || !ws) {
    (void)hipGetLastError();
    return SAGE_ERR_NO_MEMORY;
  }
  int rc = body(static_cast<char*>(ws));
  if (hipFreeAsync(ws, s) != hipSuccess && rc == SAGE_OK) rc = SAGE_ERR_LAUNCH;
  return rc;
}

}  // namespace
}  // namespace sage

using namespace sage;

extern "C" {

size_t sage_attn_workspace_bytes_ex(const sage_attn_shape* shape) {
  Problem p;
  if (make_problem(shape, &p) != SAGE_OK) return 0;
  return workspace_layout(p, nullptr);
}

size_t sage_attn_workspace_bytes(int B, int H, int N, int M, int d, int causal, unsigned variant) {
  const sage_attn_shape sh = {B, H, H, N, M, d, causal, 0.0f, variant};
  return sage_attn_workspace_bytes_ex(&sh);
}

int sage_attn_fwd_ex(const sage_attn_shape* shape, const void* q, const void* k, const void* v, void* out,
                     void* workspace, size_t ws_bytes, void* stream) {
  Problem p;
  const int rc = make_problem(shape, &p);
  return rc != SAGE_OK ? rc : fwd_checked(p, q, k, v, out, workspace, ws_bytes, stream);
}

int sage_attn_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                     int M, int d, int causal, float sm_scale, unsigned variant, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (!workspace) return SAGE_ERR_INVALID_ARG;
  const sage_attn_shape sh = {B, H, H, N, M, d, causal, sm_scale, variant};
  return sage_attn_fwd_ex(&sh, q, k, v, out, workspace, ws_bytes, stream);
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int M,
                  int d, int causal, float sm_scale, unsigned variant, void* stream) {
  const sage_attn_shape sh = {B, H, H, N, M, d, causal, sm_scale, variant};
  return sage_attn_fwd_ex(&sh, q, k, v, out, nullptr, 0, stream);
}

int sage_attn_fwd_noalloc(const sage_attn_shape* shape, const void* q, const void* k, const void* v, void* out,
                          void* stream) {
  Problem p;
  int rc = make_problem(shape, &p);
  if (rc != SAGE_OK) return rc;
  if ((rc = check_io(q, k, v, out)) != SAGE_OK) return rc;
  if (workspace_layout(p, nullptr) > SAGE_NOALLOC_MAX_BYTES) return SAGE_ERR_NO_MEMORY;
  if ((rc = device_check()) != SAGE_OK) return rc;
  void* ws = scratch_on_current_device();
  if (!ws) return SAGE_ERR_DEVICE;
  return fwd_impl(q, k, v, out, p, ws, (hipStream_t)stream);
}

size_t sage_attn_varlen_workspace_bytes(const sage_attn_varlen_shape* shape) {
  Problem p;
  if (make_problem(shape, &p) != SAGE_OK) return 0;
  return workspace_layout(p, nullptr);
}

int sage_attn_varlen_fwd(const sage_attn_varlen_shape* shape, const void* q, const void* k, const void* v, void* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  Problem p;
  const int rc = make_problem(shape, &p);
  return rc != SAGE_OK ? rc : fwd_checked(p, q, k, v, out, workspace, ws_bytes, stream);
}

int sage_attn_quantize_ex(const sage_attn_shape* shape, const void* q, const void* k, const void* v,
                          const sage_quant_views* dst, void* stream) {
  Problem p;
  int rc = make_problem(shape, &p);
  if (rc != SAGE_OK) return rc;
  if (!dst || !q || !k || !v) return SAGE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return SAGE_ERR_INVALID_ARG;
  if ((rc = device_check()) != SAGE_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, workspace_layout(p, nullptr), s) != hipSuccess || !ws) {
    (void)hipGetLastError();
    return SAGE_ERR_NO_MEMORY;
  }
  Workspace w;
  carve_workspace(p, ws, &w);
  rc = run_preprocess(p, q, k, v, w, 1.0f, dst->delta_s, s);
  size_t sz[kWsSlices];
  workspace_layout(p, sz);
  struct Copy { void* dst; const void* src; size_t n; } copies[] = {
      {dst->q_hat, w.qhat, sz[0]}, {dst->k_hat, w.khat, sz[1]}, {dst->v_hat, w.vhat, sz[2]},
      {dst->dq, w.dq, sz[3]},      {dst->dk, w.dk, sz[4]},      {dst->dv, w.dv, sz[5]},
      {dst->k_mean, w.kmean, sz[6]}, {dst->v_mean, w.vmean, sz[7]}, {dst->q_mean, w.qmean, sz[8]},
      {dst->mx_scales_q, w.qsc, sz[16]}, {dst->mx_scales_k, w.ksc, sz[17]}, {dst->mx_scales_v, w.vsc, sz[18]}};
  for (const Copy& c : copies) {
    if (rc != SAGE_OK) break;
    if (c.dst && c.n && hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s) != hipSuccess) rc = SAGE_ERR_LAUNCH;
  }
  if (hipFreeAsync(ws, s) != hipSuccess && rc == SAGE_OK) rc = SAGE_ERR_LAUNCH;
  return rc;
}

int sage_attn_quantize(const void* q, const void* k, const void* v, int B, int H, int N, int M, int d,
                       int causal, unsigned variant, const sage_quant_views* dst, void* stream) {
  const sage_attn_shape sh = {B, H, H, N, M, d, causal, 0.0f, variant};
  return sage_attn_quantize_ex(&sh, q, k, v, dst, stream);
}

size_t sage_attn_train_workspace_bytes(const sage_attn_shape* shape) {
  Problem p;
  bool smooth_k;
  if (make_train_problem(shape, &p, &smooth_k) != SAGE_OK) return 0;
  return sb_layout(p, true, nullptr);
}

int sage_attn_train_fwd(const sage_attn_shape* shape, const void* q, const void* k, const void* v, void* out,
                        float* lse, void* workspace, size_t ws_bytes, void* stream) {
  Problem p;
  bool smooth_k;
  int rc = make_train_problem(shape, &p, &smooth_k);
  if (rc != SAGE_OK) return rc;
  // keeping the quantized inputs for the backward: they go to the backward's layout of the
  // caller's workspace
  const bool keep = (p.variant & SAGE_TRAIN_KEEP_QUANT) != 0;
  if (keep && !workspace) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_io(q, k, v, out)) != SAGE_OK) return rc;
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return SAGE_ERR_INVALID_ARG;
  if (workspace && ws_bytes < sb_layout(p, true, nullptr)) return SAGE_ERR_NO_MEMORY;
  if ((rc = device_check()) != SAGE_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  return with_workspace(sb_layout(p, keep, nullptr), workspace, ws_bytes, s, [&](char* ws) {
    if (sb_prep_fwd(p, q, k, v, ws, keep, smooth_k, s) != hipSuccess) return (int)SAGE_ERR_LAUNCH;
    if (sb_forward(p, ws, keep, out, lse, s) != hipSuccess) return (int)SAGE_ERR_LAUNCH;
    return (int)SAGE_OK;
  });
}

int sage_attn_train_bwd(const sage_attn_shape* shape, const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, float* dq, float* dk, float* dv, void* workspace,
                        size_t ws_bytes, void* stream) {
  Problem p;
  bool smooth_k;
  int rc = make_train_problem(shape, &p, &smooth_k);
  if (rc != SAGE_OK) return rc;
  const bool keep = (p.variant & SAGE_TRAIN_KEEP_QUANT) != 0;  // the forward's Q^, K^, V^ are there
  if (keep && !workspace) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_io(q, k, v, out)) != SAGE_OK) return rc;
  if (!dout || !dq || !dk || !dv || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return SAGE_ERR_INVALID_ARG;
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return SAGE_ERR_INVALID_ARG;
  if ((rc = device_check()) != SAGE_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  return with_workspace(sb_layout(p, true, nullptr), workspace, ws_bytes, s, [&](char* ws) {
    if (!keep && sb_prep_fwd(p, q, k, v, ws, true, smooth_k, s) != hipSuccess) return (int)SAGE_ERR_LAUNCH;
    if (sb_prep_bwd(p, out, dout, lse, ws, s) != hipSuccess) return (int)SAGE_ERR_LAUNCH;
    if (sb_backward(p, ws, smooth_k, v, dout, dq, dk, dv, s) != hipSuccess) return (int)SAGE_ERR_LAUNCH;
    return (int)SAGE_OK;
  });
}

void sage_attn_set_profile_events(void* start, void* stop) {
  if (start && stop) {
    t_prof_start = (hipEvent_t)start;
    t_prof_stop = (hipEvent_t)stop;
  } else {
    t_prof_start = t_prof_stop = nullptr;
  }
}

const char* sage_attn_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_INVALID_ARG: return "invalid argument";
    case SAGE_ERR_UNSUPPORTED: return "unsupported (head dim, bottom-right causal with N > M, or non-gfx950 device)";
    case SAGE_ERR_NO_MEMORY: return "workspace allocation failed or workspace too small";
    case SAGE_ERR_LAUNCH: return "kernel launch failed";
    case SAGE_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

int sage_attn_version(void) { return 100; }

}  // extern "C"
