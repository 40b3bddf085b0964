// sage_probe.hip -- probes of the gfx950 instructions the attention kernels rely on (a
// measurement library beside libsage_attn.so, not part of its C ABI).
//
// What the kernels assume, and what each probe lets a test check:
//   * the FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit scales) adds
//     its C operand at full FP32 precision, while its internal sum of the 64 products of one
//     step keeps fewer bits -- the analog of the accumulator the "SageAttention2 Technical
//     Report" summary finds on its GPUs (3.4 "Two-Level Accumulation"), and the reason the
//     kernels accumulate O through the C operand;
//   * the INT8 MFMA (v_mfma_i32_32x32x32_i8) sums exactly;
//   * the E4M3 conversion (v_cvt_pk_fp8_f32) rounds to nearest even, and the kernels' clamp to
//     +-448 before it gives the saturating E4M3 of the pages' "FP8 Quantization for P~V";
//   * the unsigned-byte conversion (v_cvt_pk_u8_f32) that packs SageBwd's INT8 P codes rounds to
//     nearest even;
//   * the matrix-core rates behind the roofline (INT8, FP8, and block-scaled FP4);
//   * the HBM rates behind the preprocessing's floor: streaming reads and writes, and a buffer
//     read again after its first read (the statistics and quantization passes both read K and V).
// Every kernel runs a bounded amount of work on buffers sized by the caller; the entry points
// only enqueue work on `stream` and return a hipError_t value (0 = success).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// One wave: d = A B + C on the FP8 MFMA; lane l supplies its 32 A bytes, 32 B bytes and 16 C
// values (the instruction's operand registers, whatever the element mapping).
__global__ __launch_bounds__(64) void mfma_f8_once(const v8i* a, const v8i* b, const v16f* c, v16f* d) {
  const int l = threadIdx.x;
  d[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], c[l], 0, 0, 0, 0, 0, 0);
}

// One wave: d = A B + C on the INT8 MFMA (16 A bytes, 16 B bytes, 16 C values per lane).
__global__ __launch_bounds__(64) void mfma_i8_once(const v4i* a, const v4i* b, const v16i* c, v16i* d) {
  const int l = threadIdx.x;
  d[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[l], b[l], c[l], 0, 0, 0);
}

// E4M3 code of the FP32 value with bit pattern start + i, as the kernels form it: clamped to
// +-448 (a NaN stays NaN), then v_cvt_pk_fp8_f32 (round to nearest even).
__global__ __launch_bounds__(256) void cvt_e4m3_range(uint32_t start, uint32_t count, uint8_t* out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= count) return;
  const float x = __uint_as_float(start + i);
  const float c = fminf(fmaxf(x, -448.0f), 448.0f);
  const float y = (x == x) ? c : x;
  out[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xff);
}

// out[i] = the byte v_cvt_pk_u8_f32 makes of the FP32 value with bits start + i (i < count).
__global__ __launch_bounds__(256) void cvt_u8_range(uint32_t start, uint32_t count, uint8_t* out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= count) return;
  out[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_u8_f32(__uint_as_float(start + i), 0, 0) & 0xff);
}

// Matrix-core rate: every wave runs four independent accumulator chains of `iters` MFMAs each
// (enough independent work to keep one SIMD's matrix core busy), then folds them into one
// value per lane so that nothing is optimised away.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate(int iters, float* sink) {
  const int seed = (int)(threadIdx.x * 2654435761u);
  float s = 0.0f;
  if constexpr (KIND == 0) {
    const v4i a = {seed, seed ^ 0x5a5a5a5a, seed + 7, seed - 3};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; i++) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c3, 0, 0, 0);
    }
    for (int r = 0; r < 16; r++) s += (float)(c0[r] ^ c1[r] ^ c2[r] ^ c3[r]);
  } else {
    // E4M3 codes with exponents near 1 (0x38 = 1.0), so the chains stay finite
    const int w = 0x38383838 | (seed & 0x03030303);
    const v8i a = {w, w, w, w, w, w, w, w};
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; i++) {
      if constexpr (KIND == 1) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c1, 0, 0, 0, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c3, 0, 0, 0, 0, 0, 0);
      } else {  // E2M1 operands (format 4) with unit E8M0 scales (127)
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c0, 4, 4, 0, 127, 0, 127);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c1, 4, 4, 0, 127, 0, 127);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 4, 4, 0, 127, 0, 127);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c3, 4, 4, 0, 127, 0, 127);
      }
    }
    for (int r = 0; r < 16; r++) s += c0[r] + c1[r] + c2[r] + c3[r];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// VALU rate: every lane runs 8 independent chains of `iters` steps of one instruction kind:
//   0 v_fma_f32, 1 v_exp_f32, 2 v_cvt_pk_fp8_f32, 3 v_cvt_scalef32_pk_fp4_f32, 4 v_cvt_f32_i32
//   (with the v_cvt_i32_f32 and v_add_u32 that feed it back: 24 instructions per step),
//   5 v_exp_f32 and v_fma_f32 interleaved (8 of each per step: whether the two kinds overlap
//   or add up).
template <int KIND>
__global__ __launch_bounds__(256) void valu_rate(int iters, float seed, float* sink) {
  float x[8];
  uint32_t w[8];
  int n[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    x[k] = seed * (float)(threadIdx.x + k);
    w[k] = threadIdx.x + k;
    n[k] = (int)threadIdx.x + k;
  }
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; k++) y[k] = x[k] + 1.0f;
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      if constexpr (KIND == 0) {
        x[k] = fmaf(x[k], seed, 0.5f);
      } else if constexpr (KIND == 1) {
        x[k] = __builtin_amdgcn_exp2f(x[k]);
      } else if constexpr (KIND == 2) {
        w[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[k], x[k], (int)w[k], false);
      } else if constexpr (KIND == 3) {
        w[k] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[k], x[k], x[k], 1.0f, 0);
      } else if constexpr (KIND == 4) {
        x[k] = (float)n[k];
        n[k] = (int)x[k] + 1;
      } else {
        x[k] = __builtin_amdgcn_exp2f(x[k]);
        y[k] = fmaf(y[k], seed, 0.5f);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; k++) s += x[k] + y[k] + (float)w[k] + (float)n[k];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// Streams n16 16-byte pieces of buf over a grid-stride loop: kind 0 reads them (the sum reaches
// sink only if it is NaN, so the loads stay and nothing is written for finite data), kind 1
// writes them.
__global__ __launch_bounds__(256) void stream_rw(int kind, float4* buf, size_t n16, float* sink) {
  const size_t step = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (kind == 0) {
    float s = 0.0f;
    for (; i < n16; i += step) {
      const float4 v = buf[i];
      s += v.x + v.y + v.z + v.w;
    }
    if (s != s) sink[0] = s;
  } else {
    const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (; i < n16; i += step) buf[i] = z;
  }
}

}  // namespace

extern "C" {

// d = A B + C on the FP8 MFMA, one wave.  a, b: 64 x 32 bytes (E4M3 codes); c, d: 64 x 16 floats.
int sage_probe_mfma_f8(const void* a, const void* b, const float* c, float* d, void* stream) {
  hipLaunchKernelGGL(mfma_f8_once, dim3(1), dim3(64), 0, (hipStream_t)stream, (const v8i*)a, (const v8i*)b,
                     (const v16f*)c, (v16f*)d);
  return (int)hipGetLastError();
}

// d = A B + C on the INT8 MFMA, one wave.  a, b: 64 x 16 bytes (INT8); c, d: 64 x 16 int32.
int sage_probe_mfma_i8(const void* a, const void* b, const int* c, int* d, void* stream) {
  hipLaunchKernelGGL(mfma_i8_once, dim3(1), dim3(64), 0, (hipStream_t)stream, (const v4i*)a, (const v4i*)b,
                     (const v16i*)c, (v16i*)d);
  return (int)hipGetLastError();
}

// out[i] = E4M3 code of the FP32 value with bits start + i (i < count; start + count <= 2^32),
// through the clamp and conversion the kernels use.  out: count bytes.
int sage_probe_cvt_e4m3(unsigned start, unsigned count, unsigned char* out, void* stream) {
  if (count == 0 || (unsigned long long)start + count > (1ull << 32)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(cvt_e4m3_range, dim3((count + 255) / 256), dim3(256), 0, (hipStream_t)stream, start, count, out);
  return (int)hipGetLastError();
}

// out[i] = v_cvt_pk_u8_f32's byte of the FP32 value with bits start + i (i < count; start + count
// <= 2^32).  out: count bytes.
int sage_probe_cvt_u8(unsigned start, unsigned count, unsigned char* out, void* stream) {
  if (count == 0 || (unsigned long long)start + count > (1ull << 32)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(cvt_u8_range, dim3((count + 255) / 256), dim3(256), 0, (hipStream_t)stream, start, count, out);
  return (int)hipGetLastError();
}

// MFMA rate kernel: kind 0 INT8 32x32x32, 1 FP8 32x32x64, 2 FP4 32x32x64 (block-scaled);
// blocks work-groups of 4 waves, each wave 4 x iters MFMAs.  sink: blocks x 256 floats.
int sage_probe_mfma_rate(int kind, int blocks, int iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || kind < 0 || kind > 2) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL(mfma_rate<0>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else if (kind == 1) hipLaunchKernelGGL(mfma_rate<1>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else hipLaunchKernelGGL(mfma_rate<2>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return (int)hipGetLastError();
}

// VALU rate kernel (see valu_rate): blocks work-groups of 256 lanes, each lane 8 x iters
// instructions of the kind (kind 5: 8 x iters of each of its two kinds).  sink: blocks x 256.
int sage_probe_valu_rate(int kind, int blocks, int iters, float seed, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || kind < 0 || kind > 5) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(valu_rate<0>, dim3(blocks), dim3(256), 0, s, iters, seed, sink); break;
    case 1: hipLaunchKernelGGL(valu_rate<1>, dim3(blocks), dim3(256), 0, s, iters, seed, sink); break;
    case 2: hipLaunchKernelGGL(valu_rate<2>, dim3(blocks), dim3(256), 0, s, iters, seed, sink); break;
    case 3: hipLaunchKernelGGL(valu_rate<3>, dim3(blocks), dim3(256), 0, s, iters, seed, sink); break;
    case 4: hipLaunchKernelGGL(valu_rate<4>, dim3(blocks), dim3(256), 0, s, iters, seed, sink); break;
    default: hipLaunchKernelGGL(valu_rate<5>, dim3(blocks), dim3(256), 0, s, iters, seed, sink); break;
  }
  return (int)hipGetLastError();
}

// Reads (kind 0) or writes zeros to (kind 1) the first `bytes` of buf (a multiple of 16) with
// 8192 work-groups of 256 lanes.  sink: one float, written only if the data read sums to NaN.
int sage_probe_stream(int kind, void* buf, unsigned long long bytes, float* sink, void* stream) {
  if (kind < 0 || kind > 1 || bytes == 0 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_rw, dim3(8192), dim3(256), 0, (hipStream_t)stream, kind, (float4*)buf,
                     (size_t)(bytes / 16), sink);
  return (int)hipGetLastError();
}

}  // extern "C"
