// attn_device.hpp -- device helpers shared by the fused attention kernels (gfx950).
//
// LDS-DMA staging issued from inline asm, the lane-pair reductions of the transposed score
// accumulator (lanes l and l ^ 32 hold the same query), base-2 exponent, and the epilogue
// store of four output channels.
#pragma once

#include <cfloat>
#include <type_traits>

#include "sage_common.hpp"

namespace sage {
namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXCD = 8;  // work-groups are dealt to the 8 XCDs round-robin

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ object, in an SGPR.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((uintptr_t)(const lds_void*)p));
}

// Global -> LDS DMA of one 16-byte (or 4-byte) chunk per lane into LDS bytes
// [lds + 16 lane, +16) (resp. [lds + 4 lane, +4)).  Issued from asm so that the compiler's
// wait-count tracking does not treat every later LDS read as dependent on it; completion is
// awaited explicitly (vmcnt) before the barrier that publishes the tile.
__device__ __forceinline__ void dma16(uint32_t lds, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(gbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(gbase) : "memory", "m0");
}

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

// Compile-time loop: f(std::integral_constant<int, i>) for i in [I, N) (MFMA operand
// selectors must be immediates).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Four consecutive output channels of one row: FP32, fp16 or bf16 (RNE).
template <int OUT>  // 0 bf16, 1 fp16, 2 fp32
__device__ __forceinline__ void store_out4(void* out, size_t idx, const float (&o)[4]) {
  if (OUT == 2) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = make_float4(o[0], o[1], o[2], o[3]);
  } else if (OUT == 1) {
    uint2 u;
    u.x = f32_to_fp16_bits(o[0]) | (f32_to_fp16_bits(o[1]) << 16);
    u.y = f32_to_fp16_bits(o[2]) | (f32_to_fp16_bits(o[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = u;
  } else {
    uint2 u;
    u.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
    u.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = u;
  }
}

}  // namespace attn
}  // namespace sage
