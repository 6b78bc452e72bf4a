// Device-side numeric helpers shared by the kernel files: rounding to the
// 16-bit formats the layer stores, and the SiLU of the gated activation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

typedef uint16_t u16;

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ u16 bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

__device__ __forceinline__ float bf16_f32(u16 h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ u16 f16_rne(float x) {
  return __builtin_bit_cast(u16, (_Float16)x);  // v_cvt_f16_f32: round to nearest even
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)bf16_rne(lo) | ((uint32_t)bf16_rne(hi) << 16);
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return (uint32_t)f16_rne(lo) | ((uint32_t)f16_rne(hi) << 16);
}

// SiLU(x) = x * sigmoid(x), with the hardware reciprocal (1 ulp) in place of
// a full division.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace tttk
