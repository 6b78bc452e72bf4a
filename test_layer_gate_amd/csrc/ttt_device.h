// Device-side numeric helpers shared by the kernel files: rounding to the
// 16-bit formats the layer stores, and the SiLU of the gated activation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_launch.h"

namespace tttk {

typedef uint16_t u16;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN stays a NaN): gfx950's
// v_cvt_pk_bf16_f32, one instruction for two values.
__device__ __forceinline__ u16 bf16_rne(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

__device__ __forceinline__ float bf16_f32(u16 h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ u16 f16_rne(float x) {
  return __builtin_bit_cast(u16, (_Float16)x);  // v_cvt_f16_f32: round to nearest even
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Two values in one v_cvt_pk_f16_f32 (the same rounding as two scalar
// conversions, checked on every non-NaN fp32 pattern).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}

// The backward's SiLU factor words (one per token and d_ff feature) in the
// order a 32x32 MFMA accumulator holds them: each 32-token x 32-feature
// block is 4 KB, laid out [q][feature][lane half][4 tokens], so the 16 bytes
// of register group q of every lane sit side by side and one wave's access
// is one contiguous 1 KB span. Blocks run over the features, then the
// tokens (T_pad of them), then the batch. t32 and j32: the block's first
// token and feature (multiples of 32); lane: the lane index (feature j32 +
// lane % 32, tokens t32 + 8 q + 4 (lane / 32) .. + 3). Returns the word
// offset of the lane's 16 bytes.
__device__ __forceinline__ int64_t sa_frag_offset(int b, int t32, int j32, int q, int lane,
                                                  const Dims& g) {
  const int64_t blk = ((int64_t)b * (g.T_pad >> 5) + (t32 >> 5)) * (g.f >> 5) + (j32 >> 5);
  return blk * 1024 + q * 256 + (lane & 31) * 8 + (lane >> 5) * 4;
}

// SiLU(x) = x * sigmoid(x), with the hardware reciprocal (1 ulp) in place of
// a full division.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---------------------------------------------------------------- ranges
// Several operands are kept as fp16 copies (10 mantissa bits; normal values
// from 2^-14 to 65504): the update's Z^T and V^T, and the target's conv(X0)
// and W_target^T. Each producer notes the largest |value| it writes in
// kRangeSlots words of a range group (the bits of the non-negative float,
// combined with atomicMax, spread over the words so that atomics on one
// address stay rare). When that maximum leaves [2^-10, 65504], the operand
// is written again times 2^q, with q bringing the maximum into [2^14, 2^15),
// and its consumers divide 2^q back out. Powers of two make both exact.
// (kRangeSlots, the group indices and the exponent limits: ttt_launch.h)

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// Notes m (this lane's largest |value|, >= 0) in a range group; every lane
// of the wave must call it. One atomicMax per wave (for kernels with long
// workgroups, where these are rare).
__device__ __forceinline__ void range_note(uint32_t* group, float m) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) {
    const uint32_t slot = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) % kRangeSlots;
    atomicMax(group + slot, __float_as_uint(m));
  }
}

// The same with one atomicMax per workgroup of NT threads (for short
// workgroups, whose per-wave atomics would queue on the words); every thread
// of the workgroup must call it.
template <int NT>
__device__ __forceinline__ void range_note_block(uint32_t* group, float m) {
  __shared__ float red[NT / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
    atomicMax(group + blockIdx.x % kRangeSlots, __float_as_uint(m));
  }
}

// The largest |value| noted in a range group; every lane of the wave must
// call it.
__device__ __forceinline__ float range_read(const uint32_t* group) {
  static_assert(kRangeSlots % 64 == 0, "range words per lane");
  uint32_t v = 0u;
#pragma unroll
  for (int i = 0; i < kRangeSlots / 64; ++i) v = max(v, group[i * 64 + (threadIdx.x & 63)]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return __uint_as_float(v);
}

// The exponent q that brings a maximum a into [2^14, 2^15), or 0 when a is
// already in [2^-10, 65504], or is 0, NaN or infinite (those propagate).
__device__ __forceinline__ int range_exp(float a) {
  if (!(a > 0.0f) || !(a < __builtin_huge_valf())) return 0;
  if (a >= 0x1p-10f && a <= 65504.0f) return 0;
  int e = 0;
  (void)frexpf(a, &e);  // a = m 2^e, m in [0.5, 1): floor(log2 a) = e - 1
  return min(max(15 - e, -kRangeMaxExp), kRangeMaxExp);
}

// The exponents of the update's operands: Z^T holds Z 2^qz and V^T holds
// eta 2^(p + qv) V, so the state is carried as 2^(p + qv + qz) W. qv is held
// so that p + qv + qz stays within +-kStateMaxExp (p is eta's, within +-60,
// and qz within +-40, so qv = 0 is always allowed).
__device__ __forceinline__ void update_exps(const uint32_t* range, int p, int* qv, int* qz) {
  *qz = range_exp(range_read(range + kRangeZ * kRangeSlots));
  const int v = range_exp(range_read(range + kRangeV * kRangeSlots));
  *qv = min(max(v, -kStateMaxExp - p - *qz), kStateMaxExp - p - *qz);
}

__device__ __forceinline__ float exp2i(int q) { return ldexpf(1.0f, q); }

}  // namespace tttk
