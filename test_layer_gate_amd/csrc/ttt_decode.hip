// gfx950 kernels of the decode step: one token per sequence goes through
// the layer. Its contractions are matrix-vector products whose cost is
// reading the weights and the state once, so they are written for HBM
// bandwidth (16-byte coalesced loads, fp32 accumulation), not for MFMA.
//
// Method sources: "论文精读：In-Place Test-Time Training" reading notes —
// "In-Place 设计" (gated MLP); iplexlaw explainer of In-Place Test-Time
// Training, §3 (a chunk's outputs use the state from before its update) and
// §6 (chunk-boundary padding of the target).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_device.h"
#include "ttt_launch.h"

namespace tttk {
namespace {

constexpr int kDecThreads = 256;   // 4 waves
constexpr int kDecMaxB = 8;        // sequences per pass of the gate/up product

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Eight consecutive values at p (bf16, or fp32 rounded to bf16 as the
// prefill rounds its fp32 inputs), widened to fp32.
template <bool F32>
__device__ __forceinline__ void load8_bf16(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (F32) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 a = q[0], b = q[1];
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf16_f32(bf16_rne(x[e]));
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const u16*>(p) + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
}

// Gated activation of one token per sequence: for row j of W_g and W_u
// (one wave per row), z[b][j] = SiLU(h_b . Wg[j]) * (h_b . Wu[j]). z goes to
// zb (bf16, the apply's operand) and, as fp16, to column `col` of the
// chunk's Z^T (sb<256> rows j, zt_cols columns) for the chunk's update:
// the same roundings as the prefill's Z and Z^T. The threads of the first
// blocks also copy the token's X0 rows (as bf16) into row `col` of the
// chunk's X0 buffer [B][chunk][d].
template <bool ACT_F32, bool W_F32>
__global__ __launch_bounds__(kDecThreads) void decode_gate_up_kernel(
    const void* __restrict__ h, const void* __restrict__ x0, const void* __restrict__ Wg,
    const void* __restrict__ Wu, int B, int d, int f, u16* __restrict__ zb,
    u16* __restrict__ zt, int64_t zt_bstride, int zt_cols, u16* __restrict__ x0c, int chunk,
    int col) {
  const int64_t gid = (int64_t)blockIdx.x * kDecThreads + threadIdx.x;
  if (gid < (int64_t)B * d / 8) {
    const int b = (int)(gid / (d / 8)), c = (int)(gid % (d / 8)) * 8;
    float v[8];
    load8_bf16<ACT_F32>(x0, (int64_t)b * d + c, v);
    *reinterpret_cast<uint4*>(x0c + ((int64_t)b * chunk + col) * d + c) =
        make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                   pack_bf16(v[6], v[7]));
  }
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kDecThreads / 64) + (threadIdx.x >> 6);
  if (j >= f) return;  // uniform per wave
  for (int b0 = 0; b0 < B; b0 += kDecMaxB) {
    const int nb = min(kDecMaxB, B - b0);
    float g[kDecMaxB], u[kDecMaxB];
#pragma unroll
    for (int b = 0; b < kDecMaxB; ++b) g[b] = u[b] = 0.f;
    for (int c = lane * 8; c < d; c += 64 * 8) {
      float wg[8], wu[8];
      load8_bf16<W_F32>(Wg, (int64_t)j * d + c, wg);
      load8_bf16<W_F32>(Wu, (int64_t)j * d + c, wu);
#pragma unroll
      for (int b = 0; b < kDecMaxB; ++b) {
        if (b < nb) {
          float hv[8];
          load8_bf16<ACT_F32>(h, (int64_t)(b0 + b) * d + c, hv);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            g[b] = fmaf(hv[e], wg[e], g[b]);
            u[b] = fmaf(hv[e], wu[e], u[b]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kDecMaxB; ++b) {
      if (b < nb) {
        const float gs = wave_sum(g[b]), us = wave_sum(u[b]);
        if (lane == 0) {
          const float z = silu(gs) * us;
          zb[(int64_t)(b0 + b) * f + j] = bf16_rne(z);
          zt[(int64_t)(b0 + b) * zt_bstride + sb_offset<kZtSlab>(j, col, zt_cols)] = f16_rne(z);
        }
      }
    }
  }
}

// The apply of one token per sequence against its own bf16 state copy S_b
// (sb<256>, rows c = d_model index, columns j = d_ff index):
// part[b][s][c] = sum over split s of the d_ff columns of z[b][j] * S_b[c][j].
// A workgroup takes 32 rows and one split; its 4 waves share the split's
// 16-column groups, each wave reading one 1 KB block of the slab per group
// (32 rows x 16 columns), four groups at a time so that four loads are in
// flight, and the waves' sums meet in LDS.
constexpr int kApplySplit = 8;

__global__ __launch_bounds__(kDecThreads) void decode_apply_kernel(
    const u16* __restrict__ zb, const u16* __restrict__ S, int64_t s_bstride, int d, int f,
    float* __restrict__ part) {
  __shared__ float red[4][32];
  const int rg = blockIdx.x % (d / 32), rest = blockIdx.x / (d / 32);
  const int split = rest % kApplySplit, b = rest / kApplySplit;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = rg * 32 + (lane & 31), half = lane >> 5;
  const int groups = f / 16, per = (groups + kApplySplit - 1) / kApplySplit;
  const int g0 = split * per, g1 = min(groups, g0 + per);
  const u16* Sb = S + (int64_t)b * s_bstride;
  const u16* zr = zb + (int64_t)b * f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = g0 + w; q0 < g1; q0 += 16) {
    float sv[4][8], zv[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = min(q0 + 4 * u, g1 - 1);  // in bounds; a repeat adds nothing (below)
      const int k = q * 16 + half * 8;
      load8_bf16<false>(Sb, sb_offset<kSnapSlab>(row, k, f), sv[u]);
      load8_bf16<false>(zr, k, zv[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q0 + 4 * u < g1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u] = fmaf(zv[u][e], sv[u][e], acc[u]);
      }
  }
  float tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  tot += __shfl_xor(tot, 32);  // the two halves of the 16 columns
  if (half == 0) red[w][lane] = tot;
  __syncthreads();
  if (threadIdx.x < 32) {
    const float s = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] +
                    red[3][threadIdx.x];
    part[((int64_t)b * kApplySplit + split) * d + rg * 32 + threadIdx.x] = s;
  }
}

// o[b][c] = sum of the splits' partial sums, in split order.
template <bool OUT_F32>
__global__ __launch_bounds__(kDecThreads) void decode_apply_sum_kernel(
    const float* __restrict__ part, void* __restrict__ o, int B, int d) {
  const int64_t i = (int64_t)blockIdx.x * kDecThreads + threadIdx.x;
  if (i >= (int64_t)B * d) return;
  const int64_t b = i / d, c = i % d;
  float s = 0.f;
#pragma unroll
  for (int sp = 0; sp < kApplySplit; ++sp) s += part[(b * kApplySplit + sp) * d + c];
  if constexpr (OUT_F32)
    static_cast<float*>(o)[i] = s;
  else
    static_cast<u16*>(o)[i] = bf16_rne(s);
}

int ceil_div_i(int64_t a, int b) { return (int)((a + b - 1) / b); }

}  // namespace

int64_t decode_apply_part_floats(int B, int d) { return (int64_t)B * kApplySplit * d; }

hipError_t launch_decode_gate_up(const void* h, const void* x0, bool act_f32, const void* Wg,
                                 const void* Wu, bool w_f32, int B, int d, int f, uint16_t* zb,
                                 uint16_t* zt, int64_t zt_bstride, int zt_cols, uint16_t* x0c,
                                 int chunk, int col, hipStream_t s) {
  // One wave per row of W_g / W_u, and enough threads for the X0 copy.
  const int grid = max(ceil_div_i(f, kDecThreads / 64), ceil_div_i((int64_t)B * d / 8, kDecThreads));
#define TTT_DEC_GU(A, W)                                                                  \
  decode_gate_up_kernel<A, W><<<grid, kDecThreads, 0, s>>>(h, x0, Wg, Wu, B, d, f, zb, zt, \
                                                            zt_bstride, zt_cols, x0c, chunk, col)
  if (act_f32 && w_f32)
    TTT_DEC_GU(true, true);
  else if (act_f32)
    TTT_DEC_GU(true, false);
  else if (w_f32)
    TTT_DEC_GU(false, true);
  else
    TTT_DEC_GU(false, false);
#undef TTT_DEC_GU
  return hipGetLastError();
}

hipError_t launch_decode_apply(const uint16_t* zb, const uint16_t* S, int64_t s_bstride, int B,
                               int d, int f, float* part, void* o, bool out_f32, hipStream_t s) {
  decode_apply_kernel<<<B * kApplySplit * (d / 32), kDecThreads, 0, s>>>(zb, S, s_bstride, d, f,
                                                                         part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = ceil_div_i((int64_t)B * d, kDecThreads);
  if (out_f32)
    decode_apply_sum_kernel<true><<<grid, kDecThreads, 0, s>>>(part, o, B, d);
  else
    decode_apply_sum_kernel<false><<<grid, kDecThreads, 0, s>>>(part, o, B, d);
  return hipGetLastError();
}

}  // namespace tttk
