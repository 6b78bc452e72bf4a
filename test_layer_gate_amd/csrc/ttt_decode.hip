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
constexpr int kDecMaxB = 4;        // sequences per pass of the gate/up product
constexpr int kDecRows = 2;        // W_g / W_u rows per wave of the gate/up product

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
// (two rows per wave, so that all of a Qwen3-4B-sized d_ff's waves are
// resident at once), z[b][j] = SiLU(h_b . Wg[j]) * (h_b . Wu[j]). z goes to
// zb (bf16, the apply's operand) and to row `col` of the chunk's fp32 rows
// zc [B][chunk][f], and, as fp16, to column `col` of the chunk's Z^T
// (sb<256> rows j, zt_cols columns) for the chunk's update: the same
// roundings as the prefill's Z and Z^T. The largest |z| goes to the Z group
// of the chunk's range buffer (zrange), which the chunk's close checks. The
// threads of the first blocks also copy the token's X0 rows (as bf16) into
// row `col` of the chunk's X0 buffer [B][chunk][d].
template <bool ACT_F32, bool W_F32>
__global__ __launch_bounds__(kDecThreads) void decode_gate_up_kernel(
    const void* __restrict__ h, const void* __restrict__ x0, const void* __restrict__ Wg,
    const void* __restrict__ Wu, int B, int d, int f, u16* __restrict__ zb,
    float* __restrict__ zc, u16* __restrict__ zt, int64_t zt_bstride, int zt_cols,
    u16* __restrict__ x0c, int chunk, int col, uint32_t* __restrict__ zrange) {
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
  const int j0 = (blockIdx.x * (kDecThreads / 64) + (threadIdx.x >> 6)) * kDecRows;
  float zmax = 0.0f;
  // Waves past the last row skip the product but still reach the range
  // note's barrier (one atomic per workgroup: per wave, the notes queued on
  // the range words).
  for (int b0 = 0; j0 < f && b0 < B; b0 += kDecMaxB) {
    const int nb = min(kDecMaxB, B - b0);
    float g[kDecRows][kDecMaxB], u[kDecRows][kDecMaxB];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r)
#pragma unroll
      for (int b = 0; b < kDecMaxB; ++b) g[r][b] = u[r][b] = 0.f;
    for (int c = lane * 8; c < d; c += 64 * 8) {
      float wg[kDecRows][8], wu[kDecRows][8];
#pragma unroll
      for (int r = 0; r < kDecRows; ++r) {
        const int j = min(j0 + r, f - 1);  // in bounds; a clamped row is not stored (below)
        load8_bf16<W_F32>(Wg, (int64_t)j * d + c, wg[r]);
        load8_bf16<W_F32>(Wu, (int64_t)j * d + c, wu[r]);
      }
#pragma unroll
      for (int b = 0; b < kDecMaxB; ++b) {
        if (b < nb) {
          float hv[8];
          load8_bf16<ACT_F32>(h, (int64_t)(b0 + b) * d + c, hv);
#pragma unroll
          for (int r = 0; r < kDecRows; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              g[r][b] = fmaf(hv[e], wg[r][e], g[r][b]);
              u[r][b] = fmaf(hv[e], wu[r][e], u[r][b]);
            }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
      const int j = j0 + r;
#pragma unroll
      for (int b = 0; b < kDecMaxB; ++b) {
        if (b < nb) {
          const float gs = wave_sum(g[r][b]), us = wave_sum(u[r][b]);
          if (lane == 0 && j < f) {
            const float z = silu(gs) * us;
            zmax = fmaxf(zmax, fabsf(z));
            zb[(int64_t)(b0 + b) * f + j] = bf16_rne(z);
            zc[((int64_t)(b0 + b) * chunk + col) * f + j] = z;
            zt[(int64_t)(b0 + b) * zt_bstride + sb_offset<kZtSlab>(j, col, zt_cols)] =
                f16_rne(z);
          }
        }
      }
    }
  }
  range_note_block<kDecThreads>(zrange + kRangeZ * kRangeSlots, zmax);
}

// At a chunk's close: if the chunk's largest |z| is out of the fp16 range,
// Z^T again from the chunk's fp32 rows, times 2^qz (the update divides it
// out), as the prefill's repaired Z^T; otherwise returns at once.
__global__ __launch_bounds__(kDecThreads) void decode_zt_repair_kernel(
    const float* __restrict__ zc, u16* __restrict__ zt, int B, int f, int chunk, int64_t zt_bstride,
    int zt_cols, const uint32_t* __restrict__ zrange) {
  const int q = range_exp(range_read(zrange + kRangeZ * kRangeSlots));
  if (q == 0) return;
  const float sc = exp2i(q);
  const int64_t n = (int64_t)B * chunk * f;
  for (int64_t i = (int64_t)blockIdx.x * kDecThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kDecThreads) {
    const int j = (int)(i % f);
    const int64_t bc = i / f;
    const int col = (int)(bc % chunk), b = (int)(bc / chunk);
    zt[(int64_t)b * zt_bstride + sb_offset<kZtSlab>(j, col, zt_cols)] = f16_rne(zc[i] * sc);
  }
}

// The apply of one token per sequence against its own bf16 state copy S_b
// (sb<256>, rows c = d_model index, columns j = d_ff index): o[b][c] = sum
// over j of z[b][j] * S_b[c][j]. A workgroup takes 8 rows and all of d_ff;
// its 8 waves take every 8th 64-column block, lane (r, s) reading row r's
// columns 8s .. 8s + 7 of a block (the 8 rows' 8 columns are one 128-byte
// piece of the slab), four blocks in flight. The lanes of a row, then the
// waves (in LDS), add up in a fixed order.
constexpr int kApRows = 8, kApWaves = 8, kApInFlight = 4;

template <bool OUT_F32>
__global__ __launch_bounds__(64 * kApWaves) void decode_apply_kernel(
    const u16* __restrict__ zb, const u16* __restrict__ S, int64_t s_bstride, int d, int f,
    void* __restrict__ o) {
  __shared__ float red[kApWaves][kApRows];
  const int rg = blockIdx.x % (d / kApRows), b = blockIdx.x / (d / kApRows);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 7, sg = lane >> 3;
  const int row = rg * kApRows + r;
  const u16* Sb = S + (int64_t)b * s_bstride;
  const u16* zr = zb + (int64_t)b * f;
  const int nblk = f / 64;
  float acc[kApInFlight] = {};
  for (int q0 = w; q0 < nblk; q0 += kApWaves * kApInFlight) {
    float sv[kApInFlight][8], zv[kApInFlight][8];
#pragma unroll
    for (int u = 0; u < kApInFlight; ++u) {
      const int q = min(q0 + u * kApWaves, nblk - 1);  // in bounds; a repeat adds nothing
      const int k = q * 64 + sg * 8;
      load8_bf16<false>(Sb, sb_offset<kSnapSlab>(row, k, f), sv[u]);
      load8_bf16<false>(zr, k, zv[u]);
    }
#pragma unroll
    for (int u = 0; u < kApInFlight; ++u)
      if (q0 + u * kApWaves < nblk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u] = fmaf(zv[u][e], sv[u][e], acc[u]);
      }
  }
  float tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  tot += __shfl_xor(tot, 8);   // the 8 column groups of a row
  tot += __shfl_xor(tot, 16);
  tot += __shfl_xor(tot, 32);
  if (sg == 0) red[w][r] = tot;
  __syncthreads();
  if (threadIdx.x < kApRows) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < kApWaves; ++v) s += red[v][threadIdx.x];
    const int64_t i = (int64_t)b * d + rg * kApRows + threadIdx.x;
    if constexpr (OUT_F32)
      static_cast<float*>(o)[i] = s;
    else
      static_cast<u16*>(o)[i] = bf16_rne(s);
  }
}

int ceil_div_i(int64_t a, int b) { return (int)((a + b - 1) / b); }

}  // namespace

hipError_t launch_decode_gate_up(const void* h, const void* x0, bool act_f32, const void* Wg,
                                 const void* Wu, bool w_f32, int B, int d, int f, uint16_t* zb,
                                 float* zc, uint16_t* zt, int64_t zt_bstride, int zt_cols,
                                 uint16_t* x0c, int chunk, int col, uint32_t* zrange,
                                 hipStream_t s) {
  // kDecRows rows of W_g / W_u per wave, and enough threads for the X0 copy.
  const int grid = max(ceil_div_i(f, kDecThreads / 64 * kDecRows),
                       ceil_div_i((int64_t)B * d / 8, kDecThreads));
#define TTT_DEC_GU(A, W)                                                                     \
  decode_gate_up_kernel<A, W><<<grid, kDecThreads, 0, s>>>(h, x0, Wg, Wu, B, d, f, zb, zc, zt, \
                                                            zt_bstride, zt_cols, x0c, chunk, col, \
                                                            zrange)
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

hipError_t launch_decode_zt_repair(const float* zc, uint16_t* zt, int B, int f, int chunk,
                                  int64_t zt_bstride, int zt_cols, const uint32_t* zrange,
                                  hipStream_t s) {
  const int grid = min(ceil_div_i((int64_t)B * chunk * f, kDecThreads), 1024);
  decode_zt_repair_kernel<<<grid, kDecThreads, 0, s>>>(zc, zt, B, f, chunk, zt_bstride, zt_cols,
                                                       zrange);
  return hipGetLastError();
}

hipError_t launch_decode_apply(const uint16_t* zb, const uint16_t* S, int64_t s_bstride, int B,
                               int d, int f, void* o, bool out_f32, hipStream_t s) {
  const int grid = B * (d / kApRows);
  if (out_f32)
    decode_apply_kernel<true><<<grid, 64 * kApWaves, 0, s>>>(zb, S, s_bstride, d, f, o);
  else
    decode_apply_kernel<false><<<grid, 64 * kApWaves, 0, s>>>(zb, S, s_bstride, d, f, o);
  return hipGetLastError();
}

}  // namespace tttk
