// gfx950 (CDNA4) kernels of the In-Place TTT gated-MLP prefill.
//
// The dense contractions (gate/up projection, target projection, the
// per-chunk fast-weight update and the apply) run on one bf16 MFMA GEMM core:
// C[M][N] = sum_k A[m][k] * B[n][k], both operands K-contiguous in HBM,
// staged through LDS in 64-wide K slices with two LDS buffers, and
// multiplied with v_mfma_f32_32x32x16_bf16 (fp32 accumulation). A workgroup
// has 4 wave64s in a 2 x 2 grid; each wave owns (BM/2) x (BN/2) outputs.
// The depthwise conv, W_target transpose and fp32->bf16 casts are small
// bandwidth-bound kernels.
//
// Method sources: "论文精读：In-Place Test-Time Training" reading notes —
// "In-Place 设计" (gated MLP), "Chunk-Wise 更新机制" (update equation),
// "LM-Aligned 目标函数" (target equation); iplexlaw explainer of In-Place
// Test-Time Training, §3 (apply, then update) and §6 (exclusive prefix over
// chunk deltas).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_launch.h"

namespace tttk {
namespace {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // 4 wave64s
constexpr int kBK = 64;        // K elements per LDS stage (128 bytes per row)

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ u16 bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

__device__ __forceinline__ float bf16_f32(u16 h) {
  return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)bf16_rne(lo) | ((uint32_t)bf16_rne(hi) << 16);
}

__device__ __forceinline__ float silu(float x) {
  return x / (1.0f + __expf(-x));
}

// LDS tile of `rows` x 64 bf16, row stride 128 B. The eight 16-byte chunks of
// a row are XOR-permuted by (row ^ row >> 3) & 7 so that the 32 rows of an
// MFMA fragment read, and the eight rows of a cooperative store, fall on
// distinct banks.
__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * kBK + (((kc ^ row ^ (row >> 3)) & 7) << 3);
}

__device__ __forceinline__ bf16x8 frag(const u16* lds, int row, int kc) {
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const uint4*>(lds + lds_off(row, kc)));
}

// One 64-wide K slice of ROWS rows, moved HBM -> registers -> LDS by the
// whole workgroup, 16 bytes per thread per step. Rows at or past rows_valid
// read as zero.
template <int ROWS>
struct GTile {
  static constexpr int N = ROWS * 8 / kThreads;
  static_assert(N >= 1 && ROWS * 8 % kThreads == 0, "tile rows");
  uint4 v[N];
  __device__ __forceinline__ void load(const u16* __restrict__ base, int64_t ld,
                                       int rows_valid, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3;
      if (r < rows_valid)
        v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + (c & 7) * 8);
      else
        v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(u16* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<uint4*>(lds + lds_off(c >> 3, c & 7)) = v[i];
    }
  }
};

// Maps the linear workgroup id to (batch, tile_m, tile_n). Workgroups are
// handed to the 8 XCDs in turn, so ids are first renumbered so that each XCD
// runs one contiguous range of tiles; within a range, tiles go in groups of
// group_m rows of tiles, M fastest, so that the workgroups resident on one
// XCD share A and B slices through its L2.
struct TileIdx {
  int b, tm, tn;
};

__device__ __forceinline__ TileIdx tile_index(int tiles_m, int tiles_n, int group_m) {
  const int nblk = gridDim.x;
  int lin = blockIdx.x;
  const int xcd = lin & 7, idx = lin >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  lin = xcd * per + min(xcd, rem) + idx;
  const int per_batch = tiles_m * tiles_n;
  TileIdx t;
  t.b = lin / per_batch;
  lin -= t.b * per_batch;
  const int group = group_m * tiles_n;
  const int g = lin / group;
  const int first_m = g * group_m;
  const int gm = min(group_m, tiles_m - first_m);
  const int r = lin - g * group;
  t.tm = first_m + r % gm;
  t.tn = r / gm;
  return t;
}

struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// The GEMM core. acc[m][n] is the 32x32 MFMA tile (m, n) of this wave:
// output rows wm*BM/2 + m*32 + 8*(r/4) + 4*(lane/32) + r%4 for register r,
// output column wn*BN/2 + n*32 + lane%32 (for SPLITB see brow()).
// SPLITB: the B tile is BN/2 rows of B0 followed by BN/2 rows of B1 (the
// gate and up projections); wave wn then owns the same BN/4 columns of each,
// in acc[.][0, TN/2) (B0) and acc[.][TN/2, TN) (B1).
// hook(kt) runs before the MFMAs of K step kt, when acc holds steps < kt.
template <int BM, int BN, bool SPLITB, class Hook>
__device__ __forceinline__ void gemm_mainloop(
    const u16* __restrict__ A, int64_t lda, int a_valid,
    const u16* __restrict__ B0, const u16* __restrict__ B1, int64_t ldb,
    int b_valid, int nk, f32x16 (&acc)[BM / 64][BN / 64], u16* smem,
    const Hook& hook) {
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int STAGE = (BM + BN) * kBK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  if (nk <= 0) return;

  GTile<BM> ga;
  GTile<SPLITB ? BN / 2 : BN> gb0;
  GTile<SPLITB ? BN / 2 : 64> gb1;  // used only when SPLITB

  auto gload = [&](int kt) {
    const int64_t k = (int64_t)kt * kBK;
    ga.load(A + k, lda, a_valid, tid);
    gb0.load(B0 + k, ldb, b_valid, tid);
    if constexpr (SPLITB) gb1.load(B1 + k, ldb, b_valid, tid);
  };
  auto sstore = [&](int buf) {
    u16* s = smem + buf * STAGE;
    ga.store(s, tid);
    gb0.store(s + BM * kBK, tid);
    if constexpr (SPLITB) gb1.store(s + BM * kBK + (BN / 2) * kBK, tid);
  };
  auto brow = [&](int n) {
    if constexpr (SPLITB) {
      constexpr int H = TN / 2;
      return n < H ? wn * H * 32 + n * 32 : BN / 2 + wn * H * 32 + (n - H) * 32;
    } else {
      return wn * TN * 32 + n * 32;
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    hook(kt);
    const u16* sA = smem + cur * STAGE;
    const u16* sB = sA + BM * kBK;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int kc = 2 * s + (lane >> 5);
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int m = 0; m < TM; ++m) a[m] = frag(sA, wm * TM * 32 + m * 32 + (lane & 31), kc);
#pragma unroll
      for (int n = 0; n < TN; ++n) b[n] = frag(sB, brow(n) + (lane & 31), kc);
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
}

template <int TM, int TN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[TM][TN]) {
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n) acc[m][n] = f32x16{};
}

// ------------------------------------------------ gate/up + SiLU*mul (K1)
// M = tokens (256), N = 128 columns of Wg and the same 128 of Wu, K = d.
constexpr int K1_BM = 256, K1_BN = 256, K1_LDZ = K1_BN / 2 + 8;

__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wg,
    const u16* __restrict__ Wu, u16* __restrict__ Z, u16* __restrict__ ZT,
    int T, int T_pad, int d, int f, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) u16 smem[2 * (K1_BM + K1_BN) * kBK];
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
  const int t0 = ti.tm * K1_BM, j0 = ti.tn * (K1_BN / 2);
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_mainloop<K1_BM, K1_BN, true>(H + ((int64_t)ti.b * T + t0) * d, d, min(K1_BM, T - t0),
                                     Wg + (int64_t)j0 * d, Wu + (int64_t)j0 * d, d,
                                     min(K1_BN / 2, f - j0), d / kBK, acc, smem, NoHook{});
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  u16* sZ = smem;  // [256][K1_LDZ] staging for the token-major store
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tl = wm * 128 + m * 32 + 8 * q + 4 * (lane >> 5);
        const int jl = wn * 64 + n * 32 + (lane & 31);
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = silu(acc[m][n][4 * q + e]) * acc[m][n + 2][4 * q + e];
        const int t = t0 + tl, j = j0 + jl;
        if (ZT != nullptr && j < f)
          *reinterpret_cast<uint2*>(ZT + ((int64_t)ti.b * f + j) * T_pad + t) =
              make_uint2(pack2(z[0], z[1]), pack2(z[2], z[3]));
#pragma unroll
        for (int e = 0; e < 4; ++e) sZ[(tl + e) * K1_LDZ + jl] = bf16_rne(z[e]);
      }
  if (Z == nullptr) return;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = tid + i * kThreads;
    const int row = c >> 4, cc = c & 15;
    const int t = t0 + row, j = j0 + cc * 8;
    if (t < T && j < f)
      *reinterpret_cast<uint4*>(Z + ((int64_t)ti.b * T + t) * f + j) =
          *reinterpret_cast<const uint4*>(sZ + row * K1_LDZ + cc * 8);
  }
}

// ------------------------------------------------------ target GEMM (K2)
// M = tokens (256), N = output channels (256), K = d.
__global__ __launch_bounds__(kThreads) void target_kernel(
    const u16* __restrict__ Y, const u16* __restrict__ WtT, u16* __restrict__ VT,
    u16* __restrict__ Vtok, float scale, int T, int T_pad, int d, int tiles_m,
    int tiles_n) {
  __shared__ __attribute__((aligned(16))) u16 smem[2 * (256 + 256) * kBK];
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
  const int t0 = ti.tm * 256, c0 = ti.tn * 256;
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_mainloop<256, 256, false>(Y + ((int64_t)ti.b * T_pad + t0) * d, d, 256,
                                 WtT + (int64_t)c0 * d, nullptr, d, min(256, d - c0),
                                 d / kBK, acc, smem, NoHook{});
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + wm * 128 + m * 32 + 8 * q + 4 * (lane >> 5);
        const int c = c0 + wn * 128 + n * 32 + (lane & 31);
        if (c >= d) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[m][n][4 * q + e] * scale;
        if (VT != nullptr)
          *reinterpret_cast<uint2*>(VT + ((int64_t)ti.b * d + c) * T_pad + t) =
              make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
        if (Vtok != nullptr) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t + e < T) Vtok[((int64_t)ti.b * T + t + e) * d + c] = bf16_rne(v[e]);
        }
      }
}

// ------------------------------------------ fast-weight update (K3)
// M = d_ff (256), N = d_model (BN), K = tokens. acc starts at the state and
// absorbs (eta V)^T Z one 64-token step at a time; at every chunk start the
// state before that chunk is stored as a bf16 snapshot (exclusive prefix).
template <int BN, bool WINIT_F32>
__global__ __launch_bounds__(kThreads) void update_kernel(
    const u16* __restrict__ ZT, const u16* __restrict__ VT,
    const void* __restrict__ Winit, int64_t winit_bstride, u16* __restrict__ snap,
    int64_t snap_bstride, float* __restrict__ Wf, u16* __restrict__ shadow,
    int T_pad, int d, int f, int tok_begin, int nk, int steps_per_chunk,
    int tiles_m, int tiles_n) {
  constexpr int BM = 256, TM = BM / 64, TN = BN / 64;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * (BM + BN) * kBK];
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
  const int j0 = ti.tm * BM, c0 = ti.tn * BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int64_t df = (int64_t)d * f;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + wm * TM * 32 + m * 32 + 8 * q + 4 * (lane >> 5);
        const int c = c0 + wn * TN * 32 + n * 32 + (lane & 31);
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (c < d && j < f) {
          const int64_t o = ti.b * winit_bstride + (int64_t)c * f + j;
          if constexpr (WINIT_F32) {
            const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(Winit) + o);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const u16*>(Winit) + o);
            v[0] = __uint_as_float(x.x << 16);
            v[1] = __uint_as_float(x.x & 0xffff0000u);
            v[2] = __uint_as_float(x.y << 16);
            v[3] = __uint_as_float(x.y & 0xffff0000u);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[m][n][4 * q + e] = v[e];
      }

  auto store_bf16 = [&](u16* dst) {
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int n = 0; n < TN; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + wm * TM * 32 + m * 32 + 8 * q + 4 * (lane >> 5);
          const int c = c0 + wn * TN * 32 + n * 32 + (lane & 31);
          if (c < d && j < f)
            *reinterpret_cast<uint2*>(dst + (int64_t)c * f + j) =
                make_uint2(pack2(acc[m][n][4 * q], acc[m][n][4 * q + 1]),
                           pack2(acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]));
        }
  };

  u16* snap_b = snap ? snap + ti.b * snap_bstride : nullptr;
  auto hook = [&](int kt) {
    if (snap_b != nullptr && kt % steps_per_chunk == 0)
      store_bf16(snap_b + (int64_t)(kt / steps_per_chunk) * df);
  };
  gemm_mainloop<BM, BN, false>(ZT + ((int64_t)ti.b * f + j0) * T_pad + tok_begin, T_pad,
                               min(BM, f - j0),
                               VT + ((int64_t)ti.b * d + c0) * T_pad + tok_begin, nullptr,
                               T_pad, min(BN, d - c0), nk, acc, smem, hook);

  float* wf_b = Wf + ti.b * df;
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + wm * TM * 32 + m * 32 + 8 * q + 4 * (lane >> 5);
        const int c = c0 + wn * TN * 32 + n * 32 + (lane & 31);
        if (c < d && j < f)
          *reinterpret_cast<float4*>(wf_b + (int64_t)c * f + j) =
              make_float4(acc[m][n][4 * q], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                          acc[m][n][4 * q + 3]);
      }
  if (shadow != nullptr) store_bf16(shadow + ti.b * df);
}

// ------------------------------------------------------------ apply (K4)
// M = d_model (256), N = tokens (BN, which divides the chunk), K = d_ff.
// The tile's tokens all lie in one chunk i and read snapshot i.
template <int BN, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void apply_kernel(
    const u16* __restrict__ Z, const u16* __restrict__ snap, int64_t snap_bstride,
    int64_t snap_cstride, void* __restrict__ O, int T, int d, int f, int tok_begin,
    int chunk, int tiles_m, int tiles_n) {
  constexpr int BM = 256, TM = BM / 64, TN = BN / 64;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * (BM + BN) * kBK];
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
  const int c0 = ti.tm * BM, t0 = tok_begin + ti.tn * BN;
  const int i = t0 / chunk;
  f32x16 acc[TM][TN];
  zero_acc(acc);
  gemm_mainloop<BM, BN, false>(snap + ti.b * snap_bstride + i * snap_cstride + (int64_t)c0 * f,
                               f, min(BM, d - c0), Z + ((int64_t)ti.b * T + t0) * f, nullptr,
                               f, min(BN, T - t0), f / kBK, acc, smem, NoHook{});
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + wm * TM * 32 + m * 32 + 8 * q + 4 * (lane >> 5);
        const int t = t0 + wn * TN * 32 + n * 32 + (lane & 31);
        if (t >= T || c >= d) continue;
        const int64_t o = ((int64_t)ti.b * T + t) * d + c;
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(O) + o) =
              make_float4(acc[m][n][4 * q], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                          acc[m][n][4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<u16*>(O) + o) =
              make_uint2(pack2(acc[m][n][4 * q], acc[m][n][4 * q + 1]),
                         pack2(acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]));
        }
      }
}

// --------------------------------------------------- small kernels

__global__ __launch_bounds__(kThreads) void cast_kernel(const float* __restrict__ src,
                                                        u16* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    const float4 x = reinterpret_cast<const float4*>(src)[i];
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(pack2(x.x, x.y), pack2(x.z, x.w));
  }
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const void* __restrict__ src,
                                                             u16* __restrict__ dst, int rows,
                                                             int cols) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) {
      const int64_t o = (int64_t)r * cols + c;
      tile[i][tx] = F32 ? static_cast<const float*>(src)[o]
                        : bf16_f32(static_cast<const u16*>(src)[o]);
    }
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[(int64_t)c * rows + r] = bf16_rne(tile[tx][i]);
  }
}

template <bool TAPS_F32>
__global__ __launch_bounds__(kThreads) void conv_kernel(
    const u16* __restrict__ X0, const void* __restrict__ taps, u16* __restrict__ Y, int T,
    int T_pad, int d, int K, int chunk, int pad_chunk, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= total) return;
  const int d8 = d >> 3;
  const int c = (int)(gid % d8) * 8;
  const int64_t bt = gid / d8;
  const int t = (int)(bt % T_pad);
  const int b = (int)(bt / T_pad);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int end = pad_chunk ? min(T, (t / chunk + 1) * chunk) : T;
  for (int k = 0; k < K && t + k < end; ++k) {
    const uint4 xv = *reinterpret_cast<const uint4*>(X0 + ((int64_t)b * T + t + k) * d + c);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    float tp[8];
    if constexpr (TAPS_F32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(taps) + (int64_t)k * d + c);
      const float4 a = p[0], bq = p[1];
      tp[0] = a.x; tp[1] = a.y; tp[2] = a.z; tp[3] = a.w;
      tp[4] = bq.x; tp[5] = bq.y; tp[6] = bq.z; tp[7] = bq.w;
    } else {
      const uint4 tv = *reinterpret_cast<const uint4*>(static_cast<const u16*>(taps) + (int64_t)k * d + c);
      const uint32_t tw[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tp[2 * e] = __uint_as_float(tw[e] << 16);
        tp[2 * e + 1] = __uint_as_float(tw[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(tp[2 * e], __uint_as_float(xw[e] << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(tp[2 * e + 1], __uint_as_float(xw[e] & 0xffff0000u), acc[2 * e + 1]);
    }
  }
  *reinterpret_cast<uint4*>(Y + ((int64_t)b * T_pad + t) * d + c) =
      make_uint4(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]), pack2(acc[4], acc[5]),
                 pack2(acc[6], acc[7]));
}

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

// ------------------------------------------------------------ launchers

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  const int blocks = (int)std::min<int64_t>((n4 + kThreads - 1) / kThreads, 65536);
  if (blocks > 0) cast_kernel<<<blocks, kThreads, 0, s>>>(src, dst, n4);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, bool src_f32, uint16_t* dst, int rows, int cols,
                            hipStream_t s) {
  dim3 grid(ceil_div(cols, 64), ceil_div(rows, 64));
  if (src_f32)
    transpose_kernel<true><<<grid, kThreads, 0, s>>>(src, dst, rows, cols);
  else
    transpose_kernel<false><<<grid, kThreads, 0, s>>>(src, dst, rows, cols);
  return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* X0, const void* taps, bool taps_f32, uint16_t* Y, int B,
                       int T, int T_pad, int d, int K, int chunk, bool pad_chunk, hipStream_t s) {
  const int64_t total = (int64_t)B * T_pad * (d / 8);
  const int blocks = ceil_div(total, kThreads);
  if (taps_f32)
    conv_kernel<true><<<blocks, kThreads, 0, s>>>(X0, taps, Y, T, T_pad, d, K, chunk,
                                                  pad_chunk ? 1 : 0, total);
  else
    conv_kernel<false><<<blocks, kThreads, 0, s>>>(X0, taps, Y, T, T_pad, d, K, chunk,
                                                   pad_chunk ? 1 : 0, total);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* H, const uint16_t* Wg, const uint16_t* Wu, uint16_t* Z,
                          uint16_t* ZT, int B, int T, int T_pad, int d, int f, hipStream_t s) {
  const int tiles_m = T_pad / K1_BM, tiles_n = ceil_div(f, K1_BN / 2);
  gate_up_kernel<<<tiles_m * tiles_n * B, kThreads, 0, s>>>(H, Wg, Wu, Z, ZT, T, T_pad, d, f,
                                                            tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_target(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                         float scale, int B, int T, int T_pad, int d, hipStream_t s) {
  const int tiles_m = T_pad / 256, tiles_n = ceil_div(d, 256);
  target_kernel<<<tiles_m * tiles_n * B, kThreads, 0, s>>>(Y, WtT, VT, Vtok, scale, T, T_pad, d,
                                                           tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_update(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                         bool winit_f32, int64_t winit_bstride, uint16_t* snap,
                         int64_t snap_bstride, float* Wf, uint16_t* shadow, int B, int T_pad,
                         int d, int f, int tok_begin, int nk, int steps_per_chunk,
                         hipStream_t s) {
  constexpr int BN = 128;
  const int tiles_m = ceil_div(f, 256), tiles_n = ceil_div(d, BN);
  const int grid = tiles_m * tiles_n * B;
  if (winit_f32)
    update_kernel<BN, true><<<grid, kThreads, 0, s>>>(ZT, VT, Winit, winit_bstride, snap,
                                                     snap_bstride, Wf, shadow, T_pad, d, f,
                                                     tok_begin, nk, steps_per_chunk, tiles_m,
                                                     tiles_n);
  else
    update_kernel<BN, false><<<grid, kThreads, 0, s>>>(ZT, VT, Winit, winit_bstride, snap,
                                                      snap_bstride, Wf, shadow, T_pad, d, f,
                                                      tok_begin, nk, steps_per_chunk, tiles_m,
                                                      tiles_n);
  return hipGetLastError();
}

template <int BN>
static void apply_dispatch(const uint16_t* Z, const uint16_t* snap, int64_t sb, int64_t sc,
                           void* O, bool out_f32, int B, int T, int d, int f, int tok_begin,
                           int tok_end, int chunk, hipStream_t s) {
  const int tiles_m = ceil_div(d, 256), tiles_n = ceil_div(tok_end - tok_begin, BN);
  const int grid = tiles_m * tiles_n * B;
  if (out_f32)
    apply_kernel<BN, true><<<grid, kThreads, 0, s>>>(Z, snap, sb, sc, O, T, d, f, tok_begin,
                                                     chunk, tiles_m, tiles_n);
  else
    apply_kernel<BN, false><<<grid, kThreads, 0, s>>>(Z, snap, sb, sc, O, T, d, f, tok_begin,
                                                      chunk, tiles_m, tiles_n);
}

hipError_t launch_apply(const uint16_t* Z, const uint16_t* snap, int64_t snap_bstride,
                        int64_t snap_cstride, void* O, bool out_f32, int B, int T, int d, int f,
                        int tok_begin, int tok_end, int chunk, hipStream_t s) {
  // The token tile must not straddle a chunk: take the largest of 256, 128,
  // 64 that divides the chunk (the chunk is a multiple of 64).
  if (chunk % 256 == 0)
    apply_dispatch<256>(Z, snap, snap_bstride, snap_cstride, O, out_f32, B, T, d, f, tok_begin,
                        tok_end, chunk, s);
  else if (chunk % 128 == 0)
    apply_dispatch<128>(Z, snap, snap_bstride, snap_cstride, O, out_f32, B, T, d, f, tok_begin,
                        tok_end, chunk, s);
  else
    apply_dispatch<64>(Z, snap, snap_bstride, snap_cstride, O, out_f32, B, T, d, f, tok_begin,
                       tok_end, chunk, s);
  return hipGetLastError();
}

}  // namespace tttk
