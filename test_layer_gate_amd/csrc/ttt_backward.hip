// gfx950 kernels of the layer's backward pass: the gradients of the prefill
// with respect to H, X0, W_g, W_u, W_down0, the conv taps and W_target, for
// upstream gradients dO and dW_final.
//
// With Gbar = dL/dW_{i+1} (the state gradient after chunk i), the reverse of
// the chunk recurrence gives, per chunk i:
//   dZ_i = dO_i W_i + eta V_i Gbar,  dV_i = eta Z_i Gbar^T,
//   dL/dW_i = Gbar + dO_i^T Z_i,     dW_down0 = dL/dW_0,
// then dY = dV W_target^T, dW_target = Y^T dV, the conv's transpose for dX0
// and the taps, and the gated MLP's: dG = dZ U phi'(G), dU = dZ phi(G),
// dH = dG W_g + dU W_u, dW_g = dG^T H, dW_u = dU^T H.
// ("论文精读：In-Place Test-Time Training" reading notes, "In-Place 设计" and
// "Chunk-Wise 更新机制"; iplexlaw explainer of In-Place Test-Time Training,
// §3 and §6 for the recurrence, §2 and §7.1 for the continual training that
// needs its gradient.)
//
// Every operand here is bf16 with fp32 accumulation. The kernels in this
// file: the chunked GEMMs whose second operand is one chunk's state (dZ,
// with the SiLU's backward in its epilogue, and dV), a plain GEMM with fp32
// output (dY, dH), and the layout kernels and the conv's backward. The scans
// over tokens (the states W_i, the state gradients, dW_g, dW_u, dW_target)
// run on the prefill's update kernel (ttt_kernels.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ttt_device.h"
#include "ttt_gemm.h"
#include "ttt_launch.h"

namespace tttk {
namespace {

constexpr int kBwThreads = 256;

// f(integral_constant<int, I>) for I = B .. E - 1, each a separate inlined
// instance, so that indices derived from I are constants (an epilogue loop
// the compiler leaves rolled would index the accumulators dynamically, which
// moves them to scratch memory).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(const F& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ------------------------------------------------ chunked activation GEMM
// C[t][n] = sum_k A[t][k] S(i)[n][k] for the tokens t of one chunk i: A
// token-major bf16 ([B][T][lda], K contiguous). M = BM tokens (a divisor of
// the chunk), N = 256. dV: S(i) is chunk i's bf16 state gradient matrix
// (sb<256>, rows n, K columns) at S + b * sbs + i * scs. dZ: two
// contractions side by side in one pipeline over K = 2d, [dO | eta V]
// against S(i) = [W_i^T | Gbar^T]; the chunk's state W_i (at S + b * sbs +
// i * scs) and state gradient Gbar (at G + b * g_sbs + i * g_scs) are
// sb<256>(d x f) matrices, read transposed (kSlabT) as they are.
constexpr int KA_NW = 8, KA_BN = 256, KA_BK = 64;
template <int BM>
struct ActCfg {
  static constexpr int WGM = BM == 64 ? 1 : 2;
  static constexpr int NSTA = BM == 256 ? 2 : 3, NSTB = 3;
};

enum { kActDZ = 0, kActDV = 1 };

struct ActArgs {
  const u16* A;
  int64_t lda;
  const u16* S;
  int64_t sbs, scs;
  const u16* G;
  int64_t g_sbs, g_scs;
  int K;
  int N, chunk, n_chunks;
  float scale;
  // dZ: the SiLU's derivative factors (low half phi(G), high half U phi'(G),
  // bf16) in accumulator-fragment order (sa_frag_offset), dG and dU
  // token-major ([B][T][ld_gu]: dG of feature c in column 2c, dU in 2c + 1)
  // and as slabs sb<256>(N x B T_pad).
  const uint32_t* sa;
  u16* dgu;
  int64_t ld_gu;
  u16 *dgt, *dut;
  // dV: scale * C token-major ([B][T][ld_out]) and as a slab sb<256>(N x B T_pad)
  u16* out_tok;
  int64_t ld_out;
  u16* out_t;
};

struct PlainSink {
  u16* m;
  __device__ __forceinline__ void operator()(int64_t off, const uint4& v, bool ok) const {
    if (ok) *reinterpret_cast<uint4*>(m + off) = v;
  }
};

template <int BM, int MODE>
__device__ __forceinline__ void act_gemm(const ActArgs& a, const Dims& g, int tiles_m,
                                         int tiles_n) {
  using C = ActCfg<BM>;
  using L = Layout<BM, KA_BN, C::WGM, KA_NW>;
  TTT_GEMM_LDS_AB(lds, BM, KA_BN, KA_BK, C::NSTA, C::NSTB)
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
  const int t0 = ti.tm * BM, n0 = ti.tn * KA_BN;
  // Tiles past the sequence (t0 >= T) still run, on rows that read as
  // zero, so that their slab columns are written as zeros.
  const int i = min(t0 / a.chunk, a.n_chunks - 1);
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  {
    const Operand ao = row_major<KA_BK>(a.A + ((int64_t)ti.b * g.T + t0) * a.lda, a.lda, g.T - t0);
    if constexpr (MODE == kActDZ) {
      // The tile's columns n0 .. n0 + 255 of both (d x f) matrices start in
      // slab n0 / 64 of their first slab row.
      const int64_t col0 = (int64_t)(n0 >> 6) * (256 * 64);
      const uint32_t bytes = (uint32_t)((sb_elems<256>(g.d, g.f) - col0) * 2);
      const OperandT so{a.S + ti.b * a.sbs + i * a.scs + col0,
                        a.G + ti.b * a.g_sbs + i * a.g_scs + col0, bytes, bytes, g.d / KA_BK,
                        (int64_t)g.f};
      gemm_core_ab<KA_NW, BM, KA_BN, C::WGM, KA_BK, C::NSTA, C::NSTB, Bf16Mma, false, kRowMajor,
                   kSlabT>(ao, so, so, a.K / KA_BK, &acc[0][0], lds, NoHook{});
    } else {
      const Operand so = slab_blocked<256>(a.S + ti.b * a.sbs + i * a.scs, a.K, n0, 0);
      gemm_core_ab<KA_NW, BM, KA_BN, C::WGM, KA_BK, C::NSTA, C::NSTB, Bf16Mma, false, kRowMajor,
                   kSlab>(ao, so, so, a.K / KA_BK, &acc[0][0], lds, NoHook{});
    }
  }
  const int N = a.N;
  const int64_t kt = (int64_t)g.B * g.T_pad;
  // dV's token-major output goes through LDS (free once the core has
  // drained), so that its stores are whole 16-byte row segments: every wave
  // writes its values as bf16 rows of a BM x 256 staging tile, then all
  // threads copy the tile's rows out.
  constexpr int LDG = KA_BN + 8;  // staging row stride (elements)
  static_assert(BM * LDG <= (C::NSTA * BM + C::NSTB * KA_BN) * KA_BK, "staging fits");
  auto stage = [&](int m, int n, const f32x16& v) {
    const Frag<L> fr(true);
    const int cl = fr.col(n);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u16* sr = lds + fr.row(m, q) * LDG + cl;
#pragma unroll
      for (int e = 0; e < 4; ++e) sr[e * LDG] = bf16_rne(v[4 * q + e]);
    }
  };
  auto flush = [&](u16* dst, int64_t ld) {
    __syncthreads();
    constexpr int SEGS = BM * (KA_BN / 8);
    static_assert(SEGS % (64 * KA_NW) == 0, "whole rounds");
#pragma unroll
    for (int i = 0; i < SEGS / (64 * KA_NW); ++i) {
      const int sgi = threadIdx.x + i * (64 * KA_NW);
      const int row = sgi / (KA_BN / 8), cc = (sgi % (KA_BN / 8)) * 8;
      const int t = t0 + row, c = n0 + cc;
      if (t < g.T && c < N)
        *reinterpret_cast<uint4*>(dst + ((int64_t)ti.b * g.T + t) * ld + c) =
            *reinterpret_cast<const uint4*>(lds + row * LDG + cc);
    }
  };
  if constexpr (MODE == kActDZ) {
    // The factor words of two tiles at a time (a lane's four consecutive
    // tokens are 16 bytes), then dG and dU of both tiles: the stores of a
    // tile come before the next loads, and vmcnt completes in issue order,
    // so each load batch waits for the stores ahead of it (one wait per two
    // tiles; staging dG and dU through LDS instead took 7% longer). Each
    // (dG, dU) pair goes token-major as one 4-byte store through a buffer
    // resource based at the tile's first row and sized to its rows inside
    // the sequence (rows past it are dropped), and dG and dU as slabs.
    const int rows_ok = max(0, min(BM, g.T - t0));
    const __amdgpu_buffer_rsrc_t gu_r = __builtin_amdgcn_make_buffer_rsrc(
        a.dgu + ((int64_t)ti.b * g.T + t0) * a.ld_gu, 0, (int)(rows_ok * a.ld_gu * 2),
        kRsrcWord3);
    const int drop_gu = (int)(rows_ok * a.ld_gu * 2);
    static_assert((L::TM * L::TN) % 2 == 0, "tiles pair up");
    static_for<0, L::TM * L::TN / 2>([&](auto P) __attribute__((always_inline)) {
      constexpr int I0 = 2 * decltype(P)::value;
      // Coordinates (and the addresses made from them) per pair, through an
      // opaque copy of the thread index: computed once for all tiles, they
      // would be held across the whole epilogue.
      const Frag<L> fr(true);
      uint4 w4[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int m = (I0 + k) / L::TN, n = (I0 + k) % L::TN;
        const int col = n0 + fr.col(n);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w4[k][q] = make_uint4(0u, 0u, 0u, 0u);
          if (col < N)
            w4[k][q] = *reinterpret_cast<const uint4*>(
                a.sa + sa_frag_offset(ti.b, t0 + fr.wm * L::TM * 32 + m * 32,
                                      col - (fr.lane & 31), q, fr.lane, g));
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int m = (I0 + k) / L::TN, n = (I0 + k) % L::TN;
        const int col = n0 + fr.col(n);
        const bool cok = col < N;
        const int64_t kb = (int64_t)ti.b * g.T_pad + t0 + fr.wm * L::TM * 32 + m * 32;
        f32x16 vg, vu;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w[4] = {w4[k][q].x, w4[k][q].y, w4[k][q].z, w4[k][q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vg[4 * q + e] = acc[m][n][4 * q + e] * __uint_as_float(w[e] & 0xffff0000u);  // U phi'(G)
            vu[4 * q + e] = acc[m][n][4 * q + e] * __uint_as_float(w[e] << 16);          // phi(G)
          }
        }
        store_tile_sb<256>(kt, col, kb, vg, CvtBf16{1.0f}, cok, PlainSink{a.dgt});
        store_tile_sb<256>(kt, col, kb, vu, CvtBf16{1.0f}, cok, PlainSink{a.dut});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tr = fr.row(m, r / 4) + r % 4;  // row within the tile
          __builtin_amdgcn_raw_buffer_store_b32(
              pack_bf16(vg[r], vu[r]), gu_r, cok ? (int)((tr * a.ld_gu + 2 * col) * 2) : drop_gu,
              0, 0);
        }
      }
    });
  } else {
    static_for<0, L::TM * L::TN>([&](auto I) __attribute__((always_inline)) {
      constexpr int m = decltype(I)::value / L::TN, n = decltype(I)::value % L::TN;
      const Frag<L> fr(true);
      const int col = n0 + fr.col(n);
      f32x16 v;
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = acc[m][n][r] * a.scale;
      const int64_t kb = (int64_t)ti.b * g.T_pad + t0 + fr.wm * L::TM * 32 + m * 32;
      store_tile_sb<256>(kt, col, kb, v, CvtBf16{1.0f}, col < N, PlainSink{a.out_t});
      stage(m, n, v);
    });
    flush(a.out_tok, a.ld_out);
  }
}

// dZ and dV under kernel names of their own, for traces.
template <int BM>
__global__ __launch_bounds__(64 * KA_NW) void dz_gemm_kernel(ActArgs a, Dims g, int tiles_m,
                                                             int tiles_n) {
  act_gemm<BM, kActDZ>(a, g, tiles_m, tiles_n);
}
template <int BM>
__global__ __launch_bounds__(64 * KA_NW) void dv_gemm_kernel(ActArgs a, Dims g, int tiles_m,
                                                             int tiles_n) {
  act_gemm<BM, kActDV>(a, g, tiles_m, tiles_n);
}

// ------------------------------------------------------- plain NT GEMM
// out[b][t][n] = sum_k A[b][t][k] Bm[n][k] (fp32, ldo), bf16 operands: A
// token-major [B][T][lda], Bm [N][ldb]; K a multiple of 64.
constexpr int KN_NW = 8, KN_BM = 256, KN_BN = 256, KN_WGM = 2, KN_BK = 64, KN_NSTA = 2,
              KN_NSTB = 3;

__global__ __launch_bounds__(64 * KN_NW) void nt_gemm_kernel(const u16* __restrict__ A,
                                                             int64_t lda,
                                                             const u16* __restrict__ Bm,
                                                             int64_t ldb, int N, int K,
                                                             float* __restrict__ out,
                                                             int64_t ldo, Dims g, int tiles_m,
                                                             int tiles_n) {
  using L = Layout<KN_BM, KN_BN, KN_WGM, KN_NW>;
  TTT_GEMM_LDS_AB(lds, KN_BM, KN_BN, KN_BK, KN_NSTA, KN_NSTB)
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
  const int t0 = ti.tm * KN_BM, n0 = ti.tn * KN_BN;
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  const int nk = K / KN_BK;
  const Operand bo = row_major<KN_BK>(Bm + (int64_t)n0 * ldb, ldb, N - n0);
  gemm_core_ab<KN_NW, KN_BM, KN_BN, KN_WGM, KN_BK, KN_NSTA, KN_NSTB, Bf16Mma, false, kRowMajor,
               kRowMajor>(row_major<KN_BK>(A + ((int64_t)ti.b * g.T + t0) * lda, lda, g.T - t0),
                          bo, bo, nk, &acc[0][0], lds, NoHook{}, k_rotation<4>(ti.tm, ti.tn, nk));
  const Frag<L> fr;
#pragma unroll
  for (int m = 0; m < L::TM; ++m)
#pragma unroll
    for (int n = 0; n < L::TN; ++n) {
      const int col = n0 + fr.col(n);
      if (col >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = t0 + fr.row(m, q) + e;
          if (t < g.T) out[((int64_t)ti.b * g.T + t) * ldo + col] = acc[m][n][4 * q + e];
        }
    }
}

// ------------------------------------------------------------ layouts
// dst = src^T as bf16 slabs: src token-major [B][T][lds] (bf16 or fp32) with
// D features, dst sb<256>(D x K) where K = T_pad per sequence (dst + b *
// sb_elems(D, T_pad), column t) or, with flat, K = B T_pad (column
// b T_pad + t). Tokens t >= T are written as zero. One thread: 8 tokens x 8
// features.
template <bool F32>
__global__ __launch_bounds__(kBwThreads) void to_slab_kernel(const void* __restrict__ src,
                                                             int64_t lds_, u16* __restrict__ dst,
                                                             int B, int T, int T_pad, int D,
                                                             int flat) {
  const int64_t gid = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
  const int d8 = D / 8, tg = T_pad / 8;
  if (gid >= (int64_t)B * tg * d8) return;
  const int c = (int)(gid % d8) * 8;
  const int64_t rest = gid / d8;
  const int t = (int)(rest % tg) * 8, b = (int)(rest / tg);
  float v[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int tr = t + r;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[r][e] = 0.0f;
    if (tr < T) {
      const int64_t o = ((int64_t)b * T + tr) * lds_ + c;
      if constexpr (F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + o);
        const float4 x = p[0], y = p[1];
        v[r][0] = x.x; v[r][1] = x.y; v[r][2] = x.z; v[r][3] = x.w;
        v[r][4] = y.x; v[r][5] = y.y; v[r][6] = y.z; v[r][7] = y.w;
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const u16*>(src) + o);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[r][2 * e] = __uint_as_float(w[e] << 16);
          v[r][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      }
    }
  }
  const int64_t K = flat ? (int64_t)B * T_pad : T_pad;
  u16* db = flat ? dst : dst + (int64_t)b * sb_elems<256>(D, T_pad);
  const int64_t k = flat ? (int64_t)b * T_pad + t : t;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint4*>(db + sb_offset<256>(c + e, k, K)) =
        make_uint4(pack_bf16(v[0][e], v[1][e]), pack_bf16(v[2][e], v[3][e]),
                   pack_bf16(v[4][e], v[5][e]), pack_bf16(v[6][e], v[7][e]));
}

// dst[c * ld_dst + r * step] = bf16(src[r][c]) for a rows x cols matrix
// (bf16 or fp32).
template <bool F32>
__global__ __launch_bounds__(kBwThreads) void transpose_bf16_kernel(const void* __restrict__ src,
                                                                    u16* __restrict__ dst,
                                                                    int rows, int cols,
                                                                    int64_t ld_dst, int step) {
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
    if (c < cols && r < rows) dst[(int64_t)c * ld_dst + (int64_t)r * step] = bf16_rne(tile[tx][i]);
  }
}

// dst[r][c] = bf16(src[r][c]) with row strides ld_src and ld_dst, 8
// columns per thread.
template <bool F32>
__global__ __launch_bounds__(kBwThreads) void rows_bf16_kernel(const void* __restrict__ src,
                                                               int64_t ld_src,
                                                               u16* __restrict__ dst,
                                                               int64_t ld_dst, int64_t rows,
                                                               int cols) {
  const int64_t gid = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
  const int c8 = cols / 8;
  if (gid >= rows * c8) return;
  const int64_t r = gid / c8;
  const int c = (int)(gid % c8) * 8;
  uint4 v;
  if constexpr (F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + r * ld_src + c);
    const float4 x = p[0], y = p[1];
    v = make_uint4(pack_bf16(x.x, x.y), pack_bf16(x.z, x.w), pack_bf16(y.x, y.y),
                   pack_bf16(y.z, y.w));
  } else {
    v = *reinterpret_cast<const uint4*>(static_cast<const u16*>(src) + r * ld_src + c);
  }
  *reinterpret_cast<uint4*>(dst + r * ld_dst + c) = v;
}

// ------------------------------------------------------ conv backward
// The conv read X0[t + k] for output t while t + k was before t's bound (the
// sequence end T, or with pad_chunk the end of t's chunk). Its transpose:
// dX0[s] = sum_k taps[k] dY[s - k] over the same reads, 8 rows s x 8
// channels per thread with a window of dY rows sliding up one row per tap;
// dY is fp32 [B][T][d], dX0 fp32 [B][T][d].
__device__ __forceinline__ int conv_bound(int t, int T, int chunk, int pad_chunk) {
  return pad_chunk ? min(T, (t / chunk + 1) * chunk) : T;
}

__device__ __forceinline__ void load_row8_f32(const float* p, float (&v)[8]) {
  const float4 x = reinterpret_cast<const float4*>(p)[0], y = reinterpret_cast<const float4*>(p)[1];
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

template <bool TAPS_F32>
__device__ __forceinline__ void load_taps8(const void* taps, int64_t o, float (&tp)[8]) {
  if constexpr (TAPS_F32) {
    load_row8_f32(static_cast<const float*>(taps) + o, tp);
  } else {
    const uint4 tv = *reinterpret_cast<const uint4*>(static_cast<const u16*>(taps) + o);
    const uint32_t tw[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tp[2 * e] = __uint_as_float(tw[e] << 16);
      tp[2 * e + 1] = __uint_as_float(tw[e] & 0xffff0000u);
    }
  }
}

template <bool TAPS_F32>
__global__ __launch_bounds__(kBwThreads) void conv_bwd_x_kernel(const float* __restrict__ dY,
                                                                const void* __restrict__ taps,
                                                                float* __restrict__ dX0, int B,
                                                                int T, int d, int K, int chunk,
                                                                int pad_chunk) {
  const int64_t gid = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
  const int d8 = d / 8, tg = (T + 7) / 8;
  if (gid >= (int64_t)B * tg * d8) return;
  const int c = (int)(gid % d8) * 8;
  const int64_t rest = gid / d8;
  const int s = (int)(rest % tg) * 8, b = (int)(rest / tg);
  const float* yb = dY + (int64_t)b * T * d + c;
  float acc[8][8] = {};
  float win[8][8];  // win[r] = dY[s + r - k]
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (s + r < T) load_row8_f32(yb + (int64_t)(s + r) * d, win[r]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) win[r][e] = 0.0f;
  }
  for (int k = 0; k < K; ++k) {
    float tp[8];
    load_taps8<TAPS_F32>(taps, (int64_t)k * d + c, tp);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int t = s + r - k;  // the output that read row s + r with tap k
      if (t >= 0 && s + r < T && s + r < conv_bound(t, T, chunk, pad_chunk)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(tp[e], win[r][e], acc[r][e]);
      }
    }
#pragma unroll
    for (int r = 7; r > 0; --r)
#pragma unroll
      for (int e = 0; e < 8; ++e) win[r][e] = win[r - 1][e];
    const int nr = s - k - 1;
    if (nr >= 0) load_row8_f32(yb + (int64_t)nr * d, win[0]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) win[0][e] = 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (s + r < T) {
      float4* o = reinterpret_cast<float4*>(dX0 + ((int64_t)b * T + s + r) * d + c);
      o[0] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
      o[1] = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
    }
}

// Partial tap gradients: part[b * nblk + blk][k][c] = sum over the outputs t
// of token block blk (kTapRows tokens) of dY[t][c] X0[t + k][c], over the
// conv's reads, for taps k0 .. k0 + 7 (a window of X0 rows slides down).
constexpr int kTapRows = 256;

__global__ __launch_bounds__(kBwThreads) void conv_bwd_taps_kernel(
    const float* __restrict__ dY, const u16* __restrict__ X0, float* __restrict__ part, int B,
    int T, int d, int K, int chunk, int pad_chunk, int nblk) {
  const int64_t gid = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
  const int d8 = d / 8, kg = (K + 7) / 8;
  if (gid >= (int64_t)B * nblk * kg * d8) return;
  const int c = (int)(gid % d8) * 8;
  int64_t rest = gid / d8;
  const int k0 = (int)(rest % kg) * 8;
  rest /= kg;
  const int blk = (int)(rest % nblk), b = (int)(rest / nblk);
  const float* yb = dY + (int64_t)b * T * d + c;
  const u16* xb = X0 + (int64_t)b * T * d + c;
  auto x_row = [&](int r, float (&v)[8]) {
    if (r < T) {
      const uint4 x = *reinterpret_cast<const uint4*>(xb + (int64_t)r * d);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
  };
  float acc[8][8] = {};
  float win[8][8];  // win[j] = X0[t + k0 + j]
  const int ta = blk * kTapRows, tb = min(T, ta + kTapRows);
#pragma unroll
  for (int j = 0; j < 8; ++j) x_row(ta + k0 + j, win[j]);
  for (int t = ta; t < tb; ++t) {
    float y[8];
    load_row8_f32(yb + (int64_t)t * d, y);
    const int bound = conv_bound(t, T, chunk, pad_chunk);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < K && t + k0 + j < bound) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(y[e], win[j][e], acc[j][e]);
      }
#pragma unroll
    for (int j = 0; j < 7; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) win[j][e] = win[j + 1][e];
    x_row(t + k0 + 8, win[7]);
  }
  float* pb = part + ((int64_t)b * nblk + blk) * K * d;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (k0 + j < K) {
      float4* o = reinterpret_cast<float4*>(pb + (int64_t)(k0 + j) * d + c);
      o[0] = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      o[1] = make_float4(acc[j][4], acc[j][5], acc[j][6], acc[j][7]);
    }
}

// out[i] = sum over p < n_parts of in[p * stride + i], in order.
__global__ __launch_bounds__(kBwThreads) void sum_parts_kernel(const float* __restrict__ in,
                                                               int64_t stride, int n_parts,
                                                               float* __restrict__ out,
                                                               int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int p = 0; p < n_parts; ++p) s += in[(int64_t)p * stride + i];
  out[i] = s;
}

int grid_of(int64_t threads) { return (int)((threads + kBwThreads - 1) / kBwThreads); }

}  // namespace

// ------------------------------------------------------------ launchers

hipError_t launch_act_gemm_dz(const uint16_t* dOV, int64_t lda, const uint16_t* W, int64_t w_sbs,
                              int64_t w_scs, const uint16_t* Gs, int64_t g_sbs, int64_t g_scs,
                              int d, int f, int chunk, int n_chunks, const uint32_t* sa,
                              uint16_t* dgu, int64_t ld_gu, uint16_t* dgt, uint16_t* dut,
                              const Dims& g, hipStream_t s) {
  // The transposed reads address a state matrix with 32-bit offsets, the
  // top bit reserved.
  if (d != g.d || f != g.f || sb_elems<256>(d, f) * 2 >= (int64_t)1 << 31)
    return hipErrorInvalidValue;
  ActArgs a{};
  a.A = dOV;
  a.lda = lda;
  a.S = W;
  a.sbs = w_sbs;
  a.scs = w_scs;
  a.G = Gs;
  a.g_sbs = g_sbs;
  a.g_scs = g_scs;
  a.K = 2 * d;
  a.N = f;
  a.chunk = chunk;
  a.n_chunks = n_chunks;
  a.scale = 1.0f;
  a.sa = sa;
  a.dgu = dgu;
  a.ld_gu = ld_gu;
  a.dgt = dgt;
  a.dut = dut;
  const int bm = apply_tile_width(chunk);
  const int tiles_n = (f + KA_BN - 1) / KA_BN;
  if (bm == 256) {
    const int tiles_m = g.T_pad / 256;
    dz_gemm_kernel<256><<<tiles_m * tiles_n * g.B, 64 * KA_NW, 0, s>>>(a, g, tiles_m, tiles_n);
  } else {
    const int tiles_m = g.T_pad / 64;
    dz_gemm_kernel<64><<<tiles_m * tiles_n * g.B, 64 * KA_NW, 0, s>>>(a, g, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

hipError_t launch_act_gemm_dv(const uint16_t* Z, int64_t ldz, const uint16_t* G, int64_t sbs,
                              int64_t scs, int d, int f, int chunk, int n_chunks, float eta,
                              uint16_t* dv, int64_t ld_dv, uint16_t* dvt, const Dims& g,
                              hipStream_t s) {
  ActArgs a{};
  a.A = Z;
  a.lda = ldz;
  a.S = G;
  a.sbs = sbs;
  a.scs = scs;
  a.K = f;
  a.N = d;
  a.chunk = chunk;
  a.n_chunks = n_chunks;
  a.scale = eta;
  a.out_tok = dv;
  a.ld_out = ld_dv;
  a.out_t = dvt;
  const int bm = apply_tile_width(chunk);
  const int tiles_n = (d + KA_BN - 1) / KA_BN;
  if (bm == 256) {
    const int tiles_m = g.T_pad / 256;
    dv_gemm_kernel<256><<<tiles_m * tiles_n * g.B, 64 * KA_NW, 0, s>>>(a, g, tiles_m, tiles_n);
  } else {
    const int tiles_m = g.T_pad / 64;
    dv_gemm_kernel<64><<<tiles_m * tiles_n * g.B, 64 * KA_NW, 0, s>>>(a, g, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

hipError_t launch_nt_gemm(const uint16_t* A, int64_t lda, const uint16_t* Bm, int64_t ldb, int N,
                          int K, float* out, int64_t ldo, const Dims& g, hipStream_t s) {
  const int tiles_m = g.T_pad / KN_BM, tiles_n = (N + KN_BN - 1) / KN_BN;
  nt_gemm_kernel<<<tiles_m * tiles_n * g.B, 64 * KN_NW, 0, s>>>(A, lda, Bm, ldb, N, K, out, ldo, g,
                                                              tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_to_slab(const void* src, bool src_f32, int64_t ld_src, uint16_t* dst, int B,
                          int T, int T_pad, int D, bool flat, hipStream_t s) {
  const int grid = grid_of((int64_t)B * (T_pad / 8) * (D / 8));
  if (src_f32)
    to_slab_kernel<true><<<grid, kBwThreads, 0, s>>>(src, ld_src, dst, B, T, T_pad, D, flat ? 1 : 0);
  else
    to_slab_kernel<false><<<grid, kBwThreads, 0, s>>>(src, ld_src, dst, B, T, T_pad, D, flat ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* src, bool src_f32, uint16_t* dst, int rows,
                                 int cols, int64_t ld_dst, int step, hipStream_t s) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  if (src_f32)
    transpose_bf16_kernel<true><<<grid, kBwThreads, 0, s>>>(src, dst, rows, cols, ld_dst, step);
  else
    transpose_bf16_kernel<false><<<grid, kBwThreads, 0, s>>>(src, dst, rows, cols, ld_dst, step);
  return hipGetLastError();
}

hipError_t launch_rows_bf16(const void* src, bool src_f32, int64_t ld_src, uint16_t* dst,
                            int64_t ld_dst, int64_t rows, int cols, hipStream_t s) {
  const int grid = grid_of(rows * (cols / 8));
  if (src_f32)
    rows_bf16_kernel<true><<<grid, kBwThreads, 0, s>>>(src, ld_src, dst, ld_dst, rows, cols);
  else
    rows_bf16_kernel<false><<<grid, kBwThreads, 0, s>>>(src, ld_src, dst, ld_dst, rows, cols);
  return hipGetLastError();
}

int64_t conv_bwd_part_floats(int B, int T, int K, int d) {
  return (int64_t)B * ((T + kTapRows - 1) / kTapRows) * K * d;
}

hipError_t launch_conv_bwd(const float* dY, const uint16_t* X0, const void* taps, bool taps_f32,
                           float* dX0, float* dtaps, float* part, int B, int T, int d, int K,
                           int chunk, bool pad_chunk, hipStream_t s) {
  const int tg = (T + 7) / 8;
  const int gx = grid_of((int64_t)B * tg * (d / 8));
  if (taps_f32)
    conv_bwd_x_kernel<true><<<gx, kBwThreads, 0, s>>>(dY, taps, dX0, B, T, d, K, chunk,
                                                      pad_chunk ? 1 : 0);
  else
    conv_bwd_x_kernel<false><<<gx, kBwThreads, 0, s>>>(dY, taps, dX0, B, T, d, K, chunk,
                                                       pad_chunk ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (T + kTapRows - 1) / kTapRows;
  const int gt = grid_of((int64_t)B * nblk * ((K + 7) / 8) * (d / 8));
  conv_bwd_taps_kernel<<<gt, kBwThreads, 0, s>>>(dY, X0, part, B, T, d, K, chunk,
                                                 pad_chunk ? 1 : 0, nblk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)K * d;
  sum_parts_kernel<<<grid_of(n), kBwThreads, 0, s>>>(part, n, B * nblk, dtaps, n);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* in, int64_t stride, int n_parts, float* out, int64_t n,
                            hipStream_t s) {
  sum_parts_kernel<<<grid_of(n), kBwThreads, 0, s>>>(in, stride, n_parts, out, n);
  return hipGetLastError();
}

}  // namespace tttk
