// gfx950 (CDNA4) kernels of the In-Place TTT gated-MLP prefill.
//
// The four dense contractions (gate/up projection, target projection, the
// fast-weight update and the apply) share one MFMA GEMM core (ttt_gemm.h):
//   C[M][N] = sum_k A[m][k] * B[n][k],  both operands K-contiguous in HBM.
//
// Method sources: "论文精读：In-Place Test-Time Training" reading notes —
// "In-Place 设计" (gated MLP), "Chunk-Wise 更新机制" (update equation),
// "LM-Aligned 目标函数" (target equation); iplexlaw explainer of In-Place
// Test-Time Training, §3 (apply, then update) and §6 (exclusive prefix over
// chunk deltas).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_device.h"
#include "ttt_gemm.h"
#include "ttt_launch.h"

namespace tttk {
namespace {

// ------------------------------------------------ gate/up + SiLU*mul (K1)
// M = tokens (256), N = 128 columns of Wg and the same 128 of Wu, K = d.
// Waves 2 x 4: each wave owns 128 tokens x 32 columns of Wg and of Wu. The
// weights come packed (Wgp / Wup: one contiguous slab per tile and K step).
// The weights' stages run one step deeper than H's (160 KB of LDS): 1% faster.
constexpr int K1_NW = 8, K1_BM = 256, K1_BN = 2 * kWRows, K1_WGM = 2, K1_BK = kGateBK,
              K1_NSTA = 2, K1_NSTB = 3;
constexpr int K1_LDZ = K1_BN / 2 + 8;  // row stride of the Z staging tile in LDS
static_assert(K1_BM * K1_LDZ <= (K1_NSTA * K1_BM + K1_NSTB * K1_BN) * K1_BK,
              "Z staging fits the stages");

// One gate/up tile: Z (bf16, token-major, unless null) and zscale * Z
// (fp16, or bf16 with ZT_BF16, ZT, unless null). With sa (the backward),
// also the SiLU's derivative factors in accumulator-fragment order
// (sa_frag_offset; padding tokens get zero): the low half of each word
// bf16(phi(G)), the high half bf16(U phi'(G)), phi'(x) = sigma(x) (1 + x
// (1 - sigma(x))); with ZTb, also Z^T as bf16 at scale 1 (the training
// forward keeps both for the backward). Returns the largest |Z| of this
// lane's values.
template <bool ZT_BF16 = false>
__device__ __forceinline__ float gate_up_tile(const TileIdx& ti, u16* lds,
                                              const u16* __restrict__ H,
                                              const u16* __restrict__ Wgp,
                                              const u16* __restrict__ Wup, u16* __restrict__ Z,
                                              u16* __restrict__ ZT, const Dims& g, float zscale,
                                              uint32_t* __restrict__ sa = nullptr,
                                              u16* __restrict__ ZTb = nullptr) {
  using L = Layout<K1_BM, K1_BN, K1_WGM, K1_NW>;
  constexpr int NG = L::TN / 2;  // gate tiles per wave (and as many up tiles)
  static_assert(NG >= 1 && L::TN == 2 * NG, "gate and up tiles pair up");
  const int t0 = ti.tm * K1_BM, j0 = ti.tn * (K1_BN / 2);
  const int d = g.d, f = g.f;
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  const int nk = d / K1_BK;
  const int64_t wslab = (int64_t)ti.tn * kWRows * d;  // tile tn's packed rows
  gemm_core_ab<K1_NW, K1_BM, K1_BN, K1_WGM, K1_BK, K1_NSTA, K1_NSTB, Bf16Mma, true, kRowMajor,
               kRowMajor>(
      row_major<K1_BK>(H + ((int64_t)ti.b * g.T + t0) * d, d, min(K1_BM, g.T - t0)),
      blocked<K1_BK>(Wgp + wslab, kWRows, nk), blocked<K1_BK>(Wup + wslab, kWRows, nk), nk,
      &acc[0][0], lds, NoHook{}, k_rotation<4>(ti.tm, ti.tn, nk));
  const Frag<L> fr;
  float zmax = 0.0f;
  // Token-major Z goes through LDS so that its stores are whole 16-byte row
  // segments.
  constexpr int WROWS = K1_BM / K1_WGM;  // tile rows per wave row
#pragma unroll
  for (int m = 0; m < L::TM; ++m)
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int jl = fr.wn * NG * 32 + n * 32 + (fr.lane & 31);
      const int j = j0 + jl;
      f32x16 z;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        z[r] = silu(acc[m][n][r]) * acc[m][n + NG][r];
        zmax = fmaxf(zmax, fabsf(z[r]));
      }
      if (sa != nullptr && j < f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[m][n][4 * q + e], uv = acc[m][n + NG][4 * q + e];
            const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
            w[e] = pack_bf16(gv * sig, uv * sig * (1.0f + gv * (1.0f - sig)));
          }
          *reinterpret_cast<uint4*>(sa + sa_frag_offset(ti.b, t0 + fr.wm * L::TM * 32 + m * 32,
                                                        j - (fr.lane & 31), q, fr.lane, g)) =
              make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      if (ZTb != nullptr)
        store_tile_sb<kZtSlab>(g.T_pad, j, t0 + fr.wm * WROWS + m * 32, z, CvtBf16{1.0f}, j < f,
                               StreamSink{ZTb + ti.b * sb_elems<kZtSlab>(f, g.T_pad)});
      if (ZT != nullptr) {
        if constexpr (ZT_BF16)
          store_tile_sb<kZtSlab>(g.T_pad, j, t0 + fr.wm * WROWS + m * 32, z, CvtBf16{zscale},
                                 j < f, StreamSink{ZT + ti.b * sb_elems<kZtSlab>(f, g.T_pad)});
        else
          store_tile_sb<kZtSlab>(g.T_pad, j, t0 + fr.wm * WROWS + m * 32, z, CvtF16{zscale},
                                 j < f, StreamSink{ZT + ti.b * sb_elems<kZtSlab>(f, g.T_pad)});
      }
      if (Z != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = fr.wm * WROWS + m * 32 + 8 * q + 4 * (fr.lane >> 5);  // tile row
          u16* sZ = lds + row * K1_LDZ + jl;
#pragma unroll
          for (int e = 0; e < 4; ++e) sZ[e * K1_LDZ] = bf16_rne(z[4 * q + e]);
        }
      }
    }
  if (Z == nullptr) return zmax;
  __syncthreads();
  constexpr int CHUNKS = K1_BM * (K1_BN / 2) / 8;  // 16-byte row segments in the tile
#pragma unroll
  for (int i = 0; i < CHUNKS / (64 * K1_NW); ++i) {
    const int c = threadIdx.x + i * (64 * K1_NW);
    const int row = c >> 4, cc = c & 15;
    const u16* src = lds + row * K1_LDZ + cc * 8;
    const int t = t0 + row, jj = j0 + cc * 8;
    if (t < g.T && jj < f)
      store_stream(Z + ((int64_t)ti.b * g.T + t) * g.ld_z + jj,
                   *reinterpret_cast<const uint4*>(src));
  }
  return zmax;
}

// Z and ZT (fp16 at scale 1); the largest |Z| goes to the range group (if
// not null; only when ZT is written, the fp16 copy it guards).
__global__ __launch_bounds__(64 * K1_NW) void gate_up_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wgp, const u16* __restrict__ Wup,
    u16* __restrict__ Z, u16* __restrict__ ZT, Dims g, int tiles_m, int tiles_n,
    uint32_t* __restrict__ range) {
  TTT_GEMM_LDS_AB(lds, K1_BM, K1_BN, K1_BK, K1_NSTA, K1_NSTB)
  const float m =
      gate_up_tile(tile_index(tiles_m, tiles_n, 4), lds, H, Wgp, Wup, Z, ZT, g, 1.0f);
  if (range != nullptr) range_note(range, m);
}

// The training forward's gate/up: gate_up_kernel's Z and fp16 Z^T (with its
// range note), and for the backward Z^T as bf16 slabs and the SiLU's
// derivative factors (gate_up_tile's ZTb and sa).
__global__ __launch_bounds__(64 * K1_NW) void gate_up_train_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wgp, const u16* __restrict__ Wup,
    u16* __restrict__ Z, u16* __restrict__ ZT, u16* __restrict__ ZTb, uint32_t* __restrict__ sa,
    Dims g, int tiles_m, int tiles_n, uint32_t* __restrict__ range) {
  TTT_GEMM_LDS_AB(lds, K1_BM, K1_BN, K1_BK, K1_NSTA, K1_NSTB)
  const float m = gate_up_tile(tile_index(tiles_m, tiles_n, 4), lds, H, Wgp, Wup, Z, ZT, g, 1.0f,
                               sa, ZTb);
  range_note(range, m);
}

// The backward's recompute of gate/up: Z (bf16, token-major), Z^T as bf16
// slabs, and the SiLU's derivative factors (gate_up_tile's sa).
__global__ __launch_bounds__(64 * K1_NW) void gate_up_bwd_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wgp, const u16* __restrict__ Wup,
    u16* __restrict__ Z, u16* __restrict__ ZT, uint32_t* __restrict__ sa, Dims g, int tiles_m,
    int tiles_n) {
  TTT_GEMM_LDS_AB(lds, K1_BM, K1_BN, K1_BK, K1_NSTA, K1_NSTB)
  (void)gate_up_tile<true>(tile_index(tiles_m, tiles_n, 4), lds, H, Wgp, Wup, Z, ZT, g, 1.0f,
                           sa);
}

// ZT again, times 2^q, when Z's noted maximum is out of the fp16 range;
// otherwise returns at once. Persistent: a grid of about one workgroup per
// compute unit walks the tiles.
__global__ __launch_bounds__(64 * K1_NW) void gate_up_repair_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wgp, const u16* __restrict__ Wup,
    u16* __restrict__ ZT, Dims g, int tiles_m, int tiles_n, const uint32_t* __restrict__ range) {
  TTT_GEMM_LDS_AB(lds, K1_BM, K1_BN, K1_BK, K1_NSTA, K1_NSTB)
  const int q = range_exp(range_read(range));
  if (q == 0) return;
  const float sc = exp2i(q);
  for (int lin = blockIdx.x; lin < tiles_m * tiles_n * g.B; lin += gridDim.x) {
    __syncthreads();  // the previous tile is done with the LDS
    (void)gate_up_tile(tile_coords(lin, tiles_m, tiles_n, 4), lds, H, Wgp, Wup, nullptr, ZT, g,
                       sc);
  }
}

// ------------------------------------------------------ target GEMM (K2)
// M = tokens (256), N = output channels (256), K = d; fp16 operands.
// Y's stages run one step deeper than W_target's (160 KB of LDS): 5% faster.
constexpr int K2_NW = 8, K2_BM = 256, K2_BN = 256, K2_WGM = 2, K2_BK = 64, K2_NSTA = 3,
              K2_NSTB = 2;

// One target tile, outputs times out_scale: fp16 VT (feature-major; bf16
// with VT_BF16), bf16 Vtok ([B][T][d]) and fp16 Vrow ([B][T_pad][ld_y]),
// each unless null. Returns the largest |out_scale * V| of this lane's
// values.
template <bool VT_BF16 = false>
__device__ __forceinline__ float target_tile(const TileIdx& ti, u16* lds,
                                             const u16* __restrict__ Y,
                                             const u16* __restrict__ WtT, u16* __restrict__ VT,
                                             u16* __restrict__ Vtok, u16* __restrict__ Vrow,
                                             float out_scale, const Dims& g,
                                             int64_t vtok_ld = 0) {
  if (vtok_ld == 0) vtok_ld = g.d;
  using L = Layout<K2_BM, K2_BN, K2_WGM, K2_NW>;
  const int t0 = ti.tm * K2_BM, c0 = ti.tn * K2_BN;
  const int d = g.d;
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  const Operand wt = row_major<K2_BK>(WtT + (int64_t)c0 * g.ld_y, g.ld_y, min(K2_BN, d - c0));
  const int nk = d / K2_BK;
  gemm_core_ab<K2_NW, K2_BM, K2_BN, K2_WGM, K2_BK, K2_NSTA, K2_NSTB, F16Mma, false, kRowMajor,
               kRowMajor>(
      row_major<K2_BK>(Y + ((int64_t)ti.b * g.T_pad + t0) * g.ld_y, g.ld_y, K2_BM), wt, wt, nk,
      &acc[0][0], lds, NoHook{}, k_rotation<4>(ti.tm, ti.tn, nk));
  const Frag<L> fr;
  float vmax = 0.0f;
#pragma unroll
  for (int m = 0; m < L::TM; ++m)
#pragma unroll
    for (int n = 0; n < L::TN; ++n) {
      const int c = c0 + fr.col(n);
#pragma unroll
      for (int r = 0; r < 16; ++r) vmax = fmaxf(vmax, fabsf(acc[m][n][r]));
      if (VT != nullptr) {
        if constexpr (VT_BF16)
          store_tile_sb<kVtSlab>(g.T_pad, c, t0 + fr.wm * L::TM * 32 + m * 32, acc[m][n],
                                 CvtBf16{out_scale}, c < d,
                                 StreamSink{VT + ti.b * sb_elems<kVtSlab>(d, g.T_pad)});
        else
          store_tile_sb<kVtSlab>(g.T_pad, c, t0 + fr.wm * L::TM * 32 + m * 32, acc[m][n],
                                 CvtF16{out_scale}, c < d,
                                 StreamSink{VT + ti.b * sb_elems<kVtSlab>(d, g.T_pad)});
      }
      if (Vtok != nullptr && c < d) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t0 + fr.row(m, q);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t + e < g.T)
              Vtok[((int64_t)ti.b * g.T + t + e) * vtok_ld + c] =
                  bf16_rne(acc[m][n][4 * q + e] * out_scale);
        }
      }
    }
  // max |out_scale * V| = |out_scale| * max |V| (rounding is monotonic)
  vmax *= fabsf(out_scale);
  if (Vrow == nullptr) return vmax;
  // Token-major fp16 out_scale * V ([B][T_pad][ld_y]) through LDS, 128 tile
  // rows per pass (the rows of one wave row), so that its stores are whole
  // 16-byte row segments.
  constexpr int LDV = K2_BN + 8;
  static_assert(K2_BM / K2_WGM == 128 &&
                    128 * LDV <= (K2_NSTA * K2_BM + K2_NSTB * K2_BN) * K2_BK,
                "staging");
#pragma unroll
  for (int pass = 0; pass < K2_WGM; ++pass) {
    __syncthreads();
    if (fr.wm == pass) {
#pragma unroll
      for (int m = 0; m < L::TM; ++m)
#pragma unroll
        for (int n = 0; n < L::TN; ++n)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m * 32 + 8 * q + 4 * (fr.lane >> 5);
            u16* sv = lds + row * LDV + fr.col(n);
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[e * LDV] = f16_rne(acc[m][n][4 * q + e] * out_scale);
          }
    }
    __syncthreads();
    constexpr int SEG = 128 * (K2_BN / 8);  // 16-byte row segments per pass
#pragma unroll
    for (int k = 0; k < SEG / (64 * K2_NW); ++k) {
      const int sidx = threadIdx.x + k * (64 * K2_NW);
      const int row = sidx / (K2_BN / 8), cc = sidx % (K2_BN / 8);
      const int t = t0 + pass * 128 + row, c = c0 + cc * 8;
      if (c < d)
        store_stream(Vrow + ((int64_t)ti.b * g.T_pad + t) * g.ld_y + c,
                     *reinterpret_cast<const uint4*>(lds + row * LDV + cc * 8));
    }
  }
  return vmax;
}

// The exponents W_target^T and conv(X0) were scaled by (their range
// groups), which the target divides out.
__device__ __forceinline__ int target_in_exp(const uint32_t* range) {
  return range_exp(range_read(range + kRangeWt * kRangeSlots)) +
         range_exp(range_read(range + kRangeY * kRangeSlots));
}

// V = conv(X0) W_target: outputs at vscale * V; the largest |vscale * V|
// goes to the range's V group when note_v (the fp16 V^T it guards is
// written). range may be null (no scaled inputs).
__global__ __launch_bounds__(64 * K2_NW) void target_kernel(
    const u16* __restrict__ Y, const u16* __restrict__ WtT, u16* __restrict__ VT,
    u16* __restrict__ Vtok, u16* __restrict__ Vrow, float vscale, Dims g, int tiles_m,
    int tiles_n, uint32_t* __restrict__ range, int note_v) {
  TTT_GEMM_LDS_AB(lds, K2_BM, K2_BN, K2_BK, K2_NSTA, K2_NSTB)
  const float sc = range != nullptr ? vscale * exp2i(-target_in_exp(range)) : vscale;
  const float m = target_tile(tile_index(tiles_m, tiles_n, 4), lds, Y, WtT, VT, Vtok, Vrow, sc, g);
  if (range != nullptr && note_v) range_note(range + kRangeV * kRangeSlots, m);
}

// gate/up and the target in one launch: workgroups [0, n_gu) take gate/up
// tiles (as gate_up_kernel), the rest target tiles (as target_kernel, with
// its V^T written and V's range noted). Both configurations hold 160 KB of
// LDS and 8 waves. Used when the two launches' last rounds are part-empty
// and the target's tiles fit into gate/up's last round, so the pair takes
// one round fewer (the Qwen3-4B shape at 8k tokens: 2432 + 320 tiles, 11
// rounds of 256 instead of 10 + 2). n_gu is gate/up's tile count rounded up
// to a multiple of 8, so the XCD of a target workgroup is that of its
// position in the target range; the gate/up workgroups whose renumbered
// position is past the last tile return at once.
__global__ __launch_bounds__(64 * K1_NW) void gate_up_target_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wgp, const u16* __restrict__ Wup,
    u16* __restrict__ Z, u16* __restrict__ ZT, int gu_tiles_m, int gu_tiles_n, int n_gu,
    const u16* __restrict__ Y, const u16* __restrict__ WtT, u16* __restrict__ VT,
    u16* __restrict__ Vrow, float vscale, int t_tiles_m, int t_tiles_n, Dims g,
    uint32_t* __restrict__ range) {
  static_assert((K1_NSTA * K1_BM + K1_NSTB * K1_BN) * K1_BK ==
                    (K2_NSTA * K2_BM + K2_NSTB * K2_BN) * K2_BK && K1_NW == K2_NW,
                "one LDS array and workgroup size for both tiles");
  TTT_GEMM_LDS_AB(lds, K1_BM, K1_BN, K1_BK, K1_NSTA, K1_NSTB)
  const int id = blockIdx.x;
  if (id < n_gu) {
    // The renumbering is a permutation of [0, n_gu): the positions past the
    // last tile are the padding (not the ids past it).
    const int lin = xcd_contiguous(id, n_gu);
    if (lin >= gu_tiles_m * gu_tiles_n * g.B) return;
    const float m = gate_up_tile(tile_coords(lin, gu_tiles_m, gu_tiles_n, 4), lds, H, Wgp, Wup,
                                 Z, ZT, g, 1.0f);
    range_note(range + kRangeZ * kRangeSlots, m);
    return;
  }
  const float sc = vscale * exp2i(-target_in_exp(range));
  const TileIdx t =
      tile_coords(xcd_contiguous(id - n_gu, (int)gridDim.x - n_gu), t_tiles_m, t_tiles_n, 4);
  const float m = target_tile(t, lds, Y, WtT, VT, nullptr, Vrow, sc, g);
  range_note(range + kRangeV * kRangeSlots, m);
}

// The backward's recompute of the target: eta * V as bf16 slabs (VT) and
// token-major bf16 (Vtok, row stride vtok_ld), the inputs' range exponents
// divided out.
__global__ __launch_bounds__(64 * K2_NW) void target_bwd_kernel(
    const u16* __restrict__ Y, const u16* __restrict__ WtT, u16* __restrict__ VT,
    u16* __restrict__ Vtok, int64_t vtok_ld, float eta, Dims g, int tiles_m, int tiles_n,
    const uint32_t* __restrict__ range) {
  TTT_GEMM_LDS_AB(lds, K2_BM, K2_BN, K2_BK, K2_NSTA, K2_NSTB)
  const float sc = eta * exp2i(-target_in_exp(range));
  (void)target_tile<true>(tile_index(tiles_m, tiles_n, 4), lds, Y, WtT, VT, Vtok, nullptr, sc,
                          g, vtok_ld);
}

// VT and Vrow again, times 2^qv, when V's noted maximum is out of the fp16
// range (qv from update_exps, with eta's exponent p); otherwise returns at
// once. Persistent grid, as gate_up_repair_kernel.
__global__ __launch_bounds__(64 * K2_NW) void target_repair_kernel(
    const u16* __restrict__ Y, const u16* __restrict__ WtT, u16* __restrict__ VT,
    u16* __restrict__ Vrow, float vscale, int p, Dims g, int tiles_m, int tiles_n,
    const uint32_t* __restrict__ range) {
  TTT_GEMM_LDS_AB(lds, K2_BM, K2_BN, K2_BK, K2_NSTA, K2_NSTB)
  int qv, qz;
  update_exps(range, p, &qv, &qz);
  if (qv == 0) return;
  const float sc = vscale * exp2i(qv - target_in_exp(range));
  for (int lin = blockIdx.x; lin < tiles_m * tiles_n * g.B; lin += gridDim.x) {
    __syncthreads();  // the previous tile is done with the LDS
    (void)target_tile(tile_coords(lin, tiles_m, tiles_n, 4), lds, Y, WtT, VT, nullptr, Vrow, sc,
                      g);
  }
}

// ------------------------------------------------- update-norm clipping
// For clipping each chunk's update eta V_i^T Z_i to a Frobenius norm
// ([iplex] §6), the norm comes from two C x C Gram matrices instead of the
// d x f delta: ||V_i^T Z_i||_F^2 = sum_{s,t in chunk i} (V_s . V_t)(Z_s . Z_t).
// Both Grams are symmetric, so only the tiles of pairs (sb <= tb) of
// 256-token blocks of a chunk are formed, and an off-diagonal tile counts
// twice. Two passes over the same tiles: the first forms the V Gram tile
// (K = d_model, fp16, on vscale * V) and keeps it in the gram buffer, each
// lane its own accumulator registers; the second forms the Z Gram tile
// (K = d_ff, bf16) in KG_SPLIT parts of d_ff and writes the sum of its
// elementwise product with the kept V tile to partial[b][chunk][pair][part]
// (the sum is linear in the Z Gram, so the parts add up).
constexpr int KG_NW = 8, KG_B = 256, KG_WGM = 2, KG_SPLIT = 2, KG_NSTA = 2, KG_NSTB = 3;
constexpr int KG_THREADS = 64 * KG_NW;

struct GramTile {
  int b, i, pair, part, s0, u0, c1, weight;
};

__device__ __forceinline__ GramTile gram_tile(const Dims& g, int chunk, int nblk, int npair,
                                              int nchunks, int parts,
                                              const ChunkSpan* __restrict__ spans) {
  GramTile t;
  int rest = blockIdx.x;
  t.part = rest % parts;
  rest /= parts;
  t.pair = rest % npair;
  rest /= npair;
  t.i = rest % nchunks;
  t.b = rest / nchunks;
  int sb = 0, tb = t.pair;  // pair -> (sb, tb), sb <= tb, upper triangle row by row
  while (tb >= nblk - sb) {
    tb -= nblk - sb;
    ++sb;
  }
  tb += sb;
  // A span table's values are clamped to the sequence, so a wrong table
  // gives wrong norms, never a read outside the operands.
  const int c0 = spans ? min(max(spans[t.i].t0, 0), g.T) : t.i * chunk;
  t.c1 = spans ? min(max(spans[t.i].t1, c0), g.T) : min(g.T, c0 + chunk);
  t.s0 = c0 + sb * KG_B;
  t.u0 = c0 + tb * KG_B;
  t.weight = sb == tb ? 1 : 2;
  return t;
}

// One Gram tile X[s0..] X[u0..]^T over K columns [k0, k0 + nk * 64) of the
// row-major X (row stride ld, rows_b rows per sequence), rows at or past c1
// reading as zero.
template <class Op>
__device__ __forceinline__ void gram_tile_acc(const u16* X, int64_t ld, int64_t rows_b,
                                              const GramTile& t, int k0, int nk, f32x16* acc,
                                              u16* lds) {
  const Operand xs = row_major<64>(X + ((int64_t)t.b * rows_b + t.s0) * ld + k0, ld, t.c1 - t.s0);
  const Operand xu = row_major<64>(X + ((int64_t)t.b * rows_b + t.u0) * ld + k0, ld, t.c1 - t.u0);
  gemm_core_ab<KG_NW, KG_B, KG_B, KG_WGM, 64, KG_NSTA, KG_NSTB, Op, false, kRowMajor, kRowMajor>(
      xs, xu, xu, nk, acc, lds, NoHook{});
}

__global__ __launch_bounds__(KG_THREADS) void gram_v_kernel(
    const u16* __restrict__ Vrow, float* __restrict__ gram, Dims g, int chunk, int nblk,
    int npair, int nchunks, const ChunkSpan* __restrict__ spans) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using L = Layout<KG_B, KG_B, KG_WGM, KG_NW>;
  constexpr int NR = L::TM * L::TN * 16;  // accumulator registers per lane
  TTT_GEMM_LDS_AB(lds, KG_B, KG_B, 64, KG_NSTA, KG_NSTB)
  const GramTile t = gram_tile(g, chunk, nblk, npair, nchunks, 1, spans);
  if (t.u0 >= t.c1) return;  // uniform: blocks past a short last chunk add nothing
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  gram_tile_acc<F16Mma>(Vrow, g.ld_y, g.T_pad, t, 0, g.d / 64, &acc[0][0], lds);
  // Lane-private layout [tile][register][thread]: each register's stores are
  // 256 contiguous bytes per wave; the second pass reads them in the same
  // lanes.
  float* dst = gram + (((int64_t)t.b * nchunks + t.i) * npair + t.pair) * NR * KG_THREADS +
               threadIdx.x;
#pragma unroll
  for (int m = 0; m < L::TM; ++m)
#pragma unroll
    for (int n = 0; n < L::TN; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[((m * L::TN + n) * 16 + r) * KG_THREADS] = acc[m][n][r];
#endif
}

__global__ __launch_bounds__(KG_THREADS) void gram_norm_kernel(
    const u16* __restrict__ Z, const float* __restrict__ gram, float* __restrict__ partial,
    Dims g, int chunk, int nblk, int npair, int nchunks, const ChunkSpan* __restrict__ spans) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using L = Layout<KG_B, KG_B, KG_WGM, KG_NW>;
  constexpr int NR = L::TM * L::TN * 16;
  TTT_GEMM_LDS_AB(lds, KG_B, KG_B, 64, KG_NSTA, KG_NSTB)
  float* wsum = reinterpret_cast<float*>(lds);  // per-wave sums, once the core is done
  const GramTile t = gram_tile(g, chunk, nblk, npair, nchunks, KG_SPLIT, spans);
  const int steps = g.f / 64, per = (steps + KG_SPLIT - 1) / KG_SPLIT;
  const int k_first = t.part * per, nk = min(steps, k_first + per) - k_first;
  float sum = 0.f;
  if (t.u0 < t.c1 && nk > 0) {  // uniform
    f32x16 acc[L::TM][L::TN];
    zero_acc(acc);
    gram_tile_acc<Bf16Mma>(Z, g.ld_z, g.T, t, k_first * 64, nk, &acc[0][0], lds);
    const float* src = gram +
                       (((int64_t)t.b * nchunks + t.i) * npair + t.pair) * NR * KG_THREADS +
                       threadIdx.x;
#pragma unroll
    for (int m = 0; m < L::TM; ++m)
#pragma unroll
      for (int n = 0; n < L::TN; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sum = fmaf(acc[m][n][r], src[((m * L::TN + n) * 16 + r) * KG_THREADS], sum);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < KG_NW; ++w) tot += wsum[w];
    partial[(((int64_t)t.b * nchunks + t.i) * npair + t.pair) * KG_SPLIT + t.part] =
        (float)t.weight * tot;
  }
#endif
}

// scale[b][i] = min(1, clip / ||eta V_i^T Z_i||_F), the norm being
// norm_factor * 2^-qv * sqrt(sum of chunk i's npair partials), summed in a
// fixed order (the Gram tiles come from V at vscale * 2^qv; qv from the
// range groups when range is not null).
__global__ __launch_bounds__(kThreads) void clip_scale_kernel(const float* __restrict__ partial,
                                                             float* __restrict__ scale, int npair,
                                                             int n, float norm_factor,
                                                             float clip,
                                                             const uint32_t* __restrict__ range,
                                                             int p) {
  if (range != nullptr) {
    int qv, qz;
    update_exps(range, p, &qv, &qz);
    norm_factor *= exp2i(-qv);
  }
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= n) return;
  double s2 = 0.0;
  for (int p = 0; p < npair; ++p) s2 += (double)partial[(int64_t)idx * npair + p];
  const double nrm = (double)norm_factor * sqrt(s2 > 0.0 ? s2 : 0.0);
  scale[idx] = nrm > (double)clip ? (float)((double)clip / nrm) : 1.0f;
}

// VT *= scale of each token's chunk (a 64-token slab lies in one chunk: the
// block table's entry for a packed sequence, else token / chunk).
__global__ __launch_bounds__(kThreads) void vt_scale_kernel(u16* __restrict__ VT,
                                                           const float* __restrict__ scale,
                                                           Dims g, int chunk, int nchunks,
                                                           const BlockInfo* __restrict__ blocks,
                                                           int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n16) return;
  const int64_t e = i * 8, per_b = sb_elems<kVtSlab>(g.d, g.T_pad);
  const int b = (int)(e / per_b);
  const int64_t slab = (e % per_b) / (kVtSlab * 64);
  const int tok = (int)(slab % (g.T_pad / 64)) * 64;
  const int ci = blocks ? min(max(blocks[tok / 64].chunk, 0), nchunks - 1)
                        : min(tok / chunk, nchunks - 1);
  const float sc = scale[(int64_t)b * nchunks + ci];
  if (sc == 1.0f) return;
  uint4 v = reinterpret_cast<uint4*>(VT)[i];
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = (float)__builtin_bit_cast(_Float16, (u16)(w[k] & 0xffffu));
    const float hi = (float)__builtin_bit_cast(_Float16, (u16)(w[k] >> 16));
    w[k] = pack_f16(lo * sc, hi * sc);
  }
  reinterpret_cast<uint4*>(VT)[i] = make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------ fast-weight update (K3)
// M = d_ff (256), N = d_model (256 or 128), K = tokens; fp16 operands. acc
// starts at acc_scale * state and absorbs (vscale V)^T Z one 64-token step
// at a time; at every chunk start the state before that chunk is stored as
// a bf16 snapshot (the exclusive prefix).
// A launch covers the state in 256 x 256 regions. It runs whole rounds (one
// tile per compute unit) of wide 256 x 256 tiles and, when the regions left
// over would fill at most half a round, splits each of them into two narrow
// 256 x 128 tiles, so that the last round is one of narrow tiles instead of
// a part-empty round of wide ones. Wide tiles read half the operand bytes per
// MFMA that narrow ones do. Both the plain and the packed variant do this.
constexpr int K3_NW = 8, K3_BM = 256, K3_BK = 64, K3_WIDE = 256, K3_NARROW = 128;
template <int BN>
struct UpdCfg {
  static constexpr int WGM = BN == K3_WIDE ? 2 : 4;
  // Wide: Z^T three stages, V^T two; narrow: Z^T four, V^T two (160 KB
  // each, the whole LDS; the packed variant keeps its step table in
  // registers).
  static constexpr int NSTA = BN == K3_WIDE ? 3 : 4;
  static constexpr int NSTB = 2;
};
constexpr int kUpdLdsElems = 160 * 1024 / 2;  // the stages of either width

// Stores bf16(acc * out_scale) of a [d_ff tile] x [d_model tile] state block
// into an sb<256> d x f bf16 matrix of `bytes` bytes (row c = d_model index,
// column j = d_ff index). Buffer stores: a lane outside the matrix stores
// at offset `bytes`, which the buffer bound drops, so every wave issues
// exactly kStores of them. They are streaming, system-scope stores (nt sc1):
// the apply reads the snapshots only after this kernel, and keeping them out
// of the way of the operand stream measured 4% faster.
// OPQ: the addresses are computed at each call (Frag opaque), for the
// packed update, whose hook otherwise keeps them live across the K loop.
template <class L, bool OPQ = false>
struct SnapshotStore {
  static constexpr int kStores = L::TM * L::TN * 2;
  int j0, c0, d, f;
  int kdim;  // columns of the snapshot matrix (>= f; the state fills columns [0, f))
  float out_scale;
  uint32_t bytes;
  // Where the accumulator tiles go. The tile's d_ff start j0 is a multiple
  // of 256 and its d_model start c0 one of 128, and a wave's blocks stay
  // inside one 256-row slab row (c) and start at a multiple of 64 columns
  // (j), so every store of the wave lands at this lane's byte offset for
  // tile (0, 0) plus a constant: tile (m, n) half p of sb<256> element
  // (c, jb + 16 p + 8 h) is (m / 2) slabs (32 KB), (m % 2) column groups of
  // 32 (2 KB), n 32-row blocks (4 KB) and p 16-column halves (1 KB) further
  // on. The base is computed once per call instead of per tile.
  __device__ __forceinline__ void operator()(u16* dst, const f32x16* acc) const {
    static_assert(L::WGN * L::TN * 32 <= 128 || L::WGN * L::TN * 32 == 256,
                  "a wave's columns stay in one slab row");
    const Frag<L> fr(OPQ);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int)bytes, kRsrcWord3);
    const uint32_t lane = (uint32_t)fr.lane;
    const uint32_t jw = (uint32_t)(j0 + fr.wm * L::TM * 32);  // multiple of 64
    const uint32_t cw = (uint32_t)(c0 + fr.wn * L::TN * 32);
    const uint32_t base =
        2u * ((((cw >> 8) * ((uint32_t)kdim >> 6) + (jw >> 6)) << 14) +
              (((cw & 255u) >> 5) << 11) + ((((lane >> 5) & 1u) << 5) + (lane & 31u)) * 8u);
    const CvtBf16 cvt{out_scale};
#pragma unroll
    for (int m = 0; m < L::TM; ++m)
#pragma unroll
      for (int n = 0; n < L::TN; ++n) {
        const bool ok = cw + (uint32_t)(n * 32) + (lane & 31u) < (uint32_t)d &&
                        jw + (uint32_t)(m * 32) < (uint32_t)f;
        const uint32_t off =
            ok ? base + (uint32_t)((m >> 1) * 32768 + (m & 1) * 2048 + n * 4096) : bytes;
        const f32x16& a = acc[m * L::TN + n];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          // The two 16-byte pieces of store_tile_sb, lanes l and l ^ 32
          // trading halves with v_permlane32_swap.
          const uint32_t lo0 = cvt(a[8 * p + 0], a[8 * p + 1]), lo1 = cvt(a[8 * p + 2], a[8 * p + 3]);
          const uint32_t hi0 = cvt(a[8 * p + 4], a[8 * p + 5]), hi1 = cvt(a[8 * p + 6], a[8 * p + 7]);
          const auto x0 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);
          const auto x1 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);
          const u32x4 w = {x0[0], x1[0], x0[1], x1[1]};
          // A dropped lane stores at `bytes` or 1 KB past it: out of bounds.
          __builtin_amdgcn_raw_buffer_store_b128(w, rsrc, (int)(off + p * 1024u), 0,
                                                 kCpolNt | kCpolSc1);
        }
      }
  }
};

// acc = acc_scale * W for the wave's part of a [d_ff tile] x [d_model tile]
// state block, W element (c, j) at W + c * ld + j (bf16 or fp32). BATCHED:
// the loads are unconditional (lanes outside the matrix read element 0 and
// drop it), so that they are issued back to back and waited for once; this
// needs registers for all of them, so inside the K loop (the packed
// update's reset) the per-element conditional form is used instead.
// TRANS: element (c, j) at W + j * ld + c instead (four scalar loads).
template <class L, bool F32, bool BATCHED = true, bool OPQ = false, bool TRANS = false>
struct StateLoad {
  const void* W;
  int64_t ld;
  int j0, c0, d, f;
  float acc_scale;
  __device__ __forceinline__ void operator()(f32x16* acc) const {
    const Frag<L> fr(OPQ);
#pragma unroll
    for (int m = 0; m < L::TM; ++m)
#pragma unroll
      for (int n = 0; n < L::TN; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + fr.row(m, q);
          const int c = c0 + fr.col(n);
          const bool in = c < d && j < f;
          const int64_t o = in ? (int64_t)c * ld + j : 0;
          const float keep = in ? acc_scale : 0.0f;
          float v[4] = {0.f, 0.f, 0.f, 0.f};
          if (!BATCHED && !in) {
            // no load
          } else if constexpr (TRANS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t oe = in ? (int64_t)(j + e) * ld + c : 0;
              v[e] = F32 ? static_cast<const float*>(W)[oe]
                         : bf16_f32(static_cast<const u16*>(W)[oe]);
            }
          } else if constexpr (F32) {
            const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + o);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const u16*>(W) + o);
            v[0] = __uint_as_float(x.x << 16);
            v[1] = __uint_as_float(x.x & 0xffff0000u);
            v[2] = __uint_as_float(x.y << 16);
            v[3] = __uint_as_float(x.y & 0xffff0000u);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[m * L::TN + n][4 * q + e] = v[e] * keep;
        }
  }
};

// A packed launch's block table, reduced to what the update's hook reads
// and held in three registers per lane: lane l covers K steps [32 l,
// 32 l + 32) (2048 steps = 131072 tokens in all), bit i of chunk_start /
// doc_start flags step 32 l + i, and base is the chunk of step 32 l. The
// chunk of step kt is base + the chunk starts in (32 l, kt]. Registers
// instead of an LDS copy leave the whole LDS to the pipeline's stages; a
// global read in the loop would need a vmcnt wait, which also waits for the
// stage loads in flight.
struct StepBits {
  uint32_t chunk_start, doc_start;
  int base;
};

// The update's hook: the exclusive-prefix snapshot at every chunk start and,
// for packed documents (PACKED), the reset to the initial state at every
// document start after the first ([iplex] §6), with chunk starts taken from
// the block table. The reset's loads are waited for at once; they only
// lengthen the pipeline's waits that follow. The plain kernel is compiled
// without the reset, which would otherwise keep its addresses live across
// the K loop.
// REV: the K steps run backwards over the tokens (a reverse scan): step kt
// reads block r = nk - 1 - kt, and the snapshot of chunk i is the state
// before its last block is read, i.e. after every later chunk.
template <class L, bool F32, bool PACKED, bool REV = false>
struct ChunkSnapshots {
  static constexpr int kStores = SnapshotStore<L, PACKED>::kStores;
  static constexpr bool kReverse = REV;
  SnapshotStore<L, PACKED> store;
  StateLoad<L, F32, false, PACKED> reset;
  u16* snap;  // this sequence's snapshots, or null
  int64_t chunk_stride;
  int steps_per_chunk;
  StepBits bits;  // PACKED: this launch's steps
  int n_chunks;   // PACKED: snapshot slots (table values are clamped to them)
  int nk;         // REV: the launch's K steps
  __device__ __forceinline__ bool operator()(int kt, f32x16* acc) const {
    int slot;
    if constexpr (REV) {
      const int r = nk - 1 - kt;
      if (snap == nullptr || ((r + 1) % steps_per_chunk != 0 && kt != 0)) return false;
      slot = r / steps_per_chunk;
    } else if constexpr (PACKED) {
      // kt is uniform, so these are scalar reads of one lane's registers.
      const int lane = kt >> 5, bit = kt & 31;
      const uint32_t cs = (uint32_t)__builtin_amdgcn_readlane((int)bits.chunk_start, lane);
      const uint32_t ds = (uint32_t)__builtin_amdgcn_readlane((int)bits.doc_start, lane);
      const bool doc = ((ds >> bit) & 1u) && kt > 0;
      if (doc) reset(acc);
      // After a reset the state is W_down0 again, whose snapshot is slot 0:
      // a later document's first chunk reads that slot (the apply's tile
      // list says so), and nothing is stored here.
      if (snap == nullptr || doc || !((cs >> bit) & 1u)) return false;
      const uint32_t later = ((2u << bit) - 1u) & ~1u;  // steps 32 l + 1 .. kt
      slot = min(__builtin_amdgcn_readlane(bits.base, lane) + __builtin_popcount(cs & later),
                 n_chunks - 1);
    } else {
      if (snap == nullptr || kt % steps_per_chunk != 0) return false;
      slot = kt / steps_per_chunk;
    }
    store(snap + (int64_t)slot * chunk_stride, acc);
    return true;
  }
};

// A block's {chunk, flags} in one word, for the packed update's LDS copy.
__device__ __forceinline__ uint32_t step_word(const BlockInfo& b) {
  return ((uint32_t)b.chunk & 0x3fffffffu) | ((uint32_t)(b.flags & 3) << 30);
}
constexpr int kMaxPackedSteps = 2048;  // K steps of a packed update launch (131072 tokens)

// Every lane's StepBits from this launch's block table, staged through the
// LDS stage memory (free until the pipeline's first loads; the barrier at the
// end keeps them from overwriting it while a wave still reads). Table
// values are clamped, so a wrong table gives wrong numbers, never a wild
// address.
__device__ __forceinline__ StepBits load_step_bits(u16* lds, const BlockInfo* __restrict__ blocks,
                                                   int first_block, int nk, int n_chunks) {
  uint32_t* words = reinterpret_cast<uint32_t*>(lds);
  for (int k = threadIdx.x; k < nk; k += 64 * K3_NW) words[k] = step_word(blocks[first_block + k]);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  StepBits sb{0u, 0u, 0};
#pragma unroll 4
  for (int jj = 0; jj < 32; ++jj) {
    const int j = (jj + lane) & 31;  // skewed, so the lanes read different banks
    const int k = lane * 32 + j;
    if (k < nk) {
      const uint32_t w = words[k];
      sb.chunk_start |= ((w >> 30) & (uint32_t)kBlockChunkStart ? 1u : 0u) << j;
      sb.doc_start |= ((w >> 30) & (uint32_t)kBlockDocStart ? 1u : 0u) << j;
      if (j == 0) sb.base = min((int)(w & 0x3fffffffu), n_chunks - 1);
    }
  }
  __syncthreads();
  return sb;
}

// One update tile: d_ff rows [j0, j0 + 256) and d_model columns
// [c0, c0 + BN) of sequence b's state.
// The update's tile in general form: the state block is acc[m][n] for M
// index j (rows of the A slab matrix, g.f of them) and N index c (rows of
// the B slab matrix, g.d of them), contracted over tokens; its element
// (c, j) lives at W[c][j] (ld = g.f). MMA: fp16 or bf16 operands. REV: the
// tokens run backwards (snapshots as ChunkSnapshots). TRANS: the initial
// state is read as W[j][c] (ld = winit_ld) instead. Winit null: the state
// starts at zero; Wf null: no final store.
template <int BN, bool WINIT_F32, bool PACKED, class MMA = F16Mma, bool REV = false,
          bool TRANS = false>
__device__ __forceinline__ void update_tile(
    u16* lds, StepBits bits, int b, int j0, int c0, const u16* __restrict__ ZT,
    const u16* __restrict__ VT, const void* __restrict__ Winit, int64_t winit_bstride,
    int64_t winit_ld, float acc_scale, u16* __restrict__ snap, int64_t snap_bstride,
    float* __restrict__ Wf, u16* __restrict__ shadow, const Dims& g, int tok_begin, int nk,
    int steps_per_chunk, int n_chunks, int snap_k) {
  using C = UpdCfg<BN>;
  using L = Layout<K3_BM, BN, C::WGM, K3_NW>;
  constexpr int TM = L::TM, TN = L::TN, NSTA = C::NSTA, NSTB = C::NSTB;
  static_assert((NSTA * K3_BM + NSTB * BN) * K3_BK <= kUpdLdsElems, "stages fit");
  const int d = g.d, f = g.f;
  const Frag<L> fr;
  // Snapshots are sb<256>(d x snap_k) matrices whose first f columns hold the
  // state (snap_k = f but for the backward's side-by-side copies).
  const int64_t chunk_stride = sb_elems<kSnapSlab>(d, snap_k);
  const float out_scale = 1.0f / acc_scale;

  const void* winit_b =
      Winit == nullptr ? nullptr
      : WINIT_F32 ? (const void*)(static_cast<const float*>(Winit) + b * winit_bstride)
                  : (const void*)(static_cast<const u16*>(Winit) + b * winit_bstride);
  const StateLoad<L, WINIT_F32, true, false, TRANS> init{winit_b, winit_ld, j0, c0, d, f,
                                                         acc_scale};
  const StateLoad<L, WINIT_F32, false, PACKED> reset{winit_b, winit_ld, j0, c0, d, f,
                                                     acc_scale};
  f32x16 acc[TM][TN];
  if (winit_b != nullptr)
    init(&acc[0][0]);
  else
    zero_acc(acc);

  const SnapshotStore<L, PACKED> snapshot{j0, c0, d, f, snap_k, out_scale,
                                          (uint32_t)(chunk_stride * 2)};
  const ChunkSnapshots<L, WINIT_F32, PACKED, REV> hook{
      snapshot, reset, snap ? snap + b * snap_bstride : nullptr, chunk_stride,
      steps_per_chunk, bits, n_chunks, nk};
  // Rows past d_ff / d_model in the last slabs are never written; they only
  // feed output rows / columns that are not stored. A narrow tile reads the
  // first or second 128 rows of a 256-row V^T slab: 16 contiguous KB per K
  // step.
  static_assert(K3_BM == kZtSlab && kVtSlab == K3_WIDE && BN <= kVtSlab && K3_BK == 64,
                "update tile rows = slab rows");
  const Operand vt =
      slab_blocked<kVtSlab>(VT + b * sb_elems<kVtSlab>(d, g.T_pad), g.T_pad, c0, tok_begin);
  gemm_core_ab<K3_NW, K3_BM, BN, C::WGM, K3_BK, NSTA, NSTB, MMA, false, kSlab, kSlab>(
      slab_blocked<kZtSlab>(ZT + b * sb_elems<kZtSlab>(f, g.T_pad), g.T_pad, j0, tok_begin),
      vt, vt, nk, &acc[0][0], lds, hook);

  if (shadow != nullptr) snapshot(shadow + (int64_t)b * chunk_stride, &acc[0][0]);
  if (Wf == nullptr) return;
  float* wf_b = Wf + (int64_t)b * d * f;
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + fr.row(m, q);
        const int c = c0 + fr.col(n);
        if (c < d && j < f)
          *reinterpret_cast<float4*>(wf_b + (int64_t)c * f + j) =
              make_float4(acc[m][n][4 * q] * out_scale, acc[m][n][4 * q + 1] * out_scale,
                          acc[m][n][4 * q + 2] * out_scale, acc[m][n][4 * q + 3] * out_scale);
      }
}

// Workgroups [0, n_wide) take the wide tiles of regions [0, n_wide); the
// rest take the two narrow halves of each remaining region (regions in
// tile_coords order over regions_m x regions_n 256 x 256 regions per
// sequence, group 4).
// The state is carried as acc_scale * W, acc_scale = 2^(p + qv + qz): eta's
// exponent p and the operands' range exponents (none when range is null).
template <bool WINIT_F32, bool PACKED, class MMA = F16Mma, bool REV = false,
          bool TRANS = false>
__global__ __launch_bounds__(64 * K3_NW) void update_kernel(
    const u16* __restrict__ ZT, const u16* __restrict__ VT, const void* __restrict__ Winit,
    int64_t winit_bstride, int64_t winit_ld, int p, const uint32_t* __restrict__ range,
    u16* __restrict__ snap, int64_t snap_bstride, float* __restrict__ Wf,
    u16* __restrict__ shadow, Dims g, int tok_begin, int nk, int steps_per_chunk,
    const BlockInfo* __restrict__ blocks, int n_chunks, int regions_m, int regions_n,
    int n_wide, int snap_k) {
  __shared__ __attribute__((aligned(16))) u16 lds[kUpdLdsElems];
  int e = p;
  if (range != nullptr) {
    int qv, qz;
    update_exps(range, p, &qv, &qz);
    e += qv + qz;
  }
  const float acc_scale = exp2i(e);
  StepBits bits{0u, 0u, 0};
  // nk <= kMaxPackedSteps for a packed launch (checked on the host).
  if constexpr (PACKED) bits = load_step_bits(lds, blocks, tok_begin / K3_BK, nk, n_chunks);
  if ((int)blockIdx.x < n_wide) {
    const TileIdx t = tile_coords(xcd_contiguous(blockIdx.x, n_wide), regions_m, regions_n, 4);
    update_tile<K3_WIDE, WINIT_F32, PACKED, MMA, REV, TRANS>(
        lds, bits, t.b, t.tm * K3_BM, t.tn * K3_WIDE, ZT, VT, Winit, winit_bstride, winit_ld,
        acc_scale, snap, snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
        n_chunks, snap_k);
    return;
  }
  // n_wide is a multiple of 8 whenever narrow tiles follow, so the XCD of a
  // workgroup is that of its position in the narrow range.
  const int id = xcd_contiguous(blockIdx.x - n_wide, gridDim.x - n_wide);
  const TileIdx t = tile_coords(n_wide + id / 2, regions_m, regions_n, 4);
  const int c0 = t.tn * K3_WIDE + (id & 1) * K3_NARROW;
  if (c0 >= g.d) return;  // uniform: the half of a region past d_model
  update_tile<K3_NARROW, WINIT_F32, PACKED, MMA, REV, TRANS>(
      lds, bits, t.b, t.tm * K3_BM, c0, ZT, VT, Winit, winit_bstride, winit_ld, acc_scale,
      snap, snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk, n_chunks, snap_k);
}

// ------------------------------------------------------------ apply (K4)
// M = d_model (256), N = tokens (BN, which divides the chunk), K = d_ff.
// The tile's tokens all lie in one chunk i and read snapshot i.
// The XCD's resident apply tiles: 8 d_model tiles x 4 token tiles, which
// (with 256-token tiles) share one chunk's snapshot slabs.
constexpr int kApplyGroupM = 8;

template <int BN, bool TAIL = false>
struct ApplyCfg {
  static constexpr int NW = 8;
  static constexpr int WGM =
      BN == 256 ? 2 : (BN == 128 ? 4 : 8);
  // With 256-token tiles, Z's stages run one step deeper than the
  // snapshot's (160 KB of LDS): 10% faster. Narrower tiles keep two each,
  // but for the 128-token halves of a whole-sequence launch's last round
  // (TAIL), which have the launch's 160 KB: three snapshot stages and four
  // of Z take that round at the 8k Qwen3-4B shape from 0.22 to 0.16 ms (two
  // of each: the halves were bound by the load latency of every K step).
  static constexpr int BK = 64, NSTA = TAIL ? 3 : 2, NSTB = TAIL ? 4 : (BN == 256 ? 3 : 2);
};

// One apply tile: d_model rows [256 ti.tm, 256 ti.tm + 256) of sequence
// ti.b for the tokens [t0, t1) (at most BN, all in chunk i), from snapshot i.
template <int BN, bool OUT_F32, bool TAIL = false>
__device__ __forceinline__ void apply_tile(u16* lds, const TileIdx& ti, int t0, int t1, int i,
                                           const u16* __restrict__ Z,
                                           const u16* __restrict__ snap, int64_t snap_bstride,
                                           int64_t snap_cstride, void* __restrict__ O,
                                           const Dims& g) {
  using Cfg = ApplyCfg<BN, TAIL>;
  constexpr int BM = kSnapSlab, WGM = Cfg::WGM, BK = Cfg::BK, NSTA = Cfg::NSTA,
                NSTB = Cfg::NSTB;
  static_assert(BK == 64, "the snapshot slab is one K step");
  using L = Layout<BM, BN, WGM, Cfg::NW>;
  const int c0 = ti.tm * BM;
  const int d = g.d, f = g.f, T = g.T;
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  const Operand z =
      row_major<BK>(Z + ((int64_t)ti.b * T + t0) * g.ld_z, g.ld_z, min(BN, T - t0));
  // The rotation follows the absolute 256-token block, whatever the tile
  // width, so that every schedule and width sums each output in the same
  // order.
  const int nk = f / BK;
  gemm_core_ab<Cfg::NW, BM, BN, WGM, BK, NSTA, NSTB, Bf16Mma, false, kSlab, kRowMajor>(
      slab_blocked<kSnapSlab>(snap + ti.b * snap_bstride + i * snap_cstride, f, c0, 0), z, z, nk,
      &acc[0][0], lds, NoHook{}, k_rotation<kApplyGroupM>(ti.tm, t0 / 256, nk));
  const Frag<L> fr;
#pragma unroll
  for (int m = 0; m < L::TM; ++m)
#pragma unroll
    for (int n = 0; n < L::TN; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + fr.row(m, q);
        const int t = t0 + fr.col(n);
        if (t >= t1 || c >= d) continue;  // past the tile's chunk: another snapshot's
        const int64_t o = ((int64_t)ti.b * T + t) * d + c;
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(O) + o) =
              make_float4(acc[m][n][4 * q], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                          acc[m][n][4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<u16*>(O) + o) =
              make_uint2(pack_bf16(acc[m][n][4 * q], acc[m][n][4 * q + 1]),
                         pack_bf16(acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]));
        }
      }
}

template <int BN, bool OUT_F32>
__global__ __launch_bounds__(64 * ApplyCfg<BN>::NW) void apply_kernel(
    const u16* __restrict__ Z, const u16* __restrict__ snap, int64_t snap_bstride,
    int64_t snap_cstride, void* __restrict__ O, Dims g, int tok_begin, int tok_end, int chunk,
    const ApplyTile* __restrict__ tiles, int n_chunks, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  TTT_GEMM_LDS_AB(lds, kSnapSlab, BN, ApplyCfg<BN>::BK, ApplyCfg<BN>::NSTA, ApplyCfg<BN>::NSTB)
  const TileIdx ti = tile_index(tiles_m, tiles_n, kApplyGroupM);
  int t0, t1, i;
  if (tiles != nullptr) {
    const ApplyTile tl = tiles[ti.tn];
    t0 = min(max(tl.t0, 0), g.T);
    t1 = min(max(tl.t1, t0), g.T);
    i = min(max(tl.chunk, 0), n_chunks - 1);
  } else {
    t0 = tok_begin + ti.tn * BN;
    t1 = min(tok_end, t0 + BN);
    i = t0 / chunk;
  }
  apply_tile<BN, OUT_F32>(lds, ti, t0, t1, i, Z, snap, snap_bstride, snap_cstride, O, g);
#endif
}

// The whole sequence's apply ([0, T), chunks a multiple of 256 tokens) when
// its 256-token tiles leave a last round at most half full: workgroups
// [0, n_wide) take whole rounds of 256-token tiles, the rest the two
// 128-token halves of each tile left over (tile_coords order, as
// apply_kernel). A half sums every output in the same order as the whole
// tile would, so the results are the same bit for bit.
template <bool OUT_F32>
__global__ __launch_bounds__(64 * ApplyCfg<256>::NW) void apply_mixed_kernel(
    const u16* __restrict__ Z, const u16* __restrict__ snap, int64_t snap_bstride,
    int64_t snap_cstride, void* __restrict__ O, Dims g, int chunk, int tiles_m, int tiles_n,
    int n_wide) {
#if defined(__HIP_DEVICE_COMPILE__)
  using Tail = ApplyCfg<128, true>;
  static_assert(ApplyCfg<256>::NW == Tail::NW, "one workgroup size");
  static_assert((Tail::NSTA * kSnapSlab + Tail::NSTB * 128) <=
                    (ApplyCfg<256>::NSTA * kSnapSlab + ApplyCfg<256>::NSTB * 256),
                "the narrow tile's stages fit the wide tile's LDS");
  TTT_GEMM_LDS_AB(lds, kSnapSlab, 256, ApplyCfg<256>::BK, ApplyCfg<256>::NSTA,
                  ApplyCfg<256>::NSTB)
  if ((int)blockIdx.x < n_wide) {
    const TileIdx ti =
        tile_coords(xcd_contiguous(blockIdx.x, n_wide), tiles_m, tiles_n, kApplyGroupM);
    const int t0 = ti.tn * 256;
    apply_tile<256, OUT_F32>(lds, ti, t0, min(g.T, t0 + 256), t0 / chunk, Z, snap, snap_bstride,
                             snap_cstride, O, g);
    return;
  }
  // n_wide is a multiple of 8, so the XCD of a workgroup is that of its
  // position in the narrow range.
  const int id = xcd_contiguous(blockIdx.x - n_wide, (int)gridDim.x - n_wide);
  const TileIdx ti = tile_coords(n_wide + id / 2, tiles_m, tiles_n, kApplyGroupM);
  const int t0 = ti.tn * 256 + (id & 1) * 128;
  if (t0 >= g.T) return;  // uniform: the half of a tile past the sequence
  apply_tile<128, OUT_F32, true>(lds, ti, t0, min(g.T, t0 + 128), t0 / chunk, Z, snap,
                                 snap_bstride, snap_cstride, O, g);
#endif
}

// --------------------------------------------------- small kernels

__global__ __launch_bounds__(kThreads) void cast_kernel(const float* __restrict__ src,
                                                        u16* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    const float4 x = reinterpret_cast<const float4*>(src)[i];
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(pack_bf16(x.x, x.y), pack_bf16(x.z, x.w));
  }
}

__global__ __launch_bounds__(kThreads) void range_clear_kernel(uint32_t* __restrict__ range) {
  for (int i = threadIdx.x; i < kRangeWords; i += kThreads) range[i] = 0u;
}

// Notes max |W| over n elements (bf16, or fp32; n a multiple of 8) in a
// range group, 16 bytes per load.
template <bool F32>
__global__ __launch_bounds__(kThreads) void amax_kernel(const void* __restrict__ W, int64_t n,
                                                        uint32_t* __restrict__ group) {
  float m = 0.0f;
  const int64_t per = F32 ? 4 : 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n / per;
       i += (int64_t)gridDim.x * kThreads) {
    if constexpr (F32) {
      const float4 x = reinterpret_cast<const float4*>(W)[i];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    } else {
      const uint4 x = reinterpret_cast<const uint4*>(W)[i];
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[e] << 16)),
                           fabsf(__uint_as_float(w[e] & 0xffff0000u))));
    }
  }
  range_note_block<kThreads>(group, m);
}

// dst = fp16(src^T 2^q), q from the range group of src (null: q = 0).
template <bool F32>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const void* __restrict__ src,
                                                             u16* __restrict__ dst, int rows,
                                                             int cols, int64_t ld_dst,
                                                             const uint32_t* __restrict__ range) {
  const float sc = range != nullptr ? exp2i(range_exp(range_read(range))) : 1.0f;
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
    if (c < cols && r < rows) dst[(int64_t)c * ld_dst + r] = f16_rne(tile[tx][i] * sc);
  }
}

// Depthwise conv, kConvRows consecutive tokens x 8 channels per thread: a
// window of kConvRows X0 rows slides down one row per tap, so each row is
// loaded once per thread instead of once per tap. Output t sums tap k over
// k = 0, 1, ... in order while t + k is before its bound (the sequence end,
// or the end of the n_next look-ahead rows that follow it; the chunk end; the
// document end). Row r of the sequence is X0 row r for r < T and look-ahead
// row r - T of Xn after that.
constexpr int kConvRows = 8;
static_assert(kTokenPad % kConvRows == 0, "row windows tile the padded sequence");

__device__ __forceinline__ uint4 load_row8(const u16* X0, const u16* Xn, int r, int T,
                                           int n_next, int d) {
  if (r < T) return *reinterpret_cast<const uint4*>(X0 + (int64_t)r * d);
  if (r < T + n_next) return *reinterpret_cast<const uint4*>(Xn + (int64_t)(r - T) * d);
  return make_uint4(0u, 0u, 0u, 0u);
}

// Rows t .. t + kConvRows - 1 and channels c .. c + 7 of sequence b for
// thread index gid: Y = scale * conv(X0), written as fp16, and (unless yt
// is null) conv(X0) as bf16 into the slab matrix yt, sb<256>(d x B T_pad),
// token b T_pad + t (the batch's tokens one after another). Returns the
// largest |conv(X0)| (before the scale) of the thread's outputs.
template <bool TAPS_F32>
__device__ __forceinline__ float conv_rows(int64_t gid, const u16* __restrict__ X0,
                                           const u16* __restrict__ X0n, int n_next,
                                           const void* __restrict__ taps, u16* __restrict__ Y,
                                           const Dims& g, int K, int chunk, int pad_chunk,
                                           const BlockInfo* __restrict__ blocks, float scale,
                                           u16* __restrict__ yt = nullptr) {
  const int d = g.d, T = g.T;
  const int d8 = d >> 3;
  const int c = (int)(gid % d8) * 8;
  const int64_t bt = gid / d8;
  const int groups = g.T_pad / kConvRows;
  const int t = (int)(bt % groups) * kConvRows;
  const int b = (int)(bt / groups);
  const u16* xb = X0 + (int64_t)b * T * d + c;
  const u16* xn = X0n + (int64_t)b * n_next * d + c;  // not read when n_next == 0
  int end[kConvRows];
  int last = 0;
#pragma unroll
  for (int r = 0; r < kConvRows; ++r) {
    const int tr = t + r;
    end[r] = blocks != nullptr
                 ? min(T, pad_chunk ? blocks[tr >> 6].chunk_end : blocks[tr >> 6].doc_end)
                 : (pad_chunk ? min(T, (tr / chunk + 1) * chunk) : T + n_next);
    if (tr >= T) end[r] = 0;  // padding rows of Y stay zero
    last = max(last, end[r]);
  }
  float acc[kConvRows][8] = {};
  uint4 win[kConvRows];
#pragma unroll
  for (int r = 0; r < kConvRows; ++r) win[r] = load_row8(xb, xn, t + r, T, n_next, d);
  for (int k = 0; k < K && t + k < last; ++k) {
    float tp[8];
    if constexpr (TAPS_F32) {
      const float4* p =
          reinterpret_cast<const float4*>(static_cast<const float*>(taps) + (int64_t)k * d + c);
      const float4 a = p[0], bq = p[1];
      tp[0] = a.x; tp[1] = a.y; tp[2] = a.z; tp[3] = a.w;
      tp[4] = bq.x; tp[5] = bq.y; tp[6] = bq.z; tp[7] = bq.w;
    } else {
      const uint4 tv =
          *reinterpret_cast<const uint4*>(static_cast<const u16*>(taps) + (int64_t)k * d + c);
      const uint32_t tw[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tp[2 * e] = __uint_as_float(tw[e] << 16);
        tp[2 * e + 1] = __uint_as_float(tw[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int r = 0; r < kConvRows; ++r) {
      if (t + r + k < end[r]) {
        const uint32_t xw[4] = {win[r].x, win[r].y, win[r].z, win[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[r][2 * e] = fmaf(tp[2 * e], __uint_as_float(xw[e] << 16), acc[r][2 * e]);
          acc[r][2 * e + 1] =
              fmaf(tp[2 * e + 1], __uint_as_float(xw[e] & 0xffff0000u), acc[r][2 * e + 1]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r + 1 < kConvRows; ++r) win[r] = win[r + 1];
    win[kConvRows - 1] = load_row8(xb, xn, t + kConvRows + k, T, n_next, d);
  }
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < kConvRows; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(acc[r][e]));
    *reinterpret_cast<uint4*>(Y + ((int64_t)b * g.T_pad + t + r) * g.ld_y + c) =
        make_uint4(pack_f16(acc[r][0] * scale, acc[r][1] * scale),
                   pack_f16(acc[r][2] * scale, acc[r][3] * scale),
                   pack_f16(acc[r][4] * scale, acc[r][5] * scale),
                   pack_f16(acc[r][6] * scale, acc[r][7] * scale));
  }
  if (yt != nullptr) {
    static_assert(kConvRows == 8, "one 16-byte slab piece per channel");
    const int64_t kt = (int64_t)g.B * g.T_pad, k = (int64_t)b * g.T_pad + t;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint4*>(yt + sb_offset<256>(c + e, k, kt)) =
          make_uint4(pack_bf16(acc[0][e], acc[1][e]), pack_bf16(acc[2][e], acc[3][e]),
                     pack_bf16(acc[4][e], acc[5][e]), pack_bf16(acc[6][e], acc[7][e]));
  }
  return m;
}

// The conv (scale 1), noting its largest |value| in the range group (if
// not null).
template <bool TAPS_F32>
__global__ __launch_bounds__(kThreads) void conv_kernel(const u16* __restrict__ X0,
                                                        const u16* __restrict__ X0n, int n_next,
                                                        const void* __restrict__ taps,
                                                        u16* __restrict__ Y, Dims g, int K,
                                                        int chunk, int pad_chunk,
                                                        const BlockInfo* __restrict__ blocks,
                                                        int64_t total, uint32_t* __restrict__ range,
                                                        u16* __restrict__ yt) {
  // Neighbouring row windows overlap by K - 1 rows; keeping them on one XCD
  // lets the overlap come from that XCD's L2.
  const int64_t gid = (int64_t)xcd_contiguous_id() * kThreads + threadIdx.x;
  float m = 0.0f;
  if (gid < total)
    m = conv_rows<TAPS_F32>(gid, X0, X0n, n_next, taps, Y, g, K, chunk, pad_chunk, blocks, 1.0f,
                            yt);
  if (range != nullptr) range_note_block<kThreads>(range, m);
}

// Writes Y again times 2^q when the conv's noted maximum is out of the fp16
// range (q from range_exp); otherwise returns at once. A small persistent
// grid, so that the usual case costs one short launch.
template <bool TAPS_F32>
__global__ __launch_bounds__(kThreads) void conv_repair_kernel(
    const u16* __restrict__ X0, const u16* __restrict__ X0n, int n_next,
    const void* __restrict__ taps, u16* __restrict__ Y, Dims g, int K, int chunk, int pad_chunk,
    const BlockInfo* __restrict__ blocks, int64_t total, const uint32_t* __restrict__ range) {
  const int q = range_exp(range_read(range));
  if (q == 0) return;
  const float sc = exp2i(q);
  for (int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * kThreads)
    (void)conv_rows<TAPS_F32>(gid, X0, X0n, n_next, taps, Y, g, K, chunk, pad_chunk, blocks, sc);
}

// One thread per 8 packed elements, in packed (destination) order: row
// jb * 128 + r, columns kt * 64 + 8 * c8 .. + 8 of W -> slab (jb, kt).
template <bool F32>
__global__ __launch_bounds__(kThreads) void pack_weight_kernel(const void* __restrict__ W,
                                                              u16* __restrict__ dst, int f, int d,
                                                              int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int nk = d / kGateBK;
  const int c8 = (int)(i & 7), r = (int)((i >> 3) % kWRows);
  const int64_t slab = i / (8 * kWRows);
  const int kt = (int)(slab % nk), jb = (int)(slab / nk);
  const int row = jb * kWRows + r;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < f) {
    const int64_t o = (int64_t)row * d + kt * kGateBK + c8 * 8;
    if constexpr (F32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + o);
      const float4 a = p[0], b = p[1];
      v = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y),
                     pack_bf16(b.z, b.w));
    } else {
      v = *reinterpret_cast<const uint4*>(static_cast<const u16*>(W) + o);
    }
  }
  reinterpret_cast<uint4*>(dst)[i] = v;
}

__global__ __launch_bounds__(kThreads) void calibration_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst,
                                                                    int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

// ------------------------------------------------------------ launchers

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int blocks = (int)std::min<int64_t>((n16 + kThreads - 1) / kThreads, 8192);
  if (blocks > 0)
    calibration_copy_kernel<<<blocks, kThreads, 0, s>>>(static_cast<const uint4*>(src),
                                                        static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  const int blocks = (int)std::min<int64_t>((n4 + kThreads - 1) / kThreads, 65536);
  if (blocks > 0) cast_kernel<<<blocks, kThreads, 0, s>>>(src, dst, n4);
  return hipGetLastError();
}

hipError_t launch_range_clear(uint32_t* range, hipStream_t s) {
  range_clear_kernel<<<1, kThreads, 0, s>>>(range);
  return hipGetLastError();
}

hipError_t launch_amax(const void* W, bool w_f32, int64_t n, uint32_t* group, hipStream_t s) {
  const int64_t vecs = n / (w_f32 ? 4 : 8);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(vecs, kThreads), 512));
  if (w_f32)
    amax_kernel<true><<<blocks, kThreads, 0, s>>>(W, n, group);
  else
    amax_kernel<false><<<blocks, kThreads, 0, s>>>(W, n, group);
  return hipGetLastError();
}

hipError_t launch_transpose_f16(const void* src, bool src_f32, uint16_t* dst, int rows, int cols,
                                int64_t ld_dst, const uint32_t* range, hipStream_t s) {
  dim3 grid(ceil_div(cols, 64), ceil_div(rows, 64));
  if (src_f32)
    transpose_kernel<true><<<grid, kThreads, 0, s>>>(src, dst, rows, cols, ld_dst, range);
  else
    transpose_kernel<false><<<grid, kThreads, 0, s>>>(src, dst, rows, cols, ld_dst, range);
  return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* X0, const uint16_t* X0_next, int n_next,
                       const void* taps, bool taps_f32, uint16_t* Y, const Dims& g, int K,
                       int chunk, bool pad_chunk, const BlockInfo* blocks, uint32_t* range,
                       hipStream_t s, uint16_t* yt) {
  const int64_t total = (int64_t)g.B * (g.T_pad / kConvRows) * (g.d / 8);
  const int grid = ceil_div(total, kThreads);
  if (n_next == 0) X0_next = X0;  // never read
  if (taps_f32)
    conv_kernel<true><<<grid, kThreads, 0, s>>>(X0, X0_next, n_next, taps, Y, g, K, chunk,
                                                pad_chunk ? 1 : 0, blocks, total, range, yt);
  else
    conv_kernel<false><<<grid, kThreads, 0, s>>>(X0, X0_next, n_next, taps, Y, g, K, chunk,
                                                 pad_chunk ? 1 : 0, blocks, total, range, yt);
  return hipGetLastError();
}

// Compute units of the current device (256 if the query fails): the size of
// the persistent repair grids and of a launch's rounds of tiles.
int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return cus;
}

hipError_t launch_conv_repair(const uint16_t* X0, const uint16_t* X0_next, int n_next,
                              const void* taps, bool taps_f32, uint16_t* Y, const Dims& g, int K,
                              int chunk, bool pad_chunk, const BlockInfo* blocks,
                              const uint32_t* range, hipStream_t s) {
  const int64_t total = (int64_t)g.B * (g.T_pad / kConvRows) * (g.d / 8);
  const int grid = std::min<int64_t>(ceil_div(total, kThreads), 4 * device_cus());
  if (n_next == 0) X0_next = X0;  // never read
  if (taps_f32)
    conv_repair_kernel<true><<<grid, kThreads, 0, s>>>(X0, X0_next, n_next, taps, Y, g, K, chunk,
                                                       pad_chunk ? 1 : 0, blocks, total, range);
  else
    conv_repair_kernel<false><<<grid, kThreads, 0, s>>>(X0, X0_next, n_next, taps, Y, g, K,
                                                        chunk, pad_chunk ? 1 : 0, blocks, total,
                                                        range);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const void* W, bool w_f32, uint16_t* dst, const Dims& g,
                              hipStream_t s) {
  const int64_t total = wpack_elems(g) / 8;
  const int blocks = ceil_div(total, kThreads);
  if (w_f32)
    pack_weight_kernel<true><<<blocks, kThreads, 0, s>>>(W, dst, g.f, g.d, total);
  else
    pack_weight_kernel<false><<<blocks, kThreads, 0, s>>>(W, dst, g.f, g.d, total);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                          uint16_t* Z, uint16_t* ZT, const Dims& g, uint32_t* range,
                          hipStream_t s) {
  const int tiles_m = g.T_pad / K1_BM, tiles_n = ceil_div(g.f, K1_BN / 2);
  gate_up_kernel<<<tiles_m * tiles_n * g.B, 64 * K1_NW, 0, s>>>(H, Wgp, Wup, Z, ZT, g, tiles_m,
                                                              tiles_n, range);
  return hipGetLastError();
}

hipError_t launch_gate_up_bwd(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                              uint16_t* Z, uint16_t* ZT, uint32_t* sa, const Dims& g,
                              hipStream_t s) {
  const int tiles_m = g.T_pad / K1_BM, tiles_n = ceil_div(g.f, K1_BN / 2);
  gate_up_bwd_kernel<<<tiles_m * tiles_n * g.B, 64 * K1_NW, 0, s>>>(H, Wgp, Wup, Z, ZT, sa, g,
                                                                  tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gate_up_train(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                                uint16_t* Z, uint16_t* ZT, uint16_t* ZTb, uint32_t* sa,
                                const Dims& g, uint32_t* range, hipStream_t s) {
  const int tiles_m = g.T_pad / K1_BM, tiles_n = ceil_div(g.f, K1_BN / 2);
  gate_up_train_kernel<<<tiles_m * tiles_n * g.B, 64 * K1_NW, 0, s>>>(H, Wgp, Wup, Z, ZT, ZTb, sa,
                                                                    g, tiles_m, tiles_n, range);
  return hipGetLastError();
}

hipError_t launch_gate_up_repair(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                                 uint16_t* ZT, const Dims& g, const uint32_t* range,
                                 hipStream_t s) {
  const int tiles_m = g.T_pad / K1_BM, tiles_n = ceil_div(g.f, K1_BN / 2);
  const int grid = std::min(tiles_m * tiles_n * g.B, device_cus());
  gate_up_repair_kernel<<<grid, 64 * K1_NW, 0, s>>>(H, Wgp, Wup, ZT, g, tiles_m, tiles_n, range);
  return hipGetLastError();
}

hipError_t launch_target(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                         uint16_t* Vrow, float vscale, const Dims& g, uint32_t* range,
                         hipStream_t s) {
  const int tiles_m = g.T_pad / K2_BM, tiles_n = ceil_div(g.d, K2_BN);
  target_kernel<<<tiles_m * tiles_n * g.B, 64 * K2_NW, 0, s>>>(
      Y, WtT, VT, Vtok, Vrow, vscale, g, tiles_m, tiles_n, range, VT != nullptr ? 1 : 0);
  return hipGetLastError();
}

// Rounds of `tiles` workgroups on `cus` compute units.
static int rounds_of(int64_t tiles, int cus) { return (int)((tiles + cus - 1) / cus); }

bool gate_up_target_merges(const Dims& g) {
  const int cus = device_cus();
  const int64_t gu = (int64_t)(g.T_pad / K1_BM) * ceil_div(g.f, K1_BN / 2) * g.B;
  const int64_t tg = (int64_t)(g.T_pad / K2_BM) * ceil_div(g.d, K2_BN) * g.B;
  const int64_t gu8 = (gu + 7) / 8 * 8;
  return rounds_of(gu8 + tg, cus) < rounds_of(gu, cus) + rounds_of(tg, cus);
}

hipError_t launch_gate_up_target(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                                 uint16_t* Z, uint16_t* ZT, const uint16_t* Y,
                                 const uint16_t* WtT, uint16_t* VT, uint16_t* Vrow,
                                 float vscale, const Dims& g, uint32_t* range, hipStream_t s) {
  const int gtm = g.T_pad / K1_BM, gtn = ceil_div(g.f, K1_BN / 2);
  const int ttm = g.T_pad / K2_BM, ttn = ceil_div(g.d, K2_BN);
  const int n_gu = (gtm * gtn * g.B + 7) / 8 * 8;
  gate_up_target_kernel<<<n_gu + ttm * ttn * g.B, 64 * K1_NW, 0, s>>>(
      H, Wgp, Wup, Z, ZT, gtm, gtn, n_gu, Y, WtT, VT, Vrow, vscale, ttm, ttn, g, range);
  return hipGetLastError();
}

hipError_t launch_target_bwd(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                             int64_t vtok_ld, float eta, const Dims& g, const uint32_t* range,
                             hipStream_t s) {
  const int tiles_m = g.T_pad / K2_BM, tiles_n = ceil_div(g.d, K2_BN);
  target_bwd_kernel<<<tiles_m * tiles_n * g.B, 64 * K2_NW, 0, s>>>(Y, WtT, VT, Vtok, vtok_ld, eta,
                                                                 g, tiles_m, tiles_n, range);
  return hipGetLastError();
}

hipError_t launch_target_repair(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT,
                                uint16_t* Vrow, float vscale, int p, const Dims& g,
                                const uint32_t* range, hipStream_t s) {
  const int tiles_m = g.T_pad / K2_BM, tiles_n = ceil_div(g.d, K2_BN);
  const int grid = std::min(tiles_m * tiles_n * g.B, device_cus());
  target_repair_kernel<<<grid, 64 * K2_NW, 0, s>>>(Y, WtT, VT, Vrow, vscale, p, g, tiles_m,
                                                   tiles_n, range);
  return hipGetLastError();
}

int clip_pairs(int chunk) {
  const int nblk = ceil_div(chunk, KG_B);
  return nblk * (nblk + 1) / 2 * KG_SPLIT;
}

int64_t clip_gram_floats(int chunk) {
  const int nblk = ceil_div(chunk, KG_B);
  return (int64_t)(nblk * (nblk + 1) / 2) * KG_B * KG_B;
}

hipError_t launch_clip_scale(const uint16_t* Z, const uint16_t* Vrow, float* gram,
                             float* partial, float* scale, uint16_t* VT, const Dims& g,
                             int chunk, int nchunks, const ChunkSpan* spans,
                             const BlockInfo* blocks, float norm_factor, float clip,
                             const uint32_t* range, int p, hipStream_t s) {
  const int nblk = ceil_div(chunk, KG_B), npair = nblk * (nblk + 1) / 2;
  gram_v_kernel<<<g.B * nchunks * npair, KG_THREADS, 0, s>>>(Vrow, gram, g, chunk, nblk, npair,
                                                               nchunks, spans);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gram_norm_kernel<<<g.B * nchunks * npair * KG_SPLIT, KG_THREADS, 0, s>>>(
      Z, gram, partial, g, chunk, nblk, npair, nchunks, spans);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = g.B * nchunks;
  clip_scale_kernel<<<ceil_div(n, kThreads), kThreads, 0, s>>>(partial, scale, clip_pairs(chunk),
                                                               n, norm_factor, clip, range, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n16 = vt_elems(g) / 8;
  vt_scale_kernel<<<ceil_div(n16, kThreads), kThreads, 0, s>>>(VT, scale, g, chunk, nchunks,
                                                               blocks, n16);
  return hipGetLastError();
}

template <bool F32, bool PACKED, class MMA = F16Mma, bool REV = false, bool TRANS = false>
static void update_launch(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                          int64_t winit_bstride, int64_t winit_ld, int p, const uint32_t* range,
                          uint16_t* snap, int64_t snap_bstride, float* Wf, uint16_t* shadow,
                          const Dims& g, int tok_begin, int nk, int steps_per_chunk,
                          const BlockInfo* blocks, int n_chunks, hipStream_t s, int snap_k = 0) {
  // Wide tiles in whole rounds of one per compute unit; the regions left
  // over become narrow tiles when they fill at most half a round (two narrow
  // tiles then take about as long as one wide round would, with every
  // compute unit busy).
  const int regions_m = ceil_div(g.f, K3_BM), regions_n = ceil_div(g.d, K3_WIDE);
  const int regions = regions_m * regions_n * g.B;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    cus = 256;
  cus &= ~7;  // whole XCD rounds
  const int rem = regions % cus;
  const int n_wide = (rem == 0 || 2 * rem > cus) ? regions : regions - rem;
  const int grid = n_wide + 2 * (regions - n_wide);
  update_kernel<F32, PACKED, MMA, REV, TRANS><<<grid, 64 * K3_NW, 0, s>>>(
      ZT, VT, Winit, winit_bstride, winit_ld, p, range, snap, snap_bstride, Wf, shadow, g,
      tok_begin, nk, steps_per_chunk, blocks, n_chunks, regions_m, regions_n, n_wide,
      snap_k > 0 ? snap_k : g.f);
}

hipError_t launch_update(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                         bool winit_f32, int64_t winit_bstride, int64_t winit_ld, int p,
                         const uint32_t* range, uint16_t* snap, int64_t snap_bstride, float* Wf,
                         uint16_t* shadow, const Dims& g, int tok_begin, int tok_count,
                         int chunk, const BlockInfo* blocks, int n_chunks, hipStream_t s) {
  // Token offsets and counts are whole K steps, so that the slab operands are
  // read from a slab boundary.
  const int nk = (tok_count + K3_BK - 1) / K3_BK, steps_per_chunk = chunk / K3_BK;
  if (blocks != nullptr) {
    if (nk > kMaxPackedSteps) return hipErrorInvalidValue;  // StepBits holds 2048 steps
    if (winit_f32)
      update_launch<true, true>(ZT, VT, Winit, winit_bstride, winit_ld, p, range, snap,
                                snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                blocks, n_chunks, s);
    else
      update_launch<false, true>(ZT, VT, Winit, winit_bstride, winit_ld, p, range, snap,
                                 snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                 blocks, n_chunks, s);
  } else {
    if (winit_f32)
      update_launch<true, false>(ZT, VT, Winit, winit_bstride, winit_ld, p, range, snap,
                                 snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                 nullptr, n_chunks, s);
    else
      update_launch<false, false>(ZT, VT, Winit, winit_bstride, winit_ld, p, range, snap,
                                  snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                  nullptr, n_chunks, s);
  }
  return hipGetLastError();
}

hipError_t launch_contract_bf16(const uint16_t* A, const uint16_t* Bm, const Dims& g,
                                const void* Winit, bool winit_f32, bool winit_trans,
                                int64_t winit_bstride, int64_t winit_ld, uint16_t* snap,
                                int64_t snap_bstride, int snap_k, float* Wout, bool reverse,
                                int chunk, hipStream_t s) {
  const int nk = (g.T + K3_BK - 1) / K3_BK, spc = chunk / K3_BK;
#define TTT_CONTRACT(F32, REV, TRANS)                                                          \
  update_launch<F32, false, Bf16Mma, REV, TRANS>(A, Bm, Winit, winit_bstride, winit_ld, 0,     \
                                                 nullptr, snap, snap_bstride, Wout, nullptr, g, \
                                                 0, nk, spc, nullptr, 1, s, snap_k)
  if (reverse) {
    if (winit_trans) return hipErrorInvalidValue;
    if (winit_f32) TTT_CONTRACT(true, true, false); else TTT_CONTRACT(false, true, false);
  } else if (winit_trans) {
    if (winit_f32) TTT_CONTRACT(true, false, true); else TTT_CONTRACT(false, false, true);
  } else {
    if (winit_f32) TTT_CONTRACT(true, false, false); else TTT_CONTRACT(false, false, false);
  }
#undef TTT_CONTRACT
  return hipGetLastError();
}

template <int BN>
static void apply_dispatch(const uint16_t* Z, const uint16_t* snap, int64_t sb, int64_t sc,
                           void* O, bool out_f32, const Dims& g, int tok_begin, int tok_end,
                           int chunk, const ApplyTile* tiles, int n_tiles, int n_chunks,
                           hipStream_t s) {
  const int tiles_m = ceil_div(g.d, 256);
  const int tiles_n = tiles != nullptr ? n_tiles : ceil_div(tok_end - tok_begin, BN);
  const int grid = tiles_m * tiles_n * g.B;
  if (out_f32)
    apply_kernel<BN, true><<<grid, 64 * ApplyCfg<BN>::NW, 0, s>>>(Z, snap, sb, sc, O, g, tok_begin,
                                                     tok_end, chunk, tiles, n_chunks, tiles_m,
                                                     tiles_n);
  else
    apply_kernel<BN, false><<<grid, 64 * ApplyCfg<BN>::NW, 0, s>>>(Z, snap, sb, sc, O, g, tok_begin,
                                                      tok_end, chunk, tiles, n_chunks, tiles_m,
                                                      tiles_n);
}

hipError_t launch_apply(const uint16_t* Z, const uint16_t* snap, int64_t snap_bstride,
                        int64_t snap_cstride, void* O, bool out_f32, const Dims& g,
                        int tok_begin, int tok_end, int chunk, const ApplyTile* tiles,
                        int n_tiles, int n_chunks, hipStream_t s) {
  // A token tile must not straddle a chunk (it reads one snapshot): tiles
  // start at chunk starts and are apply_tile_width(chunk) wide, or narrower
  // (down to 64 tokens) when a launch without a tile list would otherwise
  // leave compute units idle, as the running schedule's one-chunk launches
  // do.
  int width = apply_tile_width(chunk);
  if (tiles == nullptr && tok_begin == 0 && tok_end == g.T && width == 256) {
    // The whole sequence: whole rounds of 256-token tiles, and the tiles
    // left over as 128-token halves when they fill at most half a round
    // (as the update's wide and narrow tiles).
    const int cus = device_cus() & ~7;
    const int tiles_m = ceil_div(g.d, 256), tiles_n = ceil_div(g.T, 256);
    const int n = tiles_m * tiles_n * g.B;
    const int rem = cus > 0 ? n % cus : 0;
    if (rem != 0 && 2 * rem <= cus && n > rem) {
      const int n_wide = n - rem, grid = n_wide + 2 * rem;
      if (out_f32)
        apply_mixed_kernel<true><<<grid, 64 * ApplyCfg<256>::NW, 0, s>>>(
            Z, snap, snap_bstride, snap_cstride, O, g, chunk, tiles_m, tiles_n, n_wide);
      else
        apply_mixed_kernel<false><<<grid, 64 * ApplyCfg<256>::NW, 0, s>>>(
            Z, snap, snap_bstride, snap_cstride, O, g, chunk, tiles_m, tiles_n, n_wide);
      return hipGetLastError();
    }
  }
  if (tiles == nullptr)
    while (width > 64 &&
           (int64_t)g.B * ceil_div(g.d, 256) * ceil_div(tok_end - tok_begin, width) < 256)
      width /= 2;
  switch (width) {
    case 256:
      apply_dispatch<256>(Z, snap, snap_bstride, snap_cstride, O, out_f32, g, tok_begin, tok_end,
                          chunk, tiles, n_tiles, n_chunks, s);
      break;
    case 128:
      apply_dispatch<128>(Z, snap, snap_bstride, snap_cstride, O, out_f32, g, tok_begin, tok_end,
                          chunk, tiles, n_tiles, n_chunks, s);
      break;
    default:
      apply_dispatch<64>(Z, snap, snap_bstride, snap_cstride, O, out_f32, g, tok_begin, tok_end,
                         chunk, tiles, n_tiles, n_chunks, s);
  }
  return hipGetLastError();
}

}  // namespace tttk
