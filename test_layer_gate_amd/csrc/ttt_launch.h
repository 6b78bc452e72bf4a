// Host-side launchers of the gfx950 kernels (internal to libttt_layer).
// Every launcher enqueues one kernel on `s` and returns hipGetLastError().
//
// Workspace layouts. Row-major ones have their *_ld row strides padded so
// that a row is an odd number of 128-byte lines, which spreads the rows of a
// tile over the L2's sets instead of stacking them in one.
// "sb<SR>" is the slab-blocked layout of a rows x K matrix (K a multiple of
// 64): the matrix is cut into SR-row x 64-column slabs, stored
// [ceil(rows/SR)][K/64] as contiguous SR * 128-byte blocks, so that one K
// step of one GEMM tile of SR rows is one slab. Inside a slab, 1 KB blocks
// [SR/32][4][2][32][8] hold 32 rows x 16 columns as two halves of 8 column
// values per row. A wave stores an MFMA accumulator tile into it transposed
// (the tile's M index becomes the column) with one contiguous 1 KB store per
// instruction, and the GEMM core reads a slab back with K contiguous in
// 16-byte pieces. Rows past `rows` in the last slab row are never written;
// they only feed GEMM outputs that are not stored.
//   Y   fp16 [B][T_pad][ld_y]   conv(X0); rows >= T are zero
//   WtT fp16 [d][ld_y]          W_target transposed: WtT[o][i] = W_target[i][o]
//   Z   bf16 [B][T][ld_z]       gated activation, token-major (the apply reads it)
//   ZT  fp16 [B] x sb<256>(f x T_pad)   the same, feature-major, for the
//                               update; tokens >= T are zero
//   VT  fp16 [B] x sb<256>(d x T_pad)   vscale * V, feature-major; tokens >= T zero
//   S   bf16 [B][k] x sb<256>(d x f)    per-chunk snapshots of the state
//   Wgp, Wup  bf16 [f_pad/128][d/64][128][64]   W_g and W_u packed for the
//                               gate/up GEMM: each (128 rows x 64 columns) block
//                               is one contiguous 16 KB slab, one K step of one
//                               tile's B operand; f_pad = f rounded up to 128,
//                               rows >= f are zero
// T_pad = T rounded up to a multiple of 256.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

constexpr int kTokenPad = 256;
constexpr int kZtSlab = 256;    // ZT slab rows = the update tile's M
constexpr int kVtSlab = 256;    // VT slab rows = the wide update tile's N
constexpr int kSnapSlab = 256;  // snapshot slab rows = the apply tile's M
constexpr int kWRows = 128;   // W_g / W_u rows per packed slab = half the gate/up tile's N
constexpr int kGateBK = 64;   // d_model elements per packed slab = one K step of gate/up

// One 64-token block of a packed sequence (documents back to back, each
// starting at a multiple of 64 tokens; chunks restart at every document
// start). Blocks at or past T carry the last chunk, no flags and ends T.
struct BlockInfo {
  int32_t chunk;      // index of the chunk holding the block = its snapshot
  int32_t flags;      // kBlockChunkStart | kBlockDocStart
  int32_t doc_end;    // first token after the block's document
  int32_t chunk_end;  // first token after the block's chunk
};
constexpr int32_t kBlockChunkStart = 1, kBlockDocStart = 2;

// One token tile of the apply: tokens [t0, t1) of chunk `chunk`, t1 - t0 at
// most the apply's tile width (apply_tile_width).
struct ApplyTile {
  int32_t t0, t1, chunk, reserved;
};

// The tokens [t0, t1) of one chunk of a packed sequence, in chunk order.
struct ChunkSpan {
  int32_t t0, t1;
};

// The apply's token-tile width for a chunk of `chunk` tokens: the largest of
// 256, 128 and 64 that divides it (the chunk is a multiple of 64).
inline int apply_tile_width(int chunk) {
  return chunk % 256 == 0 ? 256 : (chunk % 128 == 0 ? 128 : 64);
}

// n (a multiple of 64) padded so that n * 2 bytes is an odd number of
// 128-byte lines.
inline int64_t pad_ld(int64_t n) { return ((n / 64) % 2 == 0) ? n + 64 : n; }

struct Dims {
  int B, T, T_pad, d, f;
  int64_t ld_y, ld_z;
};

inline Dims make_dims(int B, int T, int d, int f) {
  Dims g;
  g.B = B;
  g.T = T;
  g.T_pad = (T + kTokenPad - 1) / kTokenPad * kTokenPad;
  g.d = d;
  g.f = f;
  g.ld_y = pad_ld(d);
  g.ld_z = pad_ld(f);
  return g;
}

// Element offset of (r, k) in an sb<SR> matrix with K columns.
template <int SR>
__host__ __device__ inline int64_t sb_offset(int64_t r, int64_t k, int64_t K) {
  static_assert(SR % 32 == 0, "slab rows");
  const int64_t slab = (r / SR) * (K >> 6) + (k >> 6);
  const int64_t rr = r % SR;
  return slab * (SR * 64) + ((rr >> 5) * 4 + ((k & 63) >> 4)) * 512 +
         (((k >> 3) & 1) * 32 + (rr & 31)) * 8 + (k & 7);
}
// Elements of an sb<SR> matrix of `rows` rows and K columns.
template <int SR>
__host__ __device__ inline int64_t sb_elems(int64_t rows, int64_t K) {
  return (rows + SR - 1) / SR * SR * K;
}
inline int64_t zt_elems(const Dims& g) { return (int64_t)g.B * sb_elems<kZtSlab>(g.f, g.T_pad); }
inline int64_t vt_elems(const Dims& g) { return (int64_t)g.B * sb_elems<kVtSlab>(g.d, g.T_pad); }
__host__ __device__ inline int64_t snap_elems(const Dims& g) {
  return sb_elems<kSnapSlab>(g.d, g.f);
}
inline int64_t wpack_elems(const Dims& g) {
  return (int64_t)((g.f + kWRows - 1) / kWRows) * kWRows * g.d;
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);

// dst[0, bytes) = src[0, bytes) with a plain 16-byte-per-thread copy.
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

// dst[c * ld_dst + r] = fp16(src[r][c]) for a rows x cols matrix (bf16 or fp32).
hipError_t launch_transpose_f16(const void* src, bool src_f32, uint16_t* dst, int rows,
                                int cols, int64_t ld_dst, hipStream_t s);

// Y[b][t][c] = fp16(sum_k taps[k][c] * X0[b][t + k][c]) over reads inside the
// sequence (or inside t's chunk when pad_chunk), for t < T_pad. The sequence
// may continue past T with n_next look-ahead rows, X0_next [B][n_next][d],
// which the reads of the sequence-padded conv reach. With blocks (packed
// documents, B = 1, n_next = 0) the reads stop at t's document end (or chunk
// end) instead.
hipError_t launch_conv(const uint16_t* X0, const uint16_t* X0_next, int n_next,
                       const void* taps, bool taps_f32, uint16_t* Y, const Dims& g, int K,
                       int chunk, bool pad_chunk, const BlockInfo* blocks, hipStream_t s);

// dst = W ([f][d], bf16 or fp32, rounded to bf16) in the packed Wgp layout.
hipError_t launch_pack_weight(const void* W, bool w_f32, uint16_t* dst, const Dims& g,
                              hipStream_t s);

// Z = SiLU(H Wg^T) * (H Wu^T) from packed Wgp / Wup: bf16 Z (token-major) and
// fp16 ZT; either may be null.
hipError_t launch_gate_up(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                          uint16_t* Z, uint16_t* ZT, const Dims& g, hipStream_t s);

// V = Y WtT^T (conv(X0) W_target): fp16 VT = vscale * V (feature-major),
// bf16 Vtok = vscale * V ([B][T][d]) and fp16 Vrow = vscale * V ([B][T_pad]
// [ld_y]); any may be null.
hipError_t launch_target(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                         uint16_t* Vrow, float vscale, const Dims& g, hipStream_t s);

// Update-norm clipping: per chunk i, scale[b][i] = min(1, clip /
// (norm_factor * ||Vrow_i^T Z_i||_F)) from the Gram form (gram: B * nchunks
// * clip_gram_floats(chunk) floats of V Gram tiles; partial: B * nchunks *
// clip_pairs(chunk) floats), then VT *= the scale of each token's chunk.
// Chunks are uniform (chunk i = tokens [i * chunk, min(T, (i + 1) * chunk)))
// when spans and blocks are null; a packed sequence (B = 1) passes its chunk
// spans (each at most `chunk` tokens) and its block table, which give each
// 64-token slab's chunk.
int clip_pairs(int chunk);
int64_t clip_gram_floats(int chunk);
hipError_t launch_clip_scale(const uint16_t* Z, const uint16_t* Vrow, float* gram,
                             float* partial, float* scale, uint16_t* VT, const Dims& g,
                             int chunk, int nchunks, const ChunkSpan* spans,
                             const BlockInfo* blocks, float norm_factor, float clip,
                             hipStream_t s);

// Fast-weight update over tokens [tok_begin, tok_begin + tok_count) (a
// multiple of 64), in 64-token steps (columns past T read as zero). acc =
// acc_scale * Winit; before each step that starts a chunk (every chunk / 64
// steps; with blocks, the blocks flagged kBlockChunkStart, after resetting
// acc to acc_scale * Winit at a kBlockDocStart), if snap != null, that
// chunk's snapshot (sb<256>(d x f), at snap + b * snap_bstride + chunk *
// snap_elems) = bf16(acc / acc_scale); then acc += the step's ZT x VT
// contraction over tokens. Finally Wf = acc /
// acc_scale (row-major [B][d][f]) and, if shadow != null, shadow =
// bf16(acc / acc_scale) (sb<256>(d x f) per sequence). tok_count may be 0. Winit element
// (b, c, j) is at b * winit_bstride + c * winit_ld + j. acc_scale must be a
// power of two (the scalings are then exact).
hipError_t launch_update(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                         bool winit_f32, int64_t winit_bstride, int64_t winit_ld,
                         float acc_scale, uint16_t* snap, int64_t snap_bstride, float* Wf,
                         uint16_t* shadow, const Dims& g, int tok_begin, int tok_count,
                         int chunk, const BlockInfo* blocks, int n_chunks, hipStream_t s);

// Decode step, gated activation: for one token per sequence (h, x0: [B][d],
// act dtype), zb[b][j] = bf16(z), column col of the chunk's Z^T (sb<256>, f
// rows, zt_cols columns, zt_bstride elements per sequence) = fp16(z), with
// z = SiLU(h_b Wg[j]) * (h_b Wu[j]); and x0 (as bf16) into row col of x0c
// [B][chunk][d].
hipError_t launch_decode_gate_up(const void* h, const void* x0, bool act_f32, const void* Wg,
                                 const void* Wu, bool w_f32, int B, int d, int f, uint16_t* zb,
                                 uint16_t* zt, int64_t zt_bstride, int zt_cols, uint16_t* x0c,
                                 int chunk, int col, hipStream_t s);
// Decode step, apply: o[b] = zb[b] S_b^T (S_b the bf16 state of sequence b,
// sb<256> d x f, s_bstride elements apart), through part
// (decode_apply_part_floats(B, d) floats); o is [B][d], bf16 or fp32.
int64_t decode_apply_part_floats(int B, int d);
hipError_t launch_decode_apply(const uint16_t* zb, const uint16_t* S, int64_t s_bstride, int B,
                               int d, int f, float* part, void* o, bool out_f32, hipStream_t s);

// O[b][t] = Z[b][t] W_i^T, where W_i is the bf16 state (sb<256>(d x f)) at
// snap + b * snap_bstride + i * snap_cstride. Without tiles: for tokens t in
// [tok_begin, tok_end), tok_begin a multiple of apply_tile_width(chunk), i =
// t / chunk. With tiles: for the n_tiles token tiles listed, i = the tile's
// chunk. Table entries (blocks, tiles) are clamped to [0, n_chunks) and to
// the sequence, so a wrong table gives wrong values, never a wild address.
hipError_t launch_apply(const uint16_t* Z, const uint16_t* snap, int64_t snap_bstride,
                        int64_t snap_cstride, void* O, bool out_f32, const Dims& g,
                        int tok_begin, int tok_end, int chunk, const ApplyTile* tiles,
                        int n_tiles, int n_chunks, hipStream_t s);

}  // namespace tttk
