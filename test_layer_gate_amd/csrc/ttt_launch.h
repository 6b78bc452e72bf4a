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

// Transposed reads of an sb<256> matrix M (R x K) as a GEMM B operand whose
// N index runs over M's columns and whose K index over M's rows (B[n][k] =
// M[k][n]). One K step is 64 rows of M (inside one 256-row slab row), one N
// tile 256 columns (four slabs): 32 KB that the sb image holds as 32
// contiguous 1 KB blocks of 32 rows x 16 columns. The direct-to-LDS loads
// copy each block whole, with its 16-byte pieces permuted so that the LDS
// transpose reads of a fragment fall on distinct banks.
//
// LDS image of one K step: element (k, n) (k < 64 the row within the step,
// n < 256 the column within the tile) in 1 KB block 2 (n / 16) + k / 32, at
// piece 32 h + ((k % 32) ^ 4 h ^ 8 ((n / 16) % 2)) with h = (n / 8) % 2,
// 2 bytes per column n % 8.
__host__ __device__ inline uint32_t slabt_lds_byte(int k, int n) {
  const int f16 = n >> 4, h = (n >> 3) & 1;
  const int pos = 32 * h + ((k & 31) ^ (4 * h) ^ (8 * (f16 & 1)));
  return (uint32_t)((2 * f16 + (k >> 5)) * 1024 + pos * 16 + (n & 7) * 2);
}
// HBM byte offset, from the tile's first column in the K step's first slab,
// of the 16-byte piece that lane `lane` of the load filling LDS block `blk`
// copies: the sb piece of row 32 (blk % 2) + r, columns 16 (blk / 2) + 8 h
// .. + 7, with h = lane / 32 and r = (lane % 32) ^ 4 h ^ 8 ((blk / 2) % 2),
// so that it lands at the LDS piece slabt_lds_byte gives it.
__host__ __device__ inline uint32_t slabt_piece_byte(int blk, int lane) {
  const int f16 = blk >> 1, g = blk & 1, h = lane >> 5;
  const int r = (lane & 31) ^ (4 * h) ^ (8 * (f16 & 1));
  return (uint32_t)((f16 >> 2) * 32768 + (g * 4 + (f16 & 3)) * 1024 + (32 * h + r) * 16);
}
// Byte offset of K step kl (rows 64 kl .. 64 kl + 63) of an sb<256> matrix
// with K columns from the matrix's first slab row.
__host__ __device__ inline uint32_t slabt_step_byte(int kl, int64_t K) {
  return (uint32_t)((int64_t)(kl >> 2) * (K >> 6) * 32768 + (kl & 3) * 8192);
}
// The LDS transpose read (ds_read_b64_tr_b16) gives lane i of each 16-lane
// group, as its element e (e = 0..3), element i % 4 of the 8-byte piece that
// lane 4e + i / 4 of the group addresses. The 32x32x16 MFMA B fragment of
// columns nb .. nb + 31 (nb a multiple of 32) and K values 8 kc .. 8 kc + 7
// (lanes 32-63 at kc + 1: kc = 2 sub + lane / 32 for the stage's K substep
// sub) is two such reads, rd = 0 for K values + 0..3 and rd = 1 for + 4..7,
// in which lane 4e + j of group G addresses row 8 kc + 4 rd + e, columns
// nb + 16 (G % 2) + 4 j .. + 3.
__host__ __device__ inline uint32_t slabt_tr_byte(int lane, int nb, int kc, int rd) {
  const int G = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
  return slabt_lds_byte(8 * kc + 4 * rd + e, nb + 16 * (G & 1) + 4 * j);
}
// slabt_tr_byte split into a per-lane part and a per-substep part:
// slabt_tr_byte(lane, nb, 2 sub + lane / 32, rd) = slabt_tr_lane(lane, nb, rd)
// + slabt_tr_sub(sub).
__host__ __device__ inline uint32_t slabt_tr_lane(int lane, int nb, int rd) {
  const int G = lane >> 4, e = (lane >> 2) & 3, j = lane & 3, h = j >> 1;
  const int f16 = (nb >> 4) + (G & 1), kh = lane >> 5;
  return (uint32_t)(f16 * 2048 + h * 512 + 128 * (kh ^ (f16 & 1)) + 64 * (rd ^ h) + 16 * e +
                    8 * (j & 1));
}
__host__ __device__ inline uint32_t slabt_tr_sub(int sub) {
  return (uint32_t)((sub >> 1) * 1024 + (sub & 1) * 256);
}

inline int64_t zt_elems(const Dims& g) { return (int64_t)g.B * sb_elems<kZtSlab>(g.f, g.T_pad); }
inline int64_t vt_elems(const Dims& g) { return (int64_t)g.B * sb_elems<kVtSlab>(g.d, g.T_pad); }
__host__ __device__ inline int64_t snap_elems(const Dims& g) {
  return sb_elems<kSnapSlab>(g.d, g.f);
}
inline int64_t wpack_elems(const Dims& g) {
  return (int64_t)((g.f + kWRows - 1) / kWRows) * kWRows * g.d;
}

// Operand ranges of the fp16 copies (ttt_device.h has the device side): a
// range buffer holds kRangeGroups groups of kRangeSlots words, each group the
// largest |value| noted by one producer (W_target, conv(X0), V at vscale, Z).
constexpr int kRangeSlots = 256;
enum { kRangeWt = 0, kRangeY = 1, kRangeV = 2, kRangeZ = 3, kRangeGroups = 4 };
constexpr int kRangeWords = kRangeGroups * kRangeSlots;
constexpr int kRangeMaxExp = 40;   // |q| limit of one operand's exponent
constexpr int kStateMaxExp = 100;  // |p + qv + qz| limit of the update's state scale

// Zeroes a range buffer (kRangeWords words); every call that uses one starts
// with it.
hipError_t launch_range_clear(uint32_t* range, hipStream_t s);
// Notes max |W| over n elements (bf16 or fp32, n a multiple of 8) in one
// range group.
hipError_t launch_amax(const void* W, bool w_f32, int64_t n, uint32_t* group, hipStream_t s);

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);

// dst[0, bytes) = src[0, bytes) with a plain 16-byte-per-thread copy.
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

// dst[c * ld_dst + r] = fp16(src[r][c] 2^q) for a rows x cols matrix (bf16
// or fp32), q from src's range group (range_exp of its noted maximum; 0 when
// range is null).
hipError_t launch_transpose_f16(const void* src, bool src_f32, uint16_t* dst, int rows,
                                int cols, int64_t ld_dst, const uint32_t* range, hipStream_t s);

// Y[b][t][c] = fp16(sum_k taps[k][c] * X0[b][t + k][c]) over reads inside the
// sequence (or inside t's chunk when pad_chunk), for t < T_pad. The sequence
// may continue past T with n_next look-ahead rows, X0_next [B][n_next][d],
// which the reads of the sequence-padded conv reach. With blocks (packed
// documents, B = 1, n_next = 0) the reads stop at t's document end (or chunk
// end) instead. The largest |Y| goes to the range group (if not null);
// launch_conv_repair then writes Y again times 2^q if that maximum is out of
// the fp16 range, and otherwise only reads the group.
hipError_t launch_conv(const uint16_t* X0, const uint16_t* X0_next, int n_next,
                       const void* taps, bool taps_f32, uint16_t* Y, const Dims& g, int K,
                       int chunk, bool pad_chunk, const BlockInfo* blocks, uint32_t* range,
                       hipStream_t s, uint16_t* yt = nullptr);
hipError_t launch_conv_repair(const uint16_t* X0, const uint16_t* X0_next, int n_next,
                              const void* taps, bool taps_f32, uint16_t* Y, const Dims& g, int K,
                              int chunk, bool pad_chunk, const BlockInfo* blocks,
                              const uint32_t* range, hipStream_t s);

// dst = W ([f][d], bf16 or fp32, rounded to bf16) in the packed Wgp layout.
hipError_t launch_pack_weight(const void* W, bool w_f32, uint16_t* dst, const Dims& g,
                              hipStream_t s);

// Z = SiLU(H Wg^T) * (H Wu^T) from packed Wgp / Wup: bf16 Z (token-major) and
// fp16 ZT; either may be null. With ZT, the largest |Z| goes to the range's
// Z group (if range is not null); launch_gate_up_repair then writes ZT again
// times 2^qz (qz = range_exp of that maximum) if qz != 0.
hipError_t launch_gate_up(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                          uint16_t* Z, uint16_t* ZT, const Dims& g, uint32_t* range,
                          hipStream_t s);
hipError_t launch_gate_up_repair(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                                 uint16_t* ZT, const Dims& g, const uint32_t* range,
                                 hipStream_t s);

// V = Y WtT^T (conv(X0) W_target): fp16 VT = vscale * V (feature-major),
// bf16 Vtok = vscale * V ([B][T][d]) and fp16 Vrow = vscale * V ([B][T_pad]
// [ld_y]); any may be null. With a range buffer, the exponents Y and WtT
// were scaled by (their groups) are divided out, and with VT the largest
// |vscale * V| goes to the V group. launch_target_repair then writes VT and
// Vrow again at vscale * 2^qv * V if qv != 0 (qv from the V and Z groups and
// eta's exponent p: the update's exponents).
hipError_t launch_target(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                         uint16_t* Vrow, float vscale, const Dims& g, uint32_t* range,
                         hipStream_t s);
hipError_t launch_target_repair(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT,
                                uint16_t* Vrow, float vscale, int p, const Dims& g,
                                const uint32_t* range, hipStream_t s);

// launch_gate_up (Z, ZT, range noted) and launch_target (VT, Vrow, range
// noted) as one launch, gate/up's tiles first; worth it only when
// gate_up_target_merges(g): the two launches' part-empty last rounds then
// share one round (each repair launch still follows).
bool gate_up_target_merges(const Dims& g);
hipError_t launch_gate_up_target(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                                 uint16_t* Z, uint16_t* ZT, const uint16_t* Y,
                                 const uint16_t* WtT, uint16_t* VT, uint16_t* Vrow,
                                 float vscale, const Dims& g, uint32_t* range, hipStream_t s);

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
// With a range buffer, norm_factor is divided by 2^qv (Vrow holds V at
// vscale * 2^qv).
hipError_t launch_clip_scale(const uint16_t* Z, const uint16_t* Vrow, float* gram,
                             float* partial, float* scale, uint16_t* VT, const Dims& g,
                             int chunk, int nchunks, const ChunkSpan* spans,
                             const BlockInfo* blocks, float norm_factor, float clip,
                             const uint32_t* range, int p, hipStream_t s);

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
// (b, c, j) is at b * winit_bstride + c * winit_ld + j. acc_scale = 2^(p +
// qv + qz): eta's exponent and, with a range buffer, the exponents ZT and
// VT carry (powers of two, so the scalings are exact).
hipError_t launch_update(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                         bool winit_f32, int64_t winit_bstride, int64_t winit_ld, int p,
                         const uint32_t* range, uint16_t* snap, int64_t snap_bstride, float* Wf,
                         uint16_t* shadow, const Dims& g, int tok_begin, int tok_count,
                         int chunk, const BlockInfo* blocks, int n_chunks, hipStream_t s);

// Decode step, gated activation: for one token per sequence (h, x0: [B][d],
// act dtype), zb[b][j] = bf16(z), row col of zc [B][chunk][f] = z (fp32),
// column col of the chunk's Z^T (sb<256>, f rows, zt_cols columns,
// zt_bstride elements per sequence) = fp16(z), with z = SiLU(h_b Wg[j]) *
// (h_b Wu[j]); the largest |z| goes to zrange's Z group; and x0 (as bf16)
// into row col of x0c [B][chunk][d].
hipError_t launch_decode_gate_up(const void* h, const void* x0, bool act_f32, const void* Wg,
                                 const void* Wu, bool w_f32, int B, int d, int f, uint16_t* zb,
                                 float* zc, uint16_t* zt, int64_t zt_bstride, int zt_cols,
                                 uint16_t* x0c, int chunk, int col, uint32_t* zrange,
                                 hipStream_t s);
// At a chunk's close: Z^T = fp16(zc 2^qz) for the chunk's columns if qz (from
// the Z group's maximum) is not 0; otherwise nothing.
hipError_t launch_decode_zt_repair(const float* zc, uint16_t* zt, int B, int f, int chunk,
                                  int64_t zt_bstride, int zt_cols, const uint32_t* zrange,
                                  hipStream_t s);
// Decode step, apply: o[b] = zb[b] S_b^T (S_b the bf16 state of sequence b,
// sb<256> d x f, s_bstride elements apart); o is [B][d], bf16 or fp32.
hipError_t launch_decode_apply(const uint16_t* zb, const uint16_t* S, int64_t s_bstride, int B,
                               int d, int f, void* o, bool out_f32, hipStream_t s);

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

// ------------------------------------------------------------ backward
// (ttt_backward.hip, and the prefill kernels' backward variants)

// The training forward's gate/up: Z and fp16 Z^T as launch_gate_up (range
// noted in range, not null), plus Z^T as bf16 slabs (ZTb) and the SiLU
// factors as launch_gate_up_bwd writes them (sa, B T_pad f words).
hipError_t launch_gate_up_train(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                                uint16_t* Z, uint16_t* ZT, uint16_t* ZTb, uint32_t* sa,
                                const Dims& g, uint32_t* range, hipStream_t s);
// gate/up for the backward: Z (bf16, token-major [B][T][ld_z]), ZT as bf16
// slabs (sb<256>(f x T_pad) per sequence), and sa (B T_pad f words in
// accumulator-fragment order, sa_frag_offset): per element the bf16 pair
// (phi(G), U phi'(G)) in the low and high halves of a word.
hipError_t launch_gate_up_bwd(const uint16_t* H, const uint16_t* Wgp, const uint16_t* Wup,
                              uint16_t* Z, uint16_t* ZT, uint32_t* sa, const Dims& g,
                              hipStream_t s);
// The target for the backward: eta * V as bf16 slabs (VT, sb<256>(d x T_pad)
// per sequence) and token-major bf16 (Vtok [B][T] rows of vtok_ld), the
// exponents of Y and WtT (range groups) divided out.
hipError_t launch_target_bwd(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                             int64_t vtok_ld, float eta, const Dims& g, const uint32_t* range,
                             hipStream_t s);
// A contraction over tokens on the update kernel, bf16 operands: for each
// sequence b, the state S[c][j] (j < g.f rows of the slab matrix A, c < g.d
// rows of the slab matrix Bm, both sb<256>(rows x T_pad) per sequence)
// starts at Winit (null: zero; element (c, j) at Winit + b * winit_bstride +
// c * winit_ld + j, or j * winit_ld + c with winit_trans), accumulates
// sum_t A[j][t] Bm[c][t] over the tokens (backwards with reverse), stores
// bf16 snapshots at chunk boundaries as the prefill's update does (unless
// snap is null; in reverse, chunk i's snapshot is the state after every
// later chunk) and, unless Wout is null, the final fp32 state [B][g.d][g.f].
// The snapshots are sb<256>(g.d x snap_k) matrices (snap_k >= g.f; the
// state fills their first g.f columns), snap_bstride elements per sequence.
hipError_t launch_contract_bf16(const uint16_t* A, const uint16_t* Bm, const Dims& g,
                                const void* Winit, bool winit_f32, bool winit_trans,
                                int64_t winit_bstride, int64_t winit_ld, uint16_t* snap,
                                int64_t snap_bstride, int snap_k, float* Wout, bool reverse,
                                int chunk, hipStream_t s);
// dZ for every chunk as one contraction over K = 2d: dZ_i = [dO_i | eta V_i]
// [W_i^T | Gbar_{i+1}^T]^T, the token-major bf16 operand [B][T][lda] holding
// dO in columns [0, d) and eta V in [d, 2d); the chunk's bf16 state W_i and
// state gradient Gbar_{i+1}, sb<256>(d x f) matrices as the update's
// snapshots, at W + b * w_sbs + i * w_scs and Gs + b * g_sbs + i * g_scs,
// read transposed as they are (d == g.d, f == g.f, and a matrix under
// 2 GiB); the SiLU's backward in the epilogue: dG = dZ U phi'(G), dU = dZ
// phi(G) from sa, written token-major into dgu ([B][T][ld_gu]: dG of feature
// c in column 2c, dU in 2c + 1) and as bf16 slabs dgt, dut (sb<256>(f x
// B T_pad), token b T_pad + t).
hipError_t launch_act_gemm_dz(const uint16_t* dOV, int64_t lda, const uint16_t* W, int64_t w_sbs,
                              int64_t w_scs, const uint16_t* Gs, int64_t g_sbs, int64_t g_scs,
                              int d, int f, int chunk, int n_chunks, const uint32_t* sa,
                              uint16_t* dgu, int64_t ld_gu, uint16_t* dgt, uint16_t* dut,
                              const Dims& g, hipStream_t s);
// dV_i = eta Z_i Gbar_{i+1}^T for every chunk, Gbar as bf16 sb<256>(d x f)
// snapshots: token-major bf16 dv ([B][T][ld_dv]) and slabs dvt
// (sb<256>(d x B T_pad)).
hipError_t launch_act_gemm_dv(const uint16_t* Z, int64_t ldz, const uint16_t* G, int64_t sbs,
                              int64_t scs, int d, int f, int chunk, int n_chunks, float eta,
                              uint16_t* dv, int64_t ld_dv, uint16_t* dvt, const Dims& g,
                              hipStream_t s);
// out[b][t][n] = sum_k A[b][t][k] Bm[n][k], bf16 operands, fp32 output.
hipError_t launch_nt_gemm(const uint16_t* A, int64_t lda, const uint16_t* Bm, int64_t ldb, int N,
                          int K, float* out, int64_t ldo, const Dims& g, hipStream_t s);
// Token-major [B][T][ld_src] (bf16 or fp32, D features) to bf16 slabs:
// sb<256>(D x T_pad) per sequence, or with flat sb<256>(D x B T_pad).
hipError_t launch_to_slab(const void* src, bool src_f32, int64_t ld_src, uint16_t* dst, int B,
                          int T, int T_pad, int D, bool flat, hipStream_t s);
// dst[c * ld_dst + r * step] = bf16(src[r][c]) for a rows x cols matrix.
hipError_t launch_transpose_bf16(const void* src, bool src_f32, uint16_t* dst, int rows,
                                 int cols, int64_t ld_dst, int step, hipStream_t s);
// dst[r][c] (row stride ld_dst) = bf16(src[r][c]) (row stride ld_src; bf16
// or fp32) for rows x cols (cols a multiple of 8).
hipError_t launch_rows_bf16(const void* src, bool src_f32, int64_t ld_src, uint16_t* dst,
                            int64_t ld_dst, int64_t rows, int cols, hipStream_t s);
// The conv's backward from dY (fp32 [B][T][d]) and the bf16 X0 [B][T][d]:
// dX0 (fp32 [B][T][d]) and dtaps (fp32 [K][d], over the batch), through part
// (conv_bwd_part_floats floats).
int64_t conv_bwd_part_floats(int B, int T, int K, int d);
hipError_t launch_conv_bwd(const float* dY, const uint16_t* X0, const void* taps, bool taps_f32,
                           float* dX0, float* dtaps, float* part, int B, int T, int d, int K,
                           int chunk, bool pad_chunk, hipStream_t s);
// out[i] = sum over p < n_parts of in[p * stride + i], in order.
hipError_t launch_sum_parts(const float* in, int64_t stride, int n_parts, float* out, int64_t n,
                            hipStream_t s);

}  // namespace tttk
