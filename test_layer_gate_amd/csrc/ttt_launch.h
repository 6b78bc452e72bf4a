// Host-side launchers of the gfx950 kernels (internal to libttt_layer).
// Every launcher enqueues one kernel on `s` and returns hipGetLastError().
// Layouts (row-major, bf16 stored as uint16_t bit patterns):
//   Y   [B][T_pad][d]   conv(X0), rows >= T are zero
//   WtT [d][d]          W_target transposed: WtT[o][i] = W_target[i][o]
//   Z   [B][T][f]       gated activation, token-major
//   ZT  [B][f][T_pad]   the same, feature-major, columns >= T are zero
//   VT  [B][d][T_pad]   eta * target, feature-major, columns >= T are zero
//   W   [B][d][f]       fast-weight state (fp32) and its bf16 snapshots
// T_pad = T rounded up to a multiple of 256.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

constexpr int kTokenPad = 256;

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n,
                            hipStream_t s);

// dst[c][r] = bf16(src[r][c]) for a rows x cols matrix.
hipError_t launch_transpose(const void* src, bool src_f32, uint16_t* dst,
                            int rows, int cols, hipStream_t s);

// Y[b][t][c] = sum_k taps[k][c] * X0[b][t + k][c] over reads inside the
// sequence (or inside t's chunk when pad_chunk), for t < T_pad.
hipError_t launch_conv(const uint16_t* X0, const void* taps, bool taps_f32,
                       uint16_t* Y, int B, int T, int T_pad, int d, int K,
                       int chunk, bool pad_chunk, hipStream_t s);

// Z = SiLU(H Wg^T) * (H Wu^T). Z (token-major, T rows) and/or ZT may be null.
hipError_t launch_gate_up(const uint16_t* H, const uint16_t* Wg,
                          const uint16_t* Wu, uint16_t* Z, uint16_t* ZT,
                          int B, int T, int T_pad, int d, int f, hipStream_t s);

// V = scale * (Y WtT^T). VT (feature-major) and/or Vtok ([B][T][d]) may be null.
hipError_t launch_target(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT,
                         uint16_t* Vtok, float scale, int B, int T, int T_pad,
                         int d, hipStream_t s);

// Fast-weight update over tokens [tok_begin, tok_begin + 64 * nk):
// acc = Winit; for each 64-token step kt: if snap and kt % steps_per_chunk
// == 0, snap[kt / steps_per_chunk] = bf16(acc); acc += ZT^T-slice x VT-slice.
// Then Wf = acc (fp32) and, if shadow, shadow = bf16(acc). nk may be 0.
hipError_t launch_update(const uint16_t* ZT, const uint16_t* VT,
                         const void* Winit, bool winit_f32,
                         int64_t winit_bstride, uint16_t* snap,
                         int64_t snap_bstride, float* Wf, uint16_t* shadow,
                         int B, int T_pad, int d, int f, int tok_begin, int nk,
                         int steps_per_chunk, hipStream_t s);

// O[b][t] = Z[b][t] W_i^T for tokens t in [tok_begin, tok_end), where W_i is
// the bf16 state at snap + b * snap_bstride + (t / chunk) * snap_cstride.
hipError_t launch_apply(const uint16_t* Z, const uint16_t* snap,
                        int64_t snap_bstride, int64_t snap_cstride, void* O,
                        bool out_f32, int B, int T, int d, int f, int tok_begin,
                        int tok_end, int chunk, hipStream_t s);

}  // namespace tttk
