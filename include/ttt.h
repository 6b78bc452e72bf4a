/*
 * ttt.h - C ABI of the In-Place TTT fast-weight gated-MLP prefill for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (page citations name the page title and the section / equation):
 *   Z   = SiLU(H Wg^T) * (H Wu^T)
 *         "论文精读：In-Place Test-Time Training" reading notes, "In-Place 设计",
 *         gated-MLP equation: W_gate and W_up are frozen, W_down is the fast
 *         weight.
 *   V   = Conv1D(X0) W_target, a depthwise conv whose tap k reads X0[t + k]
 *         reading notes, "LM-Aligned 目标函数", target equation; zhichai
 *         summary "In-Place TTT: ByteDance Seed's Test-Time Training Framework
 *         Gives LLMs On-the-Fly Memory", "Three Core Designs" 3 (taps
 *         [0, 1, 0, ...] with W_target = I give the next token's embedding).
 *   for each chunk i of C tokens, in order:
 *     O_i      = Z_i W^(i)^T                       (apply with the pre-update state)
 *     W^(i+1)  = W^(i) + eta * V_i^T Z_i            (then update)
 *         reading notes, "Chunk-Wise 更新机制", update equation; iplexlaw
 *         explainer of In-Place Test-Time Training, §3 (apply, then update)
 *         and §6 (the exclusive prefix scan over chunk deltas, and the state
 *         starting from the pretrained W_down for every document).
 *   W^(0) = W_down0 for every sequence of the batch; the call returns every
 *   O and the final state W^(k) (after the last chunk's update).
 *
 * Layouts are row-major. Sizes: B batch, T tokens, d = d_model, f = d_ff,
 * K conv taps, C chunk, k = ceil(T / C) chunks.
 *
 * Memory ownership: every pointer argument is device memory owned by the
 * caller. The library never allocates or frees device memory in these calls;
 * scratch space is the caller's workspace of ttt_workspace_size() bytes.
 * Inputs are only read. Calls are asynchronous on the given HIP stream
 * (a hipStream_t passed as void*, NULL = the default stream) and never
 * synchronise the device; results are valid after the stream completes.
 *
 * Errors: every argument is checked on the host before anything is
 * launched; on an error nothing is launched and no output is written.
 * Launch failures return TTT_ERR_HIP. ttt_last_error() gives a
 * human-readable reason for the most recent failure on the calling thread.
 * NaN and Inf inputs are propagated, not checked. The library keeps no
 * global state other than the optional per-launch timing record
 * (ttt_profile_*), which is not thread-safe.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ttt_status {
  TTT_OK = 0,
  TTT_ERR_INVALID_ARG = -1, /* bad size, null or misaligned pointer, bad flag */
  TTT_ERR_UNSUPPORTED = -2, /* valid for the method, not supported by the kernels */
  TTT_ERR_WORKSPACE = -3,   /* workspace smaller than ttt_workspace_size() */
  TTT_ERR_ALIAS = -4,       /* an output overlaps an input, the other output or the workspace */
  TTT_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} ttt_status;

typedef enum ttt_dtype { TTT_BF16 = 0, TTT_F32 = 1 } ttt_dtype;

enum {
  /* Chunk-local conv padding: the conv of a token reads no row past the end
   * of the token's own chunk (iplexlaw explainer §6, chunk boundaries must
   * not let the target pull future information from other chunks). Without
   * the flag, rows past the end of the sequence read as zero. */
  TTT_FLAG_PAD_CHUNK = 1u << 0,
  /* Chunk schedule. Default (neither flag) is the materialised exclusive
   * prefix: one update launch over the whole sequence writes a bf16 snapshot
   * of W^(i) for every chunk, then one apply launch covers every chunk.
   * RUNNING keeps one fp32 state and alternates apply / update per chunk. */
  TTT_FLAG_SCHED_RUNNING = 1u << 1,
  TTT_FLAG_SCHED_PREFIX = 1u << 2
};

typedef struct ttt_desc {
  int32_t batch;       /* B >= 1 */
  int32_t seq_len;     /* T >= 1 */
  int32_t d_model;     /* d: multiple of 64 */
  int32_t d_ff;        /* f: multiple of 64 */
  int32_t conv_k;      /* K: 1 .. 64 */
  int32_t act_dtype;   /* ttt_dtype of H, X0 and O */
  int32_t weight_dtype;/* ttt_dtype of Wg, Wu, W_down0, taps, W_target */
  int32_t reserved;    /* must be 0 */
  int64_t w0_batch_stride; /* elements between sequences' W_down0; 0 = one shared [d, f] */
  uint32_t flags;      /* TTT_FLAG_* */
  uint32_t reserved2;  /* must be 0 */
} ttt_desc;

/* Workspace bytes ttt_layer_forward needs for this descriptor and chunk.
 * Host only. Returns TTT_OK and writes *bytes, or an error for an invalid
 * descriptor. */
ttt_status ttt_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes);

/* The layer's prefill.
 *   H         [B, T, d]  act_dtype   hidden states entering the MLP
 *   X0        [B, T, d]  act_dtype   token embeddings
 *   Wg, Wu    [f, d]     weight_dtype frozen gate / up projections
 *   W_down0   [d, f]     weight_dtype (one per sequence at w0_batch_stride)
 *   conv_taps [K, d]     weight_dtype depthwise taps, tap k reads X0[t + k]
 *   W_target  [d, d]     weight_dtype row = input channel, V = conv(X0) W_target
 *   eta                  update step, finite
 *   chunk                C: a multiple of 64, >= 64
 *   O         [B, T, d]  act_dtype   out
 *   W_down_final [B, d, f] float32   out, the state after the last chunk
 *   workspace            >= ttt_workspace_size() bytes, 256-byte aligned
 * Every pointer must be 16-byte aligned. Arithmetic: every contraction
 * accumulates in fp32. The gate/up projection and the apply take bf16
 * operands: Z is stored in bf16 token-major for the apply, which reads a bf16
 * copy of each chunk's state. The target and the update take fp16 operands
 * (3 more mantissa bits, for the fp32 state's accuracy): conv(X0) and
 * W_target^T for the target, a feature-major fp16 copy of Z and eta * V for
 * the update. Those fp16 copies are kept in fp16's range whatever the
 * inputs' magnitudes: each producer notes its largest |value|, and a copy
 * whose maximum falls outside [2^-10, 65504] is written again times a power
 * of two that brings it to [2^14, 2^15), which its consumers divide back out
 * (exact). The state is fp32 throughout; O is act_dtype. */
ttt_status ttt_layer_forward(const ttt_desc* desc,
                             const void* H, const void* X0,
                             const void* Wg, const void* Wu,
                             const void* W_down0, const void* conv_taps,
                             const void* W_target, float eta, int32_t chunk,
                             void* O, float* W_down_final,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* The prefill without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc). It is ttt_layer_forward with its
 * workspace in a static device array of TTT_NOALLOC_SCRATCH_BYTES bytes that
 * the library's code object reserves on every device it runs on, for the
 * life of the process; the call itself allocates nothing.
 *   Arguments, layouts, flags and results are ttt_layer_forward's, minus
 *   the workspace. Problems whose ttt_workspace_size exceeds the scratch
 *   return TTT_ERR_WORKSPACE before anything is launched (64 MiB holds, for
 *   instance, 2048 tokens at d_model 256 / d_ff 1024; the Qwen3-4B shapes
 *   need the caller-workspace entry point).
 *   Every call on one GPU uses that GPU's one scratch array, which keeps
 *   the previous call's contents (nothing in it needs to start at zero):
 *   calls that overlap in time on one GPU (on different streams, or from
 *   different threads) race on it and must be serialised by the caller.
 * The device address of each GPU's array is looked up on the first call on
 * that device (TTT_ERR_HIP if the lookup fails). */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ttt_status ttt_layer_forward_noalloc(const ttt_desc* desc,
                                     const void* H, const void* X0,
                                     const void* Wg, const void* Wu,
                                     const void* W_down0, const void* conv_taps,
                                     const void* W_target, float eta, int32_t chunk,
                                     void* O, float* W_down_final, void* stream);

/* Update-norm clipping (iplexlaw explainer §6: the Frobenius norm of the
 * update delta is limited to a threshold): as ttt_layer_forward, except that
 * every chunk's update eta * V_i^T Z_i is first scaled by
 * min(1, clip_norm / ||eta * V_i^T Z_i||_F).
 *   clip_norm   > 0 and finite (TTT_ERR_INVALID_ARG otherwise)
 * The norms come from the chunk's C x C Gram matrices of Z (bf16) and V
 * (fp16), so each scale carries their rounding (relative ~1e-3). The
 * workspace (ttt_clipped_workspace_size) also holds a token-major copy of V,
 * the V Gram tiles (256 KB per pair of 256-token blocks of a chunk: 2.5 MB a
 * chunk at C = 1024) and the per-chunk norms. Every other argument, layout
 * and convention is ttt_layer_forward's. */
ttt_status ttt_clipped_workspace_size(const ttt_desc* desc, int32_t chunk, float clip_norm,
                                      size_t* bytes);
ttt_status ttt_layer_forward_clipped(const ttt_desc* desc,
                                     const void* H, const void* X0,
                                     const void* Wg, const void* Wu,
                                     const void* W_down0, const void* conv_taps,
                                     const void* W_target, float eta, int32_t chunk,
                                     float clip_norm, void* O, float* W_down_final,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Packed documents: one sequence (batch must be 1) holding n_docs
 * documents back to back, document r starting at token doc_starts[r]
 * (iplexlaw explainer §6: the fast weight returns to the pretrained W_down
 * at every document boundary, so documents do not leak into each other).
 * Each document is processed as its own sequence: the state starts from
 * W_down0, the chunks of C tokens are counted from the document's start
 * (its last chunk may be shorter), and the conv reads no row past the
 * document's end (nor past the chunk's end with TTT_FLAG_PAD_CHUNK).
 *   doc_starts  host array of n_docs int32: 0 = doc_starts[0] < doc_starts[1]
 *               < ... < seq_len, every entry a multiple of 64
 *               (TTT_ERR_UNSUPPORTED otherwise); read during the call only
 *   W_down_final [d, f] float32 out: the state after the last document
 * Everything else as ttt_layer_forward; the workspace also holds a small
 * per-64-token table, copied from the host with hipMemcpyAsync on the
 * stream (staged from pageable memory before the call returns). */
ttt_status ttt_packed_workspace_size(const ttt_desc* desc, int32_t chunk,
                                     const int32_t* doc_starts, int32_t n_docs,
                                     size_t* bytes);
ttt_status ttt_layer_forward_packed(const ttt_desc* desc,
                                    const void* H, const void* X0,
                                    const void* Wg, const void* Wu,
                                    const void* W_down0, const void* conv_taps,
                                    const void* W_target, float eta, int32_t chunk,
                                    const int32_t* doc_starts, int32_t n_docs,
                                    void* O, float* W_down_final,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* The tables ttt_layer_forward_packed builds on the host for a layout and
 * copies to its workspace (host only: no GPU call, nothing launched). For
 * inspecting and testing a layout; the same checks as
 * ttt_packed_workspace_size apply.
 *   blocks  out, one entry per 64-token block of the sequence padded to 256
 *           tokens: the chunk holding the block (chunks counted over all
 *           documents, in order), flags (TTT_BLOCK_CHUNK_START when a chunk
 *           starts at the block, TTT_BLOCK_DOC_START when a document does),
 *           and the first token after the block's document and after its
 *           chunk. Blocks at or past seq_len carry the last chunk, no flags
 *           and ends seq_len.
 *   tiles   out, the apply's token tiles: tokens [t0, t1) of one chunk, read
 *           against snapshot slot `snapshot` (0 for a document's first chunk,
 *           whose state is W_down0 like the first document's).
 *   counts  out, 3 int32: entries of blocks, entries of tiles, chunks.
 * At most max_blocks / max_tiles entries are written (counts has the full
 * numbers either way); blocks / tiles may be NULL when their max is 0. */
enum { TTT_BLOCK_CHUNK_START = 1, TTT_BLOCK_DOC_START = 2 };
typedef struct ttt_packed_block {
  int32_t chunk, flags, doc_end, chunk_end;
} ttt_packed_block;
typedef struct ttt_packed_tile {
  int32_t t0, t1, snapshot, reserved;
} ttt_packed_tile;
ttt_status ttt_packed_tables(const ttt_desc* desc, int32_t chunk, const int32_t* doc_starts,
                             int32_t n_docs, ttt_packed_block* blocks, int32_t max_blocks,
                             ttt_packed_tile* tiles, int32_t max_tiles, int32_t* counts);

/* Packed documents with update-norm clipping (iplexlaw explainer §6, both
 * the document reset and the norm clipping): ttt_layer_forward_packed,
 * where each chunk's update is first scaled as in ttt_layer_forward_clipped.
 * A chunk never spans two documents, so each document's chunks are clipped
 * as they would be if that document ran alone.
 *   clip_norm   > 0 and finite (TTT_ERR_INVALID_ARG otherwise)
 * Arguments, layout, errors and workspace use as ttt_layer_forward_packed;
 * the workspace (ttt_packed_clipped_workspace_size) adds the clipped path's
 * buffers. */
ttt_status ttt_packed_clipped_workspace_size(const ttt_desc* desc, int32_t chunk,
                                             const int32_t* doc_starts, int32_t n_docs,
                                             float clip_norm, size_t* bytes);
ttt_status ttt_layer_forward_packed_clipped(const ttt_desc* desc,
                                            const void* H, const void* X0,
                                            const void* Wg, const void* Wu,
                                            const void* W_down0, const void* conv_taps,
                                            const void* W_target, float eta, int32_t chunk,
                                            const int32_t* doc_starts, int32_t n_docs,
                                            float clip_norm, void* O, float* W_down_final,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* Continuation: the next segment of sequences whose earlier tokens went
 * through a previous call. The fast weight keeps changing over a whole
 * document and is reset only at its end (iplexlaw explainer §6 and §8), so
 * a long document may be prefilled in segments: each segment starts from the
 * state the previous one ended with, and its conv reads the first rows of
 * the next segment exactly as one call over the whole document would. Split
 * at a multiple of C, two calls give the one-call result.
 *   X0_next   [B, n_next, d] act_dtype: X0 rows T .. T + n_next - 1 of each
 *             sequence (the next segment's first tokens); 0 <= n_next <=
 *             K - 1 (TTT_ERR_INVALID_ARG otherwise). Ignored, and may be
 *             NULL, when n_next is 0. The conv reads rows past T + n_next as
 *             zero (with TTT_FLAG_PAD_CHUNK it never reads past T).
 *   W_state   [B, d, f] float32 in/out: the state before the segment (for
 *             the first segment, W_down0 widened to fp32, one per sequence),
 *             overwritten in place with the state after its last chunk. It
 *             must not overlap any other argument (TTT_ERR_ALIAS).
 *   desc->w0_batch_stride must be 0 (W_state is always [B, d, f]).
 * The workspace size comes from ttt_continue_workspace_size(). Every other
 * argument, layout and convention is ttt_layer_forward's. */
ttt_status ttt_continue_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes);
ttt_status ttt_layer_forward_continue(const ttt_desc* desc,
                                      const void* H, const void* X0,
                                      const void* X0_next, int32_t n_next,
                                      const void* Wg, const void* Wu,
                                      float* W_state, const void* conv_taps,
                                      const void* W_target, float eta, int32_t chunk,
                                      void* O, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Decode: the layer one token at a time, for B sequences together.
 * Within a chunk every output uses the state from before the chunk's update
 * (iplexlaw explainer §3); with the chunk-boundary padding of §6 a chunk's
 * target reads only the chunk's own tokens, so the update is taken as soon
 * as the chunk's last token has been processed, and decoding a document
 * token by token gives the prefill's outputs and states. Sequence padding
 * would need tokens not decoded yet, so the decode entry points require
 * TTT_FLAG_PAD_CHUNK (TTT_ERR_UNSUPPORTED otherwise).
 *   desc       seq_len must be 1 (one token per sequence per step);
 *              w0_batch_stride must be 0
 *   decode_state  device buffer of ttt_decode_state_size() bytes, 256-byte
 *              aligned, owned by the caller: the bf16 copy of each state the
 *              apply reads, the open chunk's activations and X0 rows, and
 *              scratch. One buffer per group of B sequences decoded together.
 *   W_state    [B, d, f] float32, in/out, the fast weight of each sequence.
 * ttt_decode_begin starts decoding at a chunk boundary (a document start, or
 * after ttt_layer_forward_continue on a prefix whose length is a multiple
 * of C): it writes the bf16 copy of W_state into decode_state.
 * ttt_decode_step processes the token at document position pos (the same
 * for every sequence; positions must follow one another from the boundary
 * ttt_decode_begin was called at, as the open chunk's rows are kept in
 * decode_state):
 *   h, x0      [B, d] act_dtype, the token's hidden state and embedding
 *   Wg, Wu, conv_taps, W_target   as in ttt_layer_forward
 *   o          [B, d] act_dtype out: z W^T with the current state
 * When pos closes a chunk (pos % C == C - 1), the step also takes the
 * chunk's update: W_state is updated in place and its bf16 copy refreshed.
 * Arguments are checked as in ttt_layer_forward; o, W_state and
 * decode_state may not overlap an input or each other (TTT_ERR_ALIAS). */
ttt_status ttt_decode_state_size(const ttt_desc* desc, int32_t chunk, size_t* bytes);
ttt_status ttt_decode_begin(const ttt_desc* desc, int32_t chunk, float* W_state,
                            void* decode_state, size_t decode_state_bytes, void* stream);
ttt_status ttt_decode_step(const ttt_desc* desc, const void* h, const void* x0,
                           const void* Wg, const void* Wu, const void* conv_taps,
                           const void* W_target, float eta, int32_t chunk, int32_t pos,
                           float* W_state, void* decode_state, size_t decode_state_bytes,
                           void* o, void* stream);

/* The backward pass: the gradients of the prefill (ttt_layer_forward with
 * the same arguments) for training the layer. The pages train it by
 * continual pretraining (iplexlaw explainer §2 and §7.1; zhichai summary,
 * "Limitations"), and the conv taps and W_target act on the output only
 * through the fast-weight updates (§6 initialises them so that the first
 * updates are near zero), so the gradients are taken through the chunk
 * recurrence. For upstream gradients dO = dL/dO and dW_final = dL/dW_final,
 * with Gbar = dL/dW^(i+1) (dW_final after the last chunk), chunk by chunk
 * from the last:
 *   dZ_i = dO_i W^(i) + eta V_i Gbar,  dV_i = eta Z_i Gbar^T,
 *   dL/dW^(i) = Gbar + dO_i^T Z_i,     dW_down0 = dL/dW^(0);
 * then dY = dV W_target^T, dW_target = Y^T dV (Y = conv(X0)), the conv's
 * transpose for dX0 and dtaps, and dG = dZ U phi'(G), dU = dZ phi(G) (G, U
 * the gate and up projections, phi = SiLU), dH = dG Wg + dU Wu,
 * dWg = dG^T H, dWu = dU^T H. eta is a fixed scalar and gets no gradient.
 *   H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, chunk: as in
 *             ttt_layer_forward (flags: TTT_FLAG_PAD_CHUNK as there; the
 *             schedule flags are ignored). A per-sequence W_down0 must sit
 *             at w0_batch_stride = d_model * d_ff (TTT_ERR_UNSUPPORTED
 *             otherwise).
 *   dO        [B, T, d]  act_dtype   upstream gradient of O
 *   dW_final  [B, d, f]  float32     upstream gradient of W_down_final, or
 *             NULL (zero)
 *   dH, dX0   [B, T, d]  float32     out
 *   dWg, dWu  [f, d]     float32     out, summed over the batch
 *   dW_down0  float32 out: [d, f] summed over the batch for a shared
 *             W_down0, [B, d, f] for per-sequence ones
 *   dtaps     [K, d]     float32     out, summed over the batch
 *   dW_target [d, d]     float32     out, summed over the batch
 *   workspace >= ttt_backward_workspace_size() bytes, 256-byte aligned
 * Arithmetic: the forward's activations are recomputed; every contraction
 * of the backward takes bf16 operands with fp32 accumulation, and the
 * states W^(i) and gradients Gbar of the chunks are kept as bf16 copies
 * (each gradient carries bf16-level error, about 1e-3 relative). The
 * workspace holds three sets of per-chunk d x f copies (6 k d f bytes per
 * sequence) besides activation-sized buffers. Conventions (validation before
 * any launch, asynchrony, no allocation, aliasing) as ttt_layer_forward. */
ttt_status ttt_backward_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes);
ttt_status ttt_layer_backward(const ttt_desc* desc,
                              const void* H, const void* X0,
                              const void* Wg, const void* Wu,
                              const void* W_down0, const void* conv_taps,
                              const void* W_target, float eta, int32_t chunk,
                              const void* dO, const float* dW_final,
                              float* dH, float* dX0, float* dWg, float* dWu,
                              float* dW_down0, float* dtaps, float* dW_target,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Training: the prefill that keeps what its backward reads, and that
 * backward. A training step recomputes nothing: ttt_layer_forward_train is
 * ttt_layer_forward (prefix schedule only: TTT_ERR_UNSUPPORTED with
 * TTT_FLAG_SCHED_RUNNING) whose workspace of ttt_train_workspace_size()
 * bytes, once the call has run, holds the chunks' states W^(i) (bf16), Z,
 * Z^T and the SiLU factors; ttt_layer_backward_saved takes that workspace
 * as `saved` (saved_bytes >= ttt_train_workspace_size()) with the same
 * descriptor, chunk and inputs, and returns what ttt_layer_backward
 * returns, without the gate/up recompute and the state scan (W^(i) comes
 * from the forward's snapshots: the forward's update precision, so its
 * gradients differ from ttt_layer_backward's in the last bf16 bits). The
 * caller keeps `saved` unchanged between the two calls; the backward only
 * reads it. Its own workspace is ttt_backward_saved_workspace_size() bytes.
 * Other conventions as ttt_layer_forward and ttt_layer_backward. */
ttt_status ttt_train_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes);
ttt_status ttt_layer_forward_train(const ttt_desc* desc,
                                   const void* H, const void* X0,
                                   const void* Wg, const void* Wu,
                                   const void* W_down0, const void* conv_taps,
                                   const void* W_target, float eta, int32_t chunk,
                                   void* O, float* W_down_final,
                                   void* workspace, size_t workspace_bytes, void* stream);
ttt_status ttt_backward_saved_workspace_size(const ttt_desc* desc, int32_t chunk,
                                             size_t* bytes);
ttt_status ttt_layer_backward_saved(const ttt_desc* desc,
                                    const void* H, const void* X0,
                                    const void* Wg, const void* Wu,
                                    const void* W_down0, const void* conv_taps,
                                    const void* W_target, float eta, int32_t chunk,
                                    const void* saved, size_t saved_bytes,
                                    const void* dO, const float* dW_final,
                                    float* dH, float* dX0, float* dWg, float* dWu,
                                    float* dW_down0, float* dtaps, float* dW_target,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Step entry points: one step of the layer each, for per-step checks.
 * ttt_gated_activation writes Z [B, T, d_ff] in bf16.
 * ttt_lm_target writes V [B, T, d_model] in bf16 (unscaled, eta not applied).
 * Workspace sizes come from ttt_step_workspace_size(). Same conventions as
 * ttt_layer_forward. */
ttt_status ttt_step_workspace_size(const ttt_desc* desc, size_t* bytes);
ttt_status ttt_gated_activation(const ttt_desc* desc, const void* H,
                                const void* Wg, const void* Wu, void* Z,
                                void* workspace, size_t workspace_bytes,
                                void* stream);
ttt_status ttt_lm_target(const ttt_desc* desc, const void* X0,
                         const void* conv_taps, const void* W_target, int32_t chunk,
                         void* V, void* workspace, size_t workspace_bytes,
                         void* stream);

/* The name of a status code ("TTT_OK", "TTT_ERR_INVALID_ARG", ...; codes
 * outside ttt_status give "TTT_ERR_UNKNOWN"). The string is static. */
const char* ttt_status_string(int32_t status);
/* The reason for the most recent failed call on the calling thread
 * (thread-local; valid until that thread's next call into the library).
 * ttt_last_error_message is the same function under a second name. */
const char* ttt_last_error(void);
const char* ttt_last_error_message(void);

/* Optional per-launch timing. While enabled, every kernel the library
 * launches is bracketed by HIP events on its stream. ttt_profile_read()
 * synchronises those events and reports, per kernel name, the number of
 * launches and the summed device time, writing at most max_entries of them
 * to `out`, and returns the number of distinct kernel names; the record is
 * then cleared. Not thread-safe. */
typedef struct ttt_kernel_stat {
  char name[48];
  int32_t launches;
  double total_ms;
} ttt_kernel_stat;

ttt_status ttt_profile_enable(int32_t on); /* on: clears the record */

/* Copies `bytes` bytes (a multiple of 16; both pointers 16-byte aligned,
 * not overlapping) with one plain streaming kernel, named
 * calibration_copy_kernel in profiles. It moves a known number of bytes, so
 * hardware traffic counters read on it convert counter units to bytes for
 * the layer's kernels measured in the same run. */
ttt_status ttt_copy_calibration(void* dst, const void* src, size_t bytes, void* stream);
int32_t ttt_profile_read(ttt_kernel_stat* out, int32_t max_entries);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */
