// C ABI of libttt_layer: argument checking, workspace layout, the chunk
// schedule and optional per-launch timing. Declarations and the contract of
// every entry point are in include/ttt.h.
#include "ttt.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ttt_launch.h"

namespace {

thread_local std::string g_err;

ttt_status fail(ttt_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr uint32_t kKnownFlags =
    TTT_FLAG_PAD_CHUNK | TTT_FLAG_SCHED_RUNNING | TTT_FLAG_SCHED_PREFIX;
constexpr int kMaxTaps = 64;
constexpr int64_t kMaxDim = 1 << 20;

// ------------------------------------------------------------ timing

struct TimingRecord {
  const char* name;
  hipEvent_t start, stop;
};

struct Timing {
  bool on = false;
  std::vector<TimingRecord> recs;
  std::vector<hipEvent_t> pool;
};
Timing g_timing;

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_timing.on) return launch();
  hipEvent_t a = take_event(), b = take_event();
  if (a && b) (void)hipEventRecord(a, s);
  hipError_t e = launch();
  if (a && b) {
    (void)hipEventRecord(b, s);
    g_timing.recs.push_back({name, a, b});
  }
  return e;
}

// ------------------------------------------------------------ geometry

// A chunk of the schedule: tokens [t0, t1), and whether it starts a document.
struct Chunk {
  int t0, t1;
  bool doc_start;
};

struct Geo {
  int64_t B, T, d, f, K, C, T_pad, nchunks;
  bool act_f32, w_f32, pad_chunk, running;
  int64_t w0_stride;  // elements
  tttk::Dims dims;
  std::vector<Chunk> chunks;
  std::vector<tttk::BlockInfo> blocks;     // packed documents only: per 64-token block
  std::vector<tttk::ApplyTile> tiles;      // packed documents only: the apply's token tiles
  std::vector<tttk::ChunkSpan> spans;      // packed documents only: each chunk's tokens
  float clip = 0.0f;                       // > 0: update-norm clipping limit
  bool resume = false;                     // continuation: fp32 state in place, look-ahead rows
  bool train = false;                      // training forward: keeps what the backward reads
  size_t act_bytes() const { return act_f32 ? 4 : 2; }
  size_t w_bytes() const { return w_f32 ? 4 : 2; }
};

struct Layout {
  size_t y = 0, wtt = 0, z = 0, zt = 0, vt = 0, snap = 0, hb = 0, x0b = 0, wgp = 0, wup = 0,
         blk = 0, vrow = 0, gram = 0, partial = 0, scale = 0, x0n = 0, range = 0, ztb = 0,
         sa = 0;
  size_t total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout forward_layout(const Geo& g) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const tttk::Dims& D = g.dims;
  L.range = take(tttk::kRangeWords * 4);
  L.y = take(g.B * g.T_pad * D.ld_y * 2);
  L.wtt = take(g.d * D.ld_y * 2);
  L.z = take(g.B * g.T * D.ld_z * 2);
  L.zt = take(tttk::zt_elems(D) * 2);
  L.vt = take(tttk::vt_elems(D) * 2);
  const int64_t snap_elems = tttk::snap_elems(D);
  L.snap = take(g.running ? g.B * snap_elems * 2 : g.B * g.nchunks * snap_elems * 2);
  if (g.act_f32) {
    L.hb = take(g.B * g.T * g.d * 2);
    L.x0b = take(g.B * g.T * g.d * 2);
    if (g.resume) L.x0n = take(g.B * (g.K - 1) * g.d * 2);  // bf16 look-ahead rows
  }
  L.wgp = take(tttk::wpack_elems(D) * 2);
  L.wup = take(tttk::wpack_elems(D) * 2);
  if (!g.blocks.empty())
    L.blk = take(g.blocks.size() * sizeof(tttk::BlockInfo) +
                 g.tiles.size() * sizeof(tttk::ApplyTile) +
                 g.spans.size() * sizeof(tttk::ChunkSpan));
  if (g.clip > 0.0f) {
    L.vrow = take(g.B * g.T_pad * D.ld_y * 2);
    L.gram = take(g.B * g.nchunks * tttk::clip_gram_floats((int)g.C) * 4);
    L.partial = take(g.B * g.nchunks * tttk::clip_pairs((int)g.C) * 4);
    L.scale = take(g.B * g.nchunks * 4);
  }
  if (g.train) {
    // kept for the backward (with Z and the snapshots above): Z^T in bf16
    // and the SiLU factors
    L.ztb = take(tttk::zt_elems(D) * 2);
    L.sa = take(g.B * g.T_pad * g.f * 4);
  }
  L.total = off;
  return L;
}

// Step entry points: gated activation needs the packed weights and a bf16
// copy of fp32 H; the target needs Y, WtT and a bf16 copy of fp32 X0.
Layout step_layout(const Geo& g) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.range = take(tttk::kRangeWords * 4);
  L.y = take(g.B * g.T_pad * g.dims.ld_y * 2);
  L.wtt = take(g.d * g.dims.ld_y * 2);
  if (g.act_f32) {
    L.hb = take(g.B * g.T * g.d * 2);
    L.x0b = take(g.B * g.T * g.d * 2);
  }
  L.wgp = take(tttk::wpack_elems(g.dims) * 2);
  L.wup = take(tttk::wpack_elems(g.dims) * 2);
  L.total = off;
  return L;
}

ttt_status check_desc(const ttt_desc* desc, Geo* g) {
  if (desc == nullptr) return fail(TTT_ERR_INVALID_ARG, "desc is NULL");
  const ttt_desc& D = *desc;
  if (D.batch < 1) return fail(TTT_ERR_INVALID_ARG, "batch must be >= 1");
  if (D.seq_len < 1) return fail(TTT_ERR_INVALID_ARG, "seq_len must be >= 1");
  if (D.d_model < 1 || D.d_ff < 1)
    return fail(TTT_ERR_INVALID_ARG, "d_model and d_ff must be >= 1");
  if (D.conv_k < 1) return fail(TTT_ERR_INVALID_ARG, "conv_k must be >= 1");
  if ((D.act_dtype != TTT_BF16 && D.act_dtype != TTT_F32) ||
      (D.weight_dtype != TTT_BF16 && D.weight_dtype != TTT_F32))
    return fail(TTT_ERR_INVALID_ARG, "act_dtype / weight_dtype must be TTT_BF16 or TTT_F32");
  if (D.reserved != 0 || D.reserved2 != 0)
    return fail(TTT_ERR_INVALID_ARG, "reserved fields must be 0");
  if (D.flags & ~kKnownFlags) return fail(TTT_ERR_INVALID_ARG, "unknown flag bits");
  if ((D.flags & TTT_FLAG_SCHED_RUNNING) && (D.flags & TTT_FLAG_SCHED_PREFIX))
    return fail(TTT_ERR_INVALID_ARG, "at most one schedule flag");
  if (D.d_model % 64 != 0 || D.d_ff % 64 != 0)
    return fail(TTT_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
  if (D.d_model > kMaxDim || D.d_ff > kMaxDim)
    return fail(TTT_ERR_UNSUPPORTED, "d_model / d_ff above 2^20");
  if (D.conv_k > kMaxTaps) return fail(TTT_ERR_UNSUPPORTED, "conv_k above 64");
  const int64_t df = (int64_t)D.d_model * D.d_ff;
  if (D.w0_batch_stride < 0) return fail(TTT_ERR_INVALID_ARG, "w0_batch_stride < 0");
  if (D.w0_batch_stride != 0) {
    if (D.w0_batch_stride < df)
      return fail(TTT_ERR_INVALID_ARG, "w0_batch_stride must be 0 or >= d_model * d_ff");
    const int64_t granule = D.weight_dtype == TTT_F32 ? 4 : 8;
    if (D.w0_batch_stride % granule != 0)
      return fail(TTT_ERR_INVALID_ARG, "w0_batch_stride must keep every W_down0 16-byte aligned");
  }
  const int64_t T_pad =
      (D.seq_len + tttk::kTokenPad - 1) / tttk::kTokenPad * tttk::kTokenPad;
  // Largest per-launch tile counts must fit a 32-bit grid.
  if ((int64_t)D.batch * (T_pad / 256) * (D.d_ff / 64 + 1) >= (int64_t)1 << 31)
    return fail(TTT_ERR_UNSUPPORTED, "problem too large for one launch");
  g->B = D.batch;
  g->T = D.seq_len;
  g->d = D.d_model;
  g->f = D.d_ff;
  g->K = D.conv_k;
  g->T_pad = T_pad;
  g->act_f32 = D.act_dtype == TTT_F32;
  g->w_f32 = D.weight_dtype == TTT_F32;
  g->pad_chunk = (D.flags & TTT_FLAG_PAD_CHUNK) != 0;
  g->running = (D.flags & TTT_FLAG_SCHED_RUNNING) != 0;
  g->w0_stride = D.w0_batch_stride;
  g->C = 0;
  g->nchunks = 0;
  g->dims = tttk::make_dims((int)g->B, (int)g->T, (int)g->d, (int)g->f);
  return TTT_OK;
}

ttt_status check_chunk(int32_t chunk, Geo* g) {
  if (chunk < 1) return fail(TTT_ERR_INVALID_ARG, "chunk must be >= 1");
  if (chunk % 64 != 0) return fail(TTT_ERR_UNSUPPORTED, "chunk must be a multiple of 64");
  g->C = chunk;
  g->nchunks = (g->T + chunk - 1) / chunk;
  g->chunks.clear();
  for (int64_t t = 0; t < g->T; t += chunk)
    g->chunks.push_back({(int)t, (int)std::min<int64_t>(g->T, t + chunk), t == 0});
  return TTT_OK;
}

// Packed documents: one sequence holding n_docs documents that start at
// doc_starts[r]. Chunks restart at every document start; builds the chunk
// list and the per-64-token block table the kernels read.
// Update-norm clipping: the limit on each chunk's update norm.
ttt_status check_clip(float clip_norm, Geo* g) {
  if (!(clip_norm > 0.0f) || !std::isfinite(clip_norm))
    return fail(TTT_ERR_INVALID_ARG, "clip_norm must be finite and > 0");
  g->clip = clip_norm;
  return TTT_OK;
}

ttt_status check_docs(const int32_t* doc_starts, int32_t n_docs, Geo* g) {
  if (g->B != 1) return fail(TTT_ERR_UNSUPPORTED, "packed documents need batch == 1");
  if (g->T_pad / 64 > 2048)
    return fail(TTT_ERR_UNSUPPORTED, "packed documents support up to 131072 tokens");
  if (doc_starts == nullptr) return fail(TTT_ERR_INVALID_ARG, "doc_starts is NULL");
  if (n_docs < 1) return fail(TTT_ERR_INVALID_ARG, "n_docs must be >= 1");
  if (doc_starts[0] != 0) return fail(TTT_ERR_INVALID_ARG, "doc_starts[0] must be 0");
  for (int32_t r = 1; r < n_docs; ++r) {
    if (doc_starts[r] <= doc_starts[r - 1] || doc_starts[r] >= g->T)
      return fail(TTT_ERR_INVALID_ARG,
                  "doc_starts must increase and stay below seq_len (entry " +
                      std::to_string(r) + ")");
    if (doc_starts[r] % 64 != 0)
      return fail(TTT_ERR_UNSUPPORTED, "document starts must be multiples of 64 (entry " +
                                           std::to_string(r) + ")");
  }
  const int C = (int)g->C;
  const int64_t nblk = g->T_pad / 64;
  g->chunks.clear();
  g->blocks.assign(nblk, tttk::BlockInfo{0, 0, (int32_t)g->T, (int32_t)g->T});
  for (int32_t r = 0; r < n_docs; ++r) {
    const int a = doc_starts[r], e = r + 1 < n_docs ? doc_starts[r + 1] : (int)g->T;
    for (int t0 = a; t0 < e; t0 += C) {
      const int t1 = std::min(e, t0 + C);
      const int32_t idx = (int32_t)g->chunks.size();
      g->chunks.push_back({t0, t1, t0 == a});
      for (int t = t0; t < t1; t += 64)
        g->blocks[t / 64] = {idx,
                             (t == t0 ? tttk::kBlockChunkStart : 0) |
                                 (t == a ? tttk::kBlockDocStart : 0),
                             e, t1};
    }
  }
  g->nchunks = (int64_t)g->chunks.size();
  for (int64_t b = (g->T + 63) / 64; b < nblk; ++b) g->blocks[b].chunk = (int32_t)g->nchunks - 1;
  g->spans.clear();
  for (const Chunk& c : g->chunks) g->spans.push_back({c.t0, c.t1});
  // The apply's token tiles start at every chunk start; a chunk's last tile
  // may be partial. A document's first chunk starts from W_down0, whose
  // snapshot is slot 0 (the first document's first chunk): its tiles read
  // that slot, and the update stores no copy of it.
  const int bn = tttk::apply_tile_width(C);
  g->tiles.clear();
  for (size_t i = 0; i < g->chunks.size(); ++i) {
    const int32_t slot = g->chunks[i].doc_start ? 0 : (int32_t)i;
    for (int t = g->chunks[i].t0; t < g->chunks[i].t1; t += bn)
      g->tiles.push_back({t, std::min(g->chunks[i].t1, t + bn), slot, 0});
  }
  return TTT_OK;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;
};

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

ttt_status check_ptr(const void* p, const char* name, size_t align = 16) {
  if (p == nullptr) return fail(TTT_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(TTT_ERR_INVALID_ARG,
                std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return TTT_OK;
}

Range range_of(const char* name, const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {name, lo, lo + bytes};
}

ttt_status check_aliasing(const std::vector<Range>& inputs, const std::vector<Range>& outputs) {
  for (size_t i = 0; i < outputs.size(); ++i) {
    for (const Range& in : inputs)
      if (overlaps(outputs[i], in))
        return fail(TTT_ERR_ALIAS,
                    std::string(outputs[i].name) + " overlaps input " + in.name);
    for (size_t j = i + 1; j < outputs.size(); ++j)
      if (overlaps(outputs[i], outputs[j]))
        return fail(TTT_ERR_ALIAS,
                    std::string(outputs[i].name) + " overlaps " + outputs[j].name);
  }
  return TTT_OK;
}

#define TTT_TRY(expr)                 \
  do {                                \
    ttt_status _s = (expr);           \
    if (_s != TTT_OK) return _s;      \
  } while (0)

#define TTT_LAUNCH(name, stream, call)                                            \
  do {                                                                            \
    hipError_t _e = timed(name, stream, [&]() { return (call); });                \
    if (_e != hipSuccess)                                                         \
      return fail(TTT_ERR_HIP, std::string(name) + ": " + hipGetErrorString(_e)); \
  } while (0)

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

namespace tttk_api {
// The error record of the other translation units' entry points.
__attribute__((visibility("hidden"))) ttt_status set_error(ttt_status s, const std::string& msg) {
  return fail(s, msg);
}
}  // namespace tttk_api

extern "C" {

const char* ttt_status_string(int32_t s) {
  switch (s) {
    case TTT_OK: return "TTT_OK";
    case TTT_ERR_INVALID_ARG: return "TTT_ERR_INVALID_ARG";
    case TTT_ERR_UNSUPPORTED: return "TTT_ERR_UNSUPPORTED";
    case TTT_ERR_WORKSPACE: return "TTT_ERR_WORKSPACE";
    case TTT_ERR_ALIAS: return "TTT_ERR_ALIAS";
    case TTT_ERR_HIP: return "TTT_ERR_HIP";
    default: return "TTT_ERR_UNKNOWN";
  }
}

const char* ttt_last_error(void) { return g_err.c_str(); }
const char* ttt_last_error_message(void) { return g_err.c_str(); }

ttt_status ttt_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = forward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_step_workspace_size(const ttt_desc* desc, size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = step_layout(g).total;
  return TTT_OK;
}

}  // extern "C"

namespace {

// The update's operands are fp16 with the target scaled by vscale = eta *
// 2^p, p = round(-log2 |eta|), so that eta * V sits at V's own magnitude;
// the state is carried as 2^p * W in fp32 (times the operands' own range
// exponents, read on the device) and every output is multiplied back. Powers
// of two make the scalings exact.
void update_scales(float eta, float* vscale, int* p_out) {
  *vscale = 0.0f;
  *p_out = 0;
  if (eta != 0.0f) {
    long p = std::lround(-std::log2(std::fabs((double)eta)));
    p = std::max(-60L, std::min(60L, p));
    *p_out = (int)p;
    *vscale = eta * std::ldexp(1.0f, (int)p);
  }
}

// Everything after the descriptor, chunk (or document) checks: pointer and
// workspace checks, then the launches of the whole layer. For a continuation
// (g.resume) W_down0 and W_down_final are the same fp32 [B, d, f] state,
// read as the initial state and overwritten with the final one, and X0_next
// holds n_next look-ahead rows per sequence.
ttt_status forward_impl(const Geo& g, const void* H, const void* X0, const void* Wg,
                        const void* Wu, const void* W_down0, const void* conv_taps,
                        const void* W_target, float eta, void* O, float* W_down_final,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const void* X0_next = nullptr, int n_next = 0) {
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  TTT_TRY(check_ptr(H, "H"));
  TTT_TRY(check_ptr(X0, "X0"));
  if (n_next > 0) TTT_TRY(check_ptr(X0_next, "X0_next"));
  TTT_TRY(check_ptr(Wg, "Wg"));
  TTT_TRY(check_ptr(Wu, "Wu"));
  TTT_TRY(check_ptr(W_down0, "W_down0"));
  TTT_TRY(check_ptr(conv_taps, "conv_taps"));
  TTT_TRY(check_ptr(W_target, "W_target"));
  TTT_TRY(check_ptr(O, "O"));
  TTT_TRY(check_ptr(W_down_final, "W_down_final"));
  TTT_TRY(check_ptr(workspace, "workspace", 256));
  const Layout L = forward_layout(g);
  if (workspace_bytes < L.total)
    return fail(TTT_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " bytes, needs " + std::to_string(L.total));
  const size_t ab = g.act_bytes(), wb = g.w_bytes();
  const size_t w0_bytes =
      g.w0_stride == 0 ? g.d * g.f * wb : ((g.B - 1) * g.w0_stride + g.d * g.f) * wb;
  std::vector<Range> inputs = {
      range_of("H", H, g.B * g.T * g.d * ab),
      range_of("X0", X0, g.B * g.T * g.d * ab),
      range_of("Wg", Wg, g.f * g.d * wb),
      range_of("Wu", Wu, g.f * g.d * wb),
      range_of("conv_taps", conv_taps, g.K * g.d * wb),
      range_of("W_target", W_target, g.d * g.d * wb)};
  // The continuation's state is both read and written, by the same tiles of
  // the same kernels: it is an output here.
  if (!g.resume) inputs.push_back(range_of("W_down0", W_down0, w0_bytes));
  if (n_next > 0) inputs.push_back(range_of("X0_next", X0_next, g.B * n_next * g.d * ab));
  const std::vector<Range> outputs = {
      range_of("O", O, g.B * g.T * g.d * ab),
      range_of(g.resume ? "W_state" : "W_down_final", W_down_final, g.B * g.d * g.f * 4),
      range_of("workspace", workspace, L.total)};
  TTT_TRY(check_aliasing(inputs, outputs));
  // Initial state: the caller's W_down0, or the continuation's fp32 state.
  const bool w0_f32 = g.resume || g.w_f32;
  const int64_t w0_stride = g.resume ? g.d * g.f : g.w0_stride;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const tttk::Dims& D = g.dims;
  const int64_t df = g.d * g.f;

  // Packed documents: the block table, the apply's tile list and the chunk
  // spans go to the workspace first, in one asynchronous copy. Its host
  // buffer must outlive the copy, which may run after this call returns: a
  // host function enqueued behind the copy frees it.
  const tttk::BlockInfo* blocks = nullptr;
  const tttk::ApplyTile* tiles = nullptr;
  const tttk::ChunkSpan* spans = nullptr;
  if (!g.blocks.empty()) {
    const size_t nb = g.blocks.size() * sizeof(tttk::BlockInfo);
    const size_t nt = g.tiles.size() * sizeof(tttk::ApplyTile);
    const size_t ns = g.spans.size() * sizeof(tttk::ChunkSpan);
    char* host = static_cast<char*>(std::malloc(nb + nt + ns));
    if (host == nullptr) return fail(TTT_ERR_HIP, "document table: host allocation failed");
    std::memcpy(host, g.blocks.data(), nb);
    std::memcpy(host + nb, g.tiles.data(), nt);
    std::memcpy(host + nb + nt, g.spans.data(), ns);
    char* dst = at<char>(workspace, L.blk);
    hipError_t e = hipMemcpyAsync(dst, host, nb + nt + ns, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipLaunchHostFunc(s, [](void* p) { std::free(p); }, host);
    if (e != hipSuccess) {
      // The copy may be queued: let the stream drain before freeing.
      (void)hipStreamSynchronize(s);
      std::free(host);
      return fail(TTT_ERR_HIP, std::string("document table copy: ") + hipGetErrorString(e));
    }
    blocks = reinterpret_cast<const tttk::BlockInfo*>(dst);
    tiles = reinterpret_cast<const tttk::ApplyTile*>(dst + nb);
    spans = reinterpret_cast<const tttk::ChunkSpan*>(dst + nb + nt);
  }

  // bf16 operands
  const uint16_t* Hb = static_cast<const uint16_t*>(H);
  const uint16_t* X0b = static_cast<const uint16_t*>(X0);
  const uint16_t* X0nb = static_cast<const uint16_t*>(X0_next);
  if (g.act_f32) {
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(H),
                                                      at<uint16_t>(workspace, L.hb), g.B * g.T * g.d, s));
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(X0),
                                                      at<uint16_t>(workspace, L.x0b), g.B * g.T * g.d, s));
    Hb = at<uint16_t>(workspace, L.hb);
    X0b = at<uint16_t>(workspace, L.x0b);
    if (n_next > 0) {
      TTT_LAUNCH("cast_bf16", s,
                 tttk::launch_cast_bf16(static_cast<const float*>(X0_next),
                                        at<uint16_t>(workspace, L.x0n), g.B * n_next * g.d, s));
      X0nb = at<uint16_t>(workspace, L.x0n);
    }
  }
  uint16_t* Wgp = at<uint16_t>(workspace, L.wgp);
  uint16_t* Wup = at<uint16_t>(workspace, L.wup);
  uint32_t* range = at<uint32_t>(workspace, L.range);
  TTT_LAUNCH("range_clear", s, tttk::launch_range_clear(range, s));
  TTT_LAUNCH("pack_weights", s, tttk::launch_pack_weight(Wg, g.w_f32, Wgp, D, s));
  TTT_LAUNCH("pack_weights", s, tttk::launch_pack_weight(Wu, g.w_f32, Wup, D, s));
  uint16_t* Y = at<uint16_t>(workspace, L.y);
  uint16_t* WtT = at<uint16_t>(workspace, L.wtt);
  uint16_t* Z = at<uint16_t>(workspace, L.z);
  uint16_t* ZT = at<uint16_t>(workspace, L.zt);
  uint16_t* VT = at<uint16_t>(workspace, L.vt);
  uint16_t* snap = at<uint16_t>(workspace, L.snap);

  float vscale;
  int p;
  update_scales(eta, &vscale, &p);

  // The fp16 copies (W_target^T, conv(X0), Z^T, V^T) keep their values in
  // fp16's range: each producer notes its largest |value| and a repair launch
  // rewrites the copy times 2^q when that maximum is out of range (it
  // returns at once otherwise); the consumers divide 2^q back out.
  TTT_LAUNCH("amax", s,
             tttk::launch_amax(W_target, g.w_f32, g.d * g.d, range + tttk::kRangeWt * tttk::kRangeSlots, s));
  TTT_LAUNCH("transpose_w_target", s,
             tttk::launch_transpose_f16(W_target, g.w_f32, WtT, (int)g.d, (int)g.d, D.ld_y,
                                        range + tttk::kRangeWt * tttk::kRangeSlots, s));
  uint32_t* range_y = range + tttk::kRangeY * tttk::kRangeSlots;
  TTT_LAUNCH("conv", s,
             tttk::launch_conv(X0b, X0nb, n_next, conv_taps, g.w_f32, Y, D, (int)g.K, (int)g.C,
                               g.pad_chunk, blocks, range_y, s));
  TTT_LAUNCH("conv_repair", s,
             tttk::launch_conv_repair(X0b, X0nb, n_next, conv_taps, g.w_f32, Y, D, (int)g.K,
                                      (int)g.C, g.pad_chunk, blocks, range_y, s));
  uint32_t* range_z = range + tttk::kRangeZ * tttk::kRangeSlots;
  const bool clip = g.clip > 0.0f && eta != 0.0f;
  uint16_t* Vrow = clip ? at<uint16_t>(workspace, L.vrow) : nullptr;
  if (!g.train && tttk::gate_up_target_merges(D)) {
    // Both part-empty last rounds in one: the target's tiles run in gate/up's.
    TTT_LAUNCH("gate_up_target", s,
               tttk::launch_gate_up_target(Hb, Wgp, Wup, Z, ZT, Y, WtT, VT, Vrow, vscale, D,
                                           range, s));
    TTT_LAUNCH("gate_up_repair", s,
               tttk::launch_gate_up_repair(Hb, Wgp, Wup, ZT, D, range_z, s));
  } else {
    if (g.train)
      TTT_LAUNCH("gate_up", s,
                 tttk::launch_gate_up_train(Hb, Wgp, Wup, Z, ZT, at<uint16_t>(workspace, L.ztb),
                                            at<uint32_t>(workspace, L.sa), D, range_z, s));
    else
      TTT_LAUNCH("gate_up", s, tttk::launch_gate_up(Hb, Wgp, Wup, Z, ZT, D, range_z, s));
    TTT_LAUNCH("gate_up_repair", s,
               tttk::launch_gate_up_repair(Hb, Wgp, Wup, ZT, D, range_z, s));
    TTT_LAUNCH("target", s, tttk::launch_target(Y, WtT, VT, nullptr, Vrow, vscale, D, range, s));
  }
  TTT_LAUNCH("target_repair", s,
             tttk::launch_target_repair(Y, WtT, VT, Vrow, vscale, p, D, range, s));
  if (clip) {
    // Every chunk's update eta V_i^T Z_i is scaled to a Frobenius norm of at
    // most g.clip by scaling its columns of VT; the norm comes from the rows
    // of vscale * V (times V's range exponent, which the kernel divides out),
    // hence the factor |eta| / vscale.
    TTT_LAUNCH("clip_scale", s,
               tttk::launch_clip_scale(Z, Vrow, at<float>(workspace, L.gram),
                                       at<float>(workspace, L.partial),
                                       at<float>(workspace, L.scale), VT, D, (int)g.C,
                                       (int)g.nchunks, spans, blocks, std::fabs(eta) / vscale,
                                       g.clip, range, p, s));
  }

  const int64_t snap_cstride = tttk::snap_elems(D);
  if (!g.running) {
    // Materialised exclusive prefix: snapshot i = bf16(W^(i)) for every chunk,
    // W_down_final = W^(k); then every chunk's output in one launch.
    TTT_LAUNCH("update_prefix", s,
               tttk::launch_update(ZT, VT, W_down0, w0_f32, w0_stride, g.f, p, range, snap,
                                   g.nchunks * snap_cstride, W_down_final, nullptr, D, 0,
                                   (int)g.T, (int)g.C, blocks, (int)g.nchunks, s));
    TTT_LAUNCH("apply", s,
               tttk::launch_apply(Z, snap, g.nchunks * snap_cstride, snap_cstride, O, g.act_f32,
                                  D, 0, (int)g.T, (int)g.C, tiles, (int)g.tiles.size(),
                                  (int)g.nchunks, s));
  } else {
    // Running state: W_down_final holds W^(i) in fp32, `snap` its bf16 copy;
    // both start from W_down0 at every document start.
    for (const Chunk& c : g.chunks) {
      if (c.doc_start)
        TTT_LAUNCH("update_running", s,
                   tttk::launch_update(ZT, VT, W_down0, w0_f32, w0_stride, g.f, p, range,
                                       nullptr, 0, W_down_final, snap, D, 0, 0, (int)g.C,
                                       nullptr, 1, s));
      TTT_LAUNCH("apply", s,
                 tttk::launch_apply(Z, snap, snap_cstride, 0, O, g.act_f32, D, c.t0, c.t1,
                                    (int)g.C, nullptr, 0, 1, s));
      TTT_LAUNCH("update_running", s,
                 tttk::launch_update(ZT, VT, W_down_final, true, df, g.f, p, range, nullptr, 0,
                                     W_down_final, snap, D, c.t0, c.t1 - c.t0, (int)g.C,
                                     nullptr, 1, s));
    }
  }
  return TTT_OK;
}

}  // namespace

extern "C" {

ttt_status ttt_layer_forward(const ttt_desc* desc, const void* H, const void* X0,
                             const void* Wg, const void* Wu, const void* W_down0,
                             const void* conv_taps, const void* W_target, float eta,
                             int32_t chunk, void* O, float* W_down_final, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  return forward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, O, W_down_final,
                      workspace, workspace_bytes, stream);
}

ttt_status ttt_clipped_workspace_size(const ttt_desc* desc, int32_t chunk, float clip_norm,
                                      size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_clip(clip_norm, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = forward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_layer_forward_clipped(const ttt_desc* desc, const void* H, const void* X0,
                                     const void* Wg, const void* Wu, const void* W_down0,
                                     const void* conv_taps, const void* W_target, float eta,
                                     int32_t chunk, float clip_norm, void* O,
                                     float* W_down_final, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_clip(clip_norm, &g));
  return forward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, O, W_down_final,
                      workspace, workspace_bytes, stream);
}

ttt_status ttt_packed_workspace_size(const ttt_desc* desc, int32_t chunk,
                                     const int32_t* doc_starts, int32_t n_docs,
                                     size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_docs(doc_starts, n_docs, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = forward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_layer_forward_packed(const ttt_desc* desc, const void* H, const void* X0,
                                    const void* Wg, const void* Wu, const void* W_down0,
                                    const void* conv_taps, const void* W_target, float eta,
                                    int32_t chunk, const int32_t* doc_starts, int32_t n_docs,
                                    void* O, float* W_down_final, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_docs(doc_starts, n_docs, &g));
  return forward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, O, W_down_final,
                      workspace, workspace_bytes, stream);
}

static_assert(sizeof(ttt_packed_block) == sizeof(tttk::BlockInfo) &&
                  TTT_BLOCK_CHUNK_START == tttk::kBlockChunkStart &&
                  TTT_BLOCK_DOC_START == tttk::kBlockDocStart,
              "the exported block table is the kernels' table");
static_assert(sizeof(ttt_packed_tile) == sizeof(tttk::ApplyTile), "tile entries");

ttt_status ttt_packed_tables(const ttt_desc* desc, int32_t chunk, const int32_t* doc_starts,
                             int32_t n_docs, ttt_packed_block* blocks, int32_t max_blocks,
                             ttt_packed_tile* tiles, int32_t max_tiles, int32_t* counts) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_docs(doc_starts, n_docs, &g));
  if (counts == nullptr) return fail(TTT_ERR_INVALID_ARG, "counts is NULL");
  if (max_blocks < 0 || max_tiles < 0)
    return fail(TTT_ERR_INVALID_ARG, "max_blocks / max_tiles must be >= 0");
  if ((max_blocks > 0 && blocks == nullptr) || (max_tiles > 0 && tiles == nullptr))
    return fail(TTT_ERR_INVALID_ARG, "blocks / tiles is NULL");
  counts[0] = (int32_t)g.blocks.size();
  counts[1] = (int32_t)g.tiles.size();
  counts[2] = (int32_t)g.nchunks;
  for (int32_t i = 0; i < max_blocks && i < counts[0]; ++i) {
    const tttk::BlockInfo& b = g.blocks[i];
    blocks[i] = {b.chunk, b.flags, b.doc_end, b.chunk_end};
  }
  for (int32_t i = 0; i < max_tiles && i < counts[1]; ++i) {
    const tttk::ApplyTile& t = g.tiles[i];
    tiles[i] = {t.t0, t.t1, t.chunk, 0};
  }
  return TTT_OK;
}

ttt_status ttt_packed_clipped_workspace_size(const ttt_desc* desc, int32_t chunk,
                                             const int32_t* doc_starts, int32_t n_docs,
                                             float clip_norm, size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_docs(doc_starts, n_docs, &g));
  TTT_TRY(check_clip(clip_norm, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = forward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_layer_forward_packed_clipped(const ttt_desc* desc, const void* H, const void* X0,
                                            const void* Wg, const void* Wu, const void* W_down0,
                                            const void* conv_taps, const void* W_target,
                                            float eta, int32_t chunk, const int32_t* doc_starts,
                                            int32_t n_docs, float clip_norm, void* O,
                                            float* W_down_final, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_docs(doc_starts, n_docs, &g));
  TTT_TRY(check_clip(clip_norm, &g));
  return forward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, O, W_down_final,
                      workspace, workspace_bytes, stream);
}

ttt_status ttt_continue_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  g.resume = true;
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = forward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_layer_forward_continue(const ttt_desc* desc, const void* H, const void* X0,
                                      const void* X0_next, int32_t n_next, const void* Wg,
                                      const void* Wu, float* W_state, const void* conv_taps,
                                      const void* W_target, float eta, int32_t chunk, void* O,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  g.resume = true;
  if (desc->w0_batch_stride != 0)
    return fail(TTT_ERR_INVALID_ARG,
                "w0_batch_stride must be 0: the continued state is [batch, d_model, d_ff]");
  if (n_next < 0 || n_next > g.K - 1)
    return fail(TTT_ERR_INVALID_ARG, "n_next must be in [0, conv_k - 1]");
  TTT_TRY(check_ptr(W_state, "W_state"));
  return forward_impl(g, H, X0, Wg, Wu, W_state, conv_taps, W_target, eta, O, W_state,
                      workspace, workspace_bytes, stream, X0_next, n_next);
}

// ------------------------------------------------------------ decode

}  // extern "C"

namespace {

// The decode state of B sequences: the bf16 copy of each state the apply
// reads, the open chunk's Z^T and X0 rows, and the chunk-end scratch (Y,
// W_target^T, V^T) and per-token scratch (z).
struct DecodeLayout {
  size_t shadow = 0, zt = 0, x0c = 0, zb = 0, y = 0, wtt = 0, vt = 0, zc = 0,
         range = 0, total = 0;
};

DecodeLayout decode_layout(const Geo& g, const tttk::Dims& Dc) {
  DecodeLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.shadow = take(g.B * tttk::snap_elems(Dc) * 2);
  L.zt = take(tttk::zt_elems(Dc) * 2);
  L.x0c = take(g.B * g.C * g.d * 2);
  L.zb = take(g.B * g.f * 2);
  L.y = take(g.B * Dc.T_pad * Dc.ld_y * 2);
  L.wtt = take(g.d * Dc.ld_y * 2);
  L.vt = take(tttk::vt_elems(Dc) * 2);
  L.zc = take(g.B * g.C * g.f * 4);
  L.range = take(tttk::kRangeWords * 4);
  L.total = off;
  return L;
}

// Descriptor checks of the decode entry points: one token per sequence,
// chunk-local padding, states [B, d, f]. Dc: the dims of one chunk.
ttt_status check_decode(const ttt_desc* desc, int32_t chunk, Geo* g, tttk::Dims* Dc) {
  TTT_TRY(check_desc(desc, g));
  TTT_TRY(check_chunk(chunk, g));
  if (desc->seq_len != 1)
    return fail(TTT_ERR_INVALID_ARG, "decode takes one token per sequence: seq_len must be 1");
  if (!(desc->flags & TTT_FLAG_PAD_CHUNK))
    return fail(TTT_ERR_UNSUPPORTED,
                "decode needs TTT_FLAG_PAD_CHUNK: with sequence padding a chunk's targets read "
                "tokens that are not decoded yet");
  if (desc->w0_batch_stride != 0)
    return fail(TTT_ERR_INVALID_ARG, "w0_batch_stride must be 0: W_state is [batch, d, f]");
  *Dc = tttk::make_dims((int)g->B, chunk, (int)g->d, (int)g->f);
  // A closing chunk runs the prefill kernels over the chunk's tokens.
  if ((int64_t)g->B * (Dc->T_pad / 256) * (g->f / 64 + 1) >= (int64_t)1 << 31)
    return fail(TTT_ERR_UNSUPPORTED, "chunk too large for one launch");
  return TTT_OK;
}

ttt_status check_dstate(void* dstate, size_t bytes, const DecodeLayout& L) {
  TTT_TRY(check_ptr(dstate, "decode_state", 256));
  if (bytes < L.total)
    return fail(TTT_ERR_WORKSPACE, "decode state has " + std::to_string(bytes) +
                                       " bytes, needs " + std::to_string(L.total));
  return TTT_OK;
}

}  // namespace

extern "C" {

ttt_status ttt_decode_state_size(const ttt_desc* desc, int32_t chunk, size_t* bytes) {
  Geo g;
  tttk::Dims Dc;
  TTT_TRY(check_decode(desc, chunk, &g, &Dc));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = decode_layout(g, Dc).total;
  return TTT_OK;
}

ttt_status ttt_decode_begin(const ttt_desc* desc, int32_t chunk, float* W_state,
                            void* decode_state, size_t decode_state_bytes, void* stream) {
  Geo g;
  tttk::Dims Dc;
  TTT_TRY(check_decode(desc, chunk, &g, &Dc));
  TTT_TRY(check_ptr(W_state, "W_state"));
  const DecodeLayout L = decode_layout(g, Dc);
  TTT_TRY(check_dstate(decode_state, decode_state_bytes, L));
  TTT_TRY(check_aliasing({}, {range_of("W_state", W_state, g.B * g.d * g.f * 4),
                              range_of("decode_state", decode_state, L.total)}));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The open chunk's range buffer starts empty; an update over no tokens
  // stores W_state back unchanged and writes its bf16 copy.
  TTT_LAUNCH("range_clear", s, tttk::launch_range_clear(at<uint32_t>(decode_state, L.range), s));
  TTT_LAUNCH("decode_begin", s,
             tttk::launch_update(at<uint16_t>(decode_state, L.zt),
                                 at<uint16_t>(decode_state, L.vt), W_state, true, g.d * g.f,
                                 g.f, 0, nullptr, nullptr, 0, W_state,
                                 at<uint16_t>(decode_state, L.shadow), Dc, 0, 0, (int)g.C,
                                 nullptr, 1, s));
  return TTT_OK;
}

ttt_status ttt_decode_step(const ttt_desc* desc, const void* h, const void* x0, const void* Wg,
                           const void* Wu, const void* conv_taps, const void* W_target,
                           float eta, int32_t chunk, int32_t pos, float* W_state,
                           void* decode_state, size_t decode_state_bytes, void* o,
                           void* stream) {
  Geo g;
  tttk::Dims Dc;
  TTT_TRY(check_decode(desc, chunk, &g, &Dc));
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  if (pos < 0) return fail(TTT_ERR_INVALID_ARG, "pos must be >= 0");
  TTT_TRY(check_ptr(h, "h"));
  TTT_TRY(check_ptr(x0, "x0"));
  TTT_TRY(check_ptr(Wg, "Wg"));
  TTT_TRY(check_ptr(Wu, "Wu"));
  TTT_TRY(check_ptr(conv_taps, "conv_taps"));
  TTT_TRY(check_ptr(W_target, "W_target"));
  TTT_TRY(check_ptr(W_state, "W_state"));
  TTT_TRY(check_ptr(o, "o"));
  const DecodeLayout L = decode_layout(g, Dc);
  TTT_TRY(check_dstate(decode_state, decode_state_bytes, L));
  const size_t ab = g.act_bytes(), wb = g.w_bytes();
  TTT_TRY(check_aliasing({range_of("h", h, g.B * g.d * ab), range_of("x0", x0, g.B * g.d * ab),
                          range_of("Wg", Wg, g.f * g.d * wb), range_of("Wu", Wu, g.f * g.d * wb),
                          range_of("conv_taps", conv_taps, g.K * g.d * wb),
                          range_of("W_target", W_target, g.d * g.d * wb)},
                         {range_of("o", o, g.B * g.d * ab),
                          range_of("W_state", W_state, g.B * g.d * g.f * 4),
                          range_of("decode_state", decode_state, L.total)}));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int C = (int)g.C, r = pos % C;
  uint16_t* shadow = at<uint16_t>(decode_state, L.shadow);
  uint16_t* zt = at<uint16_t>(decode_state, L.zt);
  uint16_t* x0c = at<uint16_t>(decode_state, L.x0c);
  uint16_t* zb = at<uint16_t>(decode_state, L.zb);
  float* zc = at<float>(decode_state, L.zc);
  uint32_t* range = at<uint32_t>(decode_state, L.range);
  const int64_t zt_bstride = tttk::sb_elems<tttk::kZtSlab>(g.f, Dc.T_pad);
  TTT_LAUNCH("decode_gate_up", s,
             tttk::launch_decode_gate_up(h, x0, g.act_f32, Wg, Wu, g.w_f32, (int)g.B, (int)g.d,
                                         (int)g.f, zb, zc, zt, zt_bstride, (int)Dc.T_pad, x0c, C,
                                         r, range, s));
  TTT_LAUNCH("decode_apply", s,
             tttk::launch_decode_apply(zb, shadow, tttk::snap_elems(Dc), (int)g.B, (int)g.d,
                                       (int)g.f, o, g.act_f32, s));
  if (r == C - 1) {
    // The chunk is complete: its Z^T brought into fp16's range if needed, its
    // target (reads inside the chunk only, with the same range guards as the
    // prefill), then its update, in place, with the bf16 copy refreshed for
    // the next chunk; the range buffer is cleared for the next chunk.
    float vscale;
    int p;
    update_scales(eta, &vscale, &p);
    uint16_t* y = at<uint16_t>(decode_state, L.y);
    uint16_t* wtt = at<uint16_t>(decode_state, L.wtt);
    uint16_t* vt = at<uint16_t>(decode_state, L.vt);
    uint32_t* range_wt = range + tttk::kRangeWt * tttk::kRangeSlots;
    uint32_t* range_y = range + tttk::kRangeY * tttk::kRangeSlots;
    TTT_LAUNCH("decode_zt_repair", s,
               tttk::launch_decode_zt_repair(zc, zt, (int)g.B, (int)g.f, C, zt_bstride,
                                             (int)Dc.T_pad, range, s));
    TTT_LAUNCH("amax", s, tttk::launch_amax(W_target, g.w_f32, g.d * g.d, range_wt, s));
    TTT_LAUNCH("transpose_w_target", s,
               tttk::launch_transpose_f16(W_target, g.w_f32, wtt, (int)g.d, (int)g.d, Dc.ld_y,
                                          range_wt, s));
    TTT_LAUNCH("conv", s,
               tttk::launch_conv(x0c, nullptr, 0, conv_taps, g.w_f32, y, Dc, (int)g.K, C, true,
                                 nullptr, range_y, s));
    TTT_LAUNCH("conv_repair", s,
               tttk::launch_conv_repair(x0c, nullptr, 0, conv_taps, g.w_f32, y, Dc, (int)g.K, C,
                                        true, nullptr, range_y, s));
    TTT_LAUNCH("target", s,
               tttk::launch_target(y, wtt, vt, nullptr, nullptr, vscale, Dc, range, s));
    TTT_LAUNCH("target_repair", s,
               tttk::launch_target_repair(y, wtt, vt, nullptr, vscale, p, Dc, range, s));
    TTT_LAUNCH("update_running", s,
               tttk::launch_update(zt, vt, W_state, true, g.d * g.f, g.f, p, range, nullptr, 0,
                                   W_state, shadow, Dc, 0, C, C, nullptr, 1, s));
    TTT_LAUNCH("range_clear", s, tttk::launch_range_clear(range, s));
  }
  return TTT_OK;
}

}  // extern "C"

namespace {

// The backward's workspace: the forward's recomputed activations (bf16 and
// slab copies), the states W_i^T and state gradients Gbar (both
// orientations) of every chunk, and the gradients' intermediates.
struct BwdLayout {
  size_t range = 0, wgp = 0, wup = 0, hb = 0, x0b = 0, dov = 0, y = 0, wtt = 0, yt = 0, z = 0,
         zt = 0, sa = 0, vt = 0, dot = 0, ht = 0, ws = 0, gs = 0, dw0 = 0, dgu = 0, dgt = 0,
         dut = 0, dv = 0, dvt = 0, wgut = 0, wtb = 0, dy = 0, part = 0, total = 0;
  int64_t ld_gu = 0, ld_ov = 0;
};

// With `saved` (the training forward's workspace holds Z, Z^T, the SiLU
// factors and the states) the recompute's buffers are not needed.
BwdLayout backward_layout(const Geo& g, bool saved = false) {
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const tttk::Dims& D = g.dims;
  const int64_t BT = g.B * g.T, BTp = g.B * g.T_pad;
  const int64_t snap_df = tttk::sb_elems<256>(g.d, g.f);
  L.ld_gu = tttk::pad_ld(2 * g.f);
  L.ld_ov = tttk::pad_ld(2 * g.d);
  L.range = take(tttk::kRangeWords * 4);
  if (!saved) {
    L.wgp = take(tttk::wpack_elems(D) * 2);
    L.wup = take(tttk::wpack_elems(D) * 2);
  }
  if (g.act_f32) {
    L.hb = take(BT * g.d * 2);
    L.x0b = take(BT * g.d * 2);
  }
  L.dov = take(BT * L.ld_ov * 2);
  L.y = take(BTp * D.ld_y * 2);
  L.wtt = take(g.d * D.ld_y * 2);
  L.yt = take(tttk::sb_elems<256>(g.d, BTp) * 2);
  if (!saved) {
    L.z = take(BT * D.ld_z * 2);
    L.zt = take(tttk::zt_elems(D) * 2);
    L.sa = take(BTp * g.f * 4);
  }
  L.vt = take(tttk::vt_elems(D) * 2);
  L.dot = take(tttk::vt_elems(D) * 2);
  L.ht = take(tttk::sb_elems<256>(g.d, BTp) * 2);
  if (!saved) L.ws = take(g.B * g.nchunks * snap_df * 2);
  L.gs = take(g.B * g.nchunks * snap_df * 2);
  if (g.w0_stride == 0 && g.B > 1) L.dw0 = take(g.B * g.d * g.f * 4);
  L.dgu = take(BT * L.ld_gu * 2);
  L.dgt = take(tttk::sb_elems<256>(g.f, BTp) * 2);
  L.dut = take(tttk::sb_elems<256>(g.f, BTp) * 2);
  L.dv = take(BT * g.d * 2);
  L.dvt = take(tttk::sb_elems<256>(g.d, BTp) * 2);
  L.wgut = take(g.d * L.ld_gu * 2);
  if (g.w_f32) L.wtb = take(g.d * g.d * 2);
  L.dy = take(BT * g.d * 4);
  L.part = take(tttk::conv_bwd_part_floats((int)g.B, (int)g.T, (int)g.K, (int)g.d) * 4);
  L.total = off;
  return L;
}

// The training forward and its backward: the descriptor and chunk checks of
// the prefill; the prefix schedule only (its per-chunk snapshots are what
// the backward reads).
ttt_status check_train_desc(const ttt_desc* desc, int32_t chunk, Geo* g) {
  TTT_TRY(check_desc(desc, g));
  TTT_TRY(check_chunk(chunk, g));
  if (g->running)
    return fail(TTT_ERR_UNSUPPORTED,
                "the training forward keeps every chunk's state: prefix schedule only");
  g->train = true;
  return TTT_OK;
}

// The backward of a prefill (see ttt_layer_backward). With `saved` (the
// workspace of ttt_layer_forward_train on the same arguments, g.train set),
// Z, Z^T, the SiLU factors and the states W_i come from it: the gate/up
// recompute and the state scan are skipped, and W_i^T is the transpose of
// the forward's bf16 snapshots.
ttt_status backward_impl(const Geo& g, const void* H, const void* X0, const void* Wg,
                         const void* Wu, const void* W_down0, const void* conv_taps,
                         const void* W_target, float eta, const void* saved, size_t saved_bytes,
                         const void* dO, const float* dW_final, float* dH, float* dX0,
                         float* dWg, float* dWu, float* dW_down0, float* dtaps, float* dW_target,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!std::isfinite(eta)) return fail(TTT_ERR_INVALID_ARG, "eta must be finite");
  const char* names[] = {"H", "X0", "Wg", "Wu", "W_down0", "conv_taps", "W_target", "dO",
                         "dH", "dX0", "dWg", "dWu", "dW_down0", "dtaps", "dW_target"};
  const void* ptrs[] = {H, X0, Wg, Wu, W_down0, conv_taps, W_target, dO,
                        dH, dX0, dWg, dWu, dW_down0, dtaps, dW_target};
  for (int i = 0; i < 15; ++i) TTT_TRY(check_ptr(ptrs[i], names[i]));
  if (dW_final != nullptr) TTT_TRY(check_ptr(dW_final, "dW_final"));
  TTT_TRY(check_ptr(workspace, "workspace", 256));
  const bool sv = saved != nullptr;
  Layout F;
  if (sv) {
    TTT_TRY(check_ptr(saved, "saved", 256));
    F = forward_layout(g);
    if (saved_bytes < F.total)
      return fail(TTT_ERR_WORKSPACE, "saved has " + std::to_string(saved_bytes) +
                                         " bytes, the training forward's workspace is " +
                                         std::to_string(F.total));
  }
  if (g.w0_stride != 0 && g.w0_stride != g.d * g.f)
    return fail(TTT_ERR_UNSUPPORTED,
                "the backward needs per-sequence W_down0 at stride d_model * d_ff (or shared)");
  const BwdLayout L = backward_layout(g, sv);
  if (workspace_bytes < L.total)
    return fail(TTT_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " bytes, needs " + std::to_string(L.total));
  const size_t ab = g.act_bytes(), wb = g.w_bytes();
  const int64_t df = g.d * g.f;
  const size_t w0_bytes = g.w0_stride == 0 ? df * wb : g.B * df * wb;
  std::vector<Range> inputs = {range_of("H", H, g.B * g.T * g.d * ab),
                               range_of("X0", X0, g.B * g.T * g.d * ab),
                               range_of("Wg", Wg, g.f * g.d * wb),
                               range_of("Wu", Wu, g.f * g.d * wb),
                               range_of("W_down0", W_down0, w0_bytes),
                               range_of("conv_taps", conv_taps, g.K * g.d * wb),
                               range_of("W_target", W_target, g.d * g.d * wb),
                               range_of("dO", dO, g.B * g.T * g.d * ab)};
  if (dW_final != nullptr) inputs.push_back(range_of("dW_final", dW_final, g.B * df * 4));
  if (sv) inputs.push_back(range_of("saved", saved, F.total));
  const std::vector<Range> outputs = {
      range_of("dH", dH, g.B * g.T * g.d * 4), range_of("dX0", dX0, g.B * g.T * g.d * 4),
      range_of("dWg", dWg, df * 4), range_of("dWu", dWu, df * 4),
      range_of("dW_down0", dW_down0, (g.w0_stride == 0 ? 1 : g.B) * df * 4),
      range_of("dtaps", dtaps, g.K * g.d * 4), range_of("dW_target", dW_target, g.d * g.d * 4),
      range_of("workspace", workspace, L.total)};
  TTT_TRY(check_aliasing(inputs, outputs));

  hipStream_t s = static_cast<hipStream_t>(stream);
  const tttk::Dims& D = g.dims;
  const int B = (int)g.B, T = (int)g.T, d = (int)g.d, f = (int)g.f, C = (int)g.C;
  const int nch = (int)g.nchunks;
  const int64_t snap_df = tttk::sb_elems<256>(g.d, g.f);
  uint32_t* range = at<uint32_t>(workspace, L.range);
  uint32_t* range_y = range + tttk::kRangeY * tttk::kRangeSlots;
  uint32_t* range_wt = range + tttk::kRangeWt * tttk::kRangeSlots;
  TTT_LAUNCH("range_clear", s, tttk::launch_range_clear(range, s));

  // bf16 operands; dO goes to the first d columns of [dO | eta V]
  const uint16_t* Hb = static_cast<const uint16_t*>(H);
  const uint16_t* X0b = static_cast<const uint16_t*>(X0);
  if (g.act_f32) {
    const int64_t n = g.B * g.T * g.d;
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(H), at<uint16_t>(workspace, L.hb), n, s));
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(X0), at<uint16_t>(workspace, L.x0b), n, s));
    Hb = at<uint16_t>(workspace, L.hb);
    X0b = at<uint16_t>(workspace, L.x0b);
  }
  uint16_t* DOV = at<uint16_t>(workspace, L.dov);
  TTT_LAUNCH("bwd_rows", s,
             tttk::launch_rows_bf16(dO, g.act_f32, g.d, DOV, L.ld_ov, g.B * g.T, d, s));

  // The forward's activations again (bf16 for the backward's contractions);
  // Z, Z^T and the SiLU factors from the training forward when it saved them.
  auto saved_at = [&](size_t off) { return reinterpret_cast<const char*>(saved) + off; };
  uint16_t* Wgp = sv ? nullptr : at<uint16_t>(workspace, L.wgp);
  uint16_t* Wup = sv ? nullptr : at<uint16_t>(workspace, L.wup);
  if (!sv) {
    TTT_LAUNCH("pack_weights", s, tttk::launch_pack_weight(Wg, g.w_f32, Wgp, D, s));
    TTT_LAUNCH("pack_weights", s, tttk::launch_pack_weight(Wu, g.w_f32, Wup, D, s));
  }
  uint16_t* Y = at<uint16_t>(workspace, L.y);
  uint16_t* WtT = at<uint16_t>(workspace, L.wtt);
  uint16_t* YT = at<uint16_t>(workspace, L.yt);
  TTT_LAUNCH("amax", s, tttk::launch_amax(W_target, g.w_f32, g.d * g.d, range_wt, s));
  TTT_LAUNCH("transpose_w_target", s,
             tttk::launch_transpose_f16(W_target, g.w_f32, WtT, d, d, D.ld_y, range_wt, s));
  TTT_LAUNCH("conv", s,
             tttk::launch_conv(X0b, nullptr, 0, conv_taps, g.w_f32, Y, D, (int)g.K, C,
                               g.pad_chunk, nullptr, range_y, s, YT));
  TTT_LAUNCH("conv_repair", s,
             tttk::launch_conv_repair(X0b, nullptr, 0, conv_taps, g.w_f32, Y, D, (int)g.K, C,
                                      g.pad_chunk, nullptr, range_y, s));
  const uint16_t* Z;
  const uint16_t* ZT;
  const uint32_t* SA;
  if (sv) {
    Z = reinterpret_cast<const uint16_t*>(saved_at(F.z));
    ZT = reinterpret_cast<const uint16_t*>(saved_at(F.ztb));
    SA = reinterpret_cast<const uint32_t*>(saved_at(F.sa));
  } else {
    uint16_t* z = at<uint16_t>(workspace, L.z);
    uint16_t* zt = at<uint16_t>(workspace, L.zt);
    uint32_t* sa = at<uint32_t>(workspace, L.sa);
    TTT_LAUNCH("bwd_gate_up", s, tttk::launch_gate_up_bwd(Hb, Wgp, Wup, z, zt, sa, D, s));
    Z = z;
    ZT = zt;
    SA = sa;
  }
  uint16_t* VT = at<uint16_t>(workspace, L.vt);
  TTT_LAUNCH("bwd_target", s,
             tttk::launch_target_bwd(Y, WtT, VT, DOV + g.d, L.ld_ov, eta, D, range, s));
  uint16_t* DOT = at<uint16_t>(workspace, L.dot);
  uint16_t* HT = at<uint16_t>(workspace, L.ht);
  TTT_LAUNCH("bwd_to_slab", s,
             tttk::launch_to_slab(dO, g.act_f32, g.d, DOT, B, T, (int)g.T_pad, d, false, s));
  TTT_LAUNCH("bwd_to_slab", s,
             tttk::launch_to_slab(Hb, false, g.d, HT, B, T, (int)g.T_pad, d, true, s));

  // The states W_i of every chunk (bf16 sb<256>(d x f)): the training
  // forward's snapshots, or the forward's update again on bf16 operands.
  const uint16_t* WS;
  if (sv) {
    WS = reinterpret_cast<const uint16_t*>(saved_at(F.snap));
  } else {
    uint16_t* ws = at<uint16_t>(workspace, L.ws);
    TTT_LAUNCH("bwd_states", s,
               tttk::launch_contract_bf16(ZT, VT, D, W_down0, g.w_f32, false, g.w0_stride, g.f,
                                          ws, g.nchunks * snap_df, f, nullptr, false, C, s));
    WS = ws;
  }
  // The state gradients Gbar_{i+1} = dW_final + sum_{j > i} dO_j^T Z_j of
  // every chunk, backwards over the tokens (the scan ends at dW_down0).
  uint16_t* GS = at<uint16_t>(workspace, L.gs);
  float* dw0_all = (g.w0_stride == 0 && g.B > 1) ? at<float>(workspace, L.dw0) : dW_down0;
  TTT_LAUNCH("bwd_state_grads", s,
             tttk::launch_contract_bf16(ZT, DOT, D, dW_final, true, false, df, g.f, GS,
                                        g.nchunks * snap_df, f, dw0_all, true, C, s));
  if (dw0_all != dW_down0)
    TTT_LAUNCH("bwd_sum", s, tttk::launch_sum_parts(dw0_all, df, B, dW_down0, df, s));

  // dZ (and through the SiLU's backward, dG and dU), then dV.
  uint16_t* DGU = at<uint16_t>(workspace, L.dgu);
  uint16_t* DGT = at<uint16_t>(workspace, L.dgt);
  uint16_t* DUT = at<uint16_t>(workspace, L.dut);
  TTT_LAUNCH("bwd_dz", s,
             tttk::launch_act_gemm_dz(DOV, L.ld_ov, WS, g.nchunks * snap_df, snap_df, GS,
                                      g.nchunks * snap_df, snap_df, d, f, C, nch, SA, DGU,
                                      L.ld_gu, DGT, DUT, D, s));
  uint16_t* DV = at<uint16_t>(workspace, L.dv);
  uint16_t* DVT = at<uint16_t>(workspace, L.dvt);
  TTT_LAUNCH("bwd_dv", s,
             tttk::launch_act_gemm_dv(Z, D.ld_z, GS, g.nchunks * snap_df, snap_df, d, f, C, nch,
                                      eta, DV, g.d, DVT, D, s));

  // The target's and the conv's backward.
  const uint16_t* Wtb = static_cast<const uint16_t*>(W_target);
  if (g.w_f32) {
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(W_target),
                                                      at<uint16_t>(workspace, L.wtb), g.d * g.d, s));
    Wtb = at<uint16_t>(workspace, L.wtb);
  }
  float* DY = at<float>(workspace, L.dy);
  TTT_LAUNCH("bwd_dy", s, tttk::launch_nt_gemm(DV, g.d, Wtb, g.d, d, d, DY, g.d, D, s));
  TTT_LAUNCH("bwd_conv", s,
             tttk::launch_conv_bwd(DY, X0b, conv_taps, g.w_f32, dX0, dtaps,
                                   at<float>(workspace, L.part), B, T, d, (int)g.K, C,
                                   g.pad_chunk, s));
  const tttk::Dims Dflat_dd = tttk::make_dims(1, (int)(g.B * g.T_pad), d, d);
  TTT_LAUNCH("bwd_dw_target", s,
             tttk::launch_contract_bf16(DVT, YT, Dflat_dd, nullptr, true, false, 0, 0, nullptr,
                                        0, 0, dW_target, false, 64, s));

  // The gated MLP's weight gradients and dH.
  const tttk::Dims Dflat_fd = tttk::make_dims(1, (int)(g.B * g.T_pad), f, d);
  TTT_LAUNCH("bwd_dw_gate_up", s,
             tttk::launch_contract_bf16(HT, DGT, Dflat_fd, nullptr, true, false, 0, 0, nullptr,
                                        0, 0, dWg, false, 64, s));
  TTT_LAUNCH("bwd_dw_gate_up", s,
             tttk::launch_contract_bf16(HT, DUT, Dflat_fd, nullptr, true, false, 0, 0, nullptr,
                                        0, 0, dWu, false, 64, s));
  uint16_t* WGUT = at<uint16_t>(workspace, L.wgut);
  // [Wg ; Wu] transposed with the rows of Wg and Wu interleaved, as dG and dU
  // are in dgu.
  TTT_LAUNCH("bwd_transpose_w", s,
             tttk::launch_transpose_bf16(Wg, g.w_f32, WGUT, f, d, L.ld_gu, 2, s));
  TTT_LAUNCH("bwd_transpose_w", s,
             tttk::launch_transpose_bf16(Wu, g.w_f32, WGUT + 1, f, d, L.ld_gu, 2, s));
  TTT_LAUNCH("bwd_dh", s,
             tttk::launch_nt_gemm(DGU, L.ld_gu, WGUT, L.ld_gu, d, 2 * f, dH, g.d, D, s));
  return TTT_OK;
}

}  // namespace

extern "C" {

ttt_status ttt_backward_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = backward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_layer_backward(const ttt_desc* desc, const void* H, const void* X0,
                              const void* Wg, const void* Wu, const void* W_down0,
                              const void* conv_taps, const void* W_target, float eta,
                              int32_t chunk, const void* dO, const float* dW_final, float* dH,
                              float* dX0, float* dWg, float* dWu, float* dW_down0, float* dtaps,
                              float* dW_target, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  return backward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, nullptr, 0, dO,
                       dW_final, dH, dX0, dWg, dWu, dW_down0, dtaps, dW_target, workspace,
                       workspace_bytes, stream);
}

ttt_status ttt_train_workspace_size(const ttt_desc* desc, int32_t chunk, size_t* bytes) {
  Geo g;
  TTT_TRY(check_train_desc(desc, chunk, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = forward_layout(g).total;
  return TTT_OK;
}

ttt_status ttt_layer_forward_train(const ttt_desc* desc, const void* H, const void* X0,
                                   const void* Wg, const void* Wu, const void* W_down0,
                                   const void* conv_taps, const void* W_target, float eta,
                                   int32_t chunk, void* O, float* W_down_final, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_train_desc(desc, chunk, &g));
  return forward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, O, W_down_final,
                      workspace, workspace_bytes, stream);
}

ttt_status ttt_backward_saved_workspace_size(const ttt_desc* desc, int32_t chunk,
                                             size_t* bytes) {
  Geo g;
  TTT_TRY(check_train_desc(desc, chunk, &g));
  if (bytes == nullptr) return fail(TTT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = backward_layout(g, true).total;
  return TTT_OK;
}

ttt_status ttt_layer_backward_saved(const ttt_desc* desc, const void* H, const void* X0,
                                    const void* Wg, const void* Wu, const void* W_down0,
                                    const void* conv_taps, const void* W_target, float eta,
                                    int32_t chunk, const void* saved, size_t saved_bytes,
                                    const void* dO, const float* dW_final, float* dH, float* dX0,
                                    float* dWg, float* dWu, float* dW_down0, float* dtaps,
                                    float* dW_target, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  Geo g;
  TTT_TRY(check_train_desc(desc, chunk, &g));
  TTT_TRY(check_ptr(saved, "saved", 256));
  return backward_impl(g, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, saved, saved_bytes,
                       dO, dW_final, dH, dX0, dWg, dWu, dW_down0, dtaps, dW_target, workspace,
                       workspace_bytes, stream);
}

ttt_status ttt_gated_activation(const ttt_desc* desc, const void* H, const void* Wg,
                                const void* Wu, void* Z, void* workspace, size_t workspace_bytes,
                                void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_ptr(H, "H"));
  TTT_TRY(check_ptr(Wg, "Wg"));
  TTT_TRY(check_ptr(Wu, "Wu"));
  TTT_TRY(check_ptr(Z, "Z"));
  const Layout L = step_layout(g);
  if (L.total > 0) TTT_TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < L.total)
    return fail(TTT_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " bytes, needs " + std::to_string(L.total));
  const size_t ab = g.act_bytes(), wb = g.w_bytes();
  TTT_TRY(check_aliasing({range_of("H", H, g.B * g.T * g.d * ab),
                          range_of("Wg", Wg, g.f * g.d * wb),
                          range_of("Wu", Wu, g.f * g.d * wb)},
                         {range_of("Z", Z, g.B * g.T * g.f * 2),
                          range_of("workspace", workspace, L.total)}));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* Hb = static_cast<const uint16_t*>(H);
  if (g.act_f32) {
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(H),
                                                      at<uint16_t>(workspace, L.hb), g.B * g.T * g.d, s));
    Hb = at<uint16_t>(workspace, L.hb);
  }
  tttk::Dims D = g.dims;
  D.ld_z = g.f;  // the caller's Z is dense [B, T, d_ff]
  uint16_t* Wgp = at<uint16_t>(workspace, L.wgp);
  uint16_t* Wup = at<uint16_t>(workspace, L.wup);
  TTT_LAUNCH("pack_weights", s, tttk::launch_pack_weight(Wg, g.w_f32, Wgp, D, s));
  TTT_LAUNCH("pack_weights", s, tttk::launch_pack_weight(Wu, g.w_f32, Wup, D, s));
  TTT_LAUNCH("gate_up", s,
             tttk::launch_gate_up(Hb, Wgp, Wup, static_cast<uint16_t*>(Z), nullptr, D, nullptr, s));
  return TTT_OK;
}

ttt_status ttt_lm_target(const ttt_desc* desc, const void* X0, const void* conv_taps,
                         const void* W_target, int32_t chunk, void* V, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Geo g;
  TTT_TRY(check_desc(desc, &g));
  TTT_TRY(check_chunk(chunk, &g));
  TTT_TRY(check_ptr(X0, "X0"));
  TTT_TRY(check_ptr(conv_taps, "conv_taps"));
  TTT_TRY(check_ptr(W_target, "W_target"));
  TTT_TRY(check_ptr(V, "V"));
  TTT_TRY(check_ptr(workspace, "workspace", 256));
  const Layout L = step_layout(g);
  if (workspace_bytes < L.total)
    return fail(TTT_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " bytes, needs " + std::to_string(L.total));
  const size_t ab = g.act_bytes(), wb = g.w_bytes();
  TTT_TRY(check_aliasing({range_of("X0", X0, g.B * g.T * g.d * ab),
                          range_of("conv_taps", conv_taps, g.K * g.d * wb),
                          range_of("W_target", W_target, g.d * g.d * wb)},
                         {range_of("V", V, g.B * g.T * g.d * 2),
                          range_of("workspace", workspace, L.total)}));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* X0b = static_cast<const uint16_t*>(X0);
  if (g.act_f32) {
    TTT_LAUNCH("cast_bf16", s, tttk::launch_cast_bf16(static_cast<const float*>(X0),
                                                      at<uint16_t>(workspace, L.x0b), g.B * g.T * g.d, s));
    X0b = at<uint16_t>(workspace, L.x0b);
  }
  uint16_t* Y = at<uint16_t>(workspace, L.y);
  uint16_t* WtT = at<uint16_t>(workspace, L.wtt);
  uint32_t* range = at<uint32_t>(workspace, L.range);
  uint32_t* range_y = range + tttk::kRangeY * tttk::kRangeSlots;
  TTT_LAUNCH("range_clear", s, tttk::launch_range_clear(range, s));
  TTT_LAUNCH("amax", s,
             tttk::launch_amax(W_target, g.w_f32, g.d * g.d, range + tttk::kRangeWt * tttk::kRangeSlots, s));
  TTT_LAUNCH("transpose_w_target", s,
             tttk::launch_transpose_f16(W_target, g.w_f32, WtT, (int)g.d, (int)g.d, g.dims.ld_y,
                                        range + tttk::kRangeWt * tttk::kRangeSlots, s));
  TTT_LAUNCH("conv", s,
             tttk::launch_conv(X0b, nullptr, 0, conv_taps, g.w_f32, Y, g.dims, (int)g.K,
                               (int)g.C, g.pad_chunk, nullptr, range_y, s));
  TTT_LAUNCH("conv_repair", s,
             tttk::launch_conv_repair(X0b, nullptr, 0, conv_taps, g.w_f32, Y, g.dims, (int)g.K,
                                      (int)g.C, g.pad_chunk, nullptr, range_y, s));
  TTT_LAUNCH("target", s,
             tttk::launch_target(Y, WtT, nullptr, static_cast<uint16_t*>(V), nullptr, 1.0f,
                                 g.dims, range, s));
  return TTT_OK;
}

ttt_status ttt_copy_calibration(void* dst, const void* src, size_t bytes, void* stream) {
  TTT_TRY(check_ptr(dst, "dst"));
  TTT_TRY(check_ptr(src, "src"));
  if (bytes % 16 != 0) return fail(TTT_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  TTT_TRY(check_aliasing({range_of("src", src, bytes)}, {range_of("dst", dst, bytes)}));
  hipStream_t s = static_cast<hipStream_t>(stream);
  TTT_LAUNCH("calibration_copy", s, tttk::launch_copy(src, dst, (int64_t)bytes, s));
  return TTT_OK;
}

ttt_status ttt_profile_enable(int32_t on) {
  for (auto& r : g_timing.recs) {
    g_timing.pool.push_back(r.start);
    g_timing.pool.push_back(r.stop);
  }
  g_timing.recs.clear();
  g_timing.on = on != 0;
  return TTT_OK;
}

int32_t ttt_profile_read(ttt_kernel_stat* out, int32_t max_entries) {
  std::vector<ttt_kernel_stat> stats;
  for (auto& r : g_timing.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      ttt_kernel_stat* st = nullptr;
      for (auto& x : stats)
        if (std::strcmp(x.name, r.name) == 0) st = &x;
      if (st == nullptr) {
        stats.push_back({});
        st = &stats.back();
        std::snprintf(st->name, sizeof(st->name), "%s", r.name);
      }
      st->launches += 1;
      st->total_ms += ms;
    }
    g_timing.pool.push_back(r.start);
    g_timing.pool.push_back(r.stop);
  }
  g_timing.recs.clear();
  const int32_t n = (int32_t)stats.size();
  for (int32_t i = 0; i < n && i < max_entries && out != nullptr; ++i) out[i] = stats[i];
  return n;
}

}  // extern "C"
