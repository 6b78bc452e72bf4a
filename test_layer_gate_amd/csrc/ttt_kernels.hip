// gfx950 (CDNA4) kernels of the In-Place TTT gated-MLP prefill.
//
// The four dense contractions (gate/up projection, target projection, the
// fast-weight update and the apply) share one MFMA GEMM core:
//   C[M][N] = sum_k A[m][k] * B[n][k],  both operands K-contiguous in HBM.
// A workgroup is NW wave64s (8 in every kernel here, two per SIMD) in a
// WGM x WGN grid; each wave owns a block of 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation). K advances BK
// elements (32 or 64) per step through LDS stages, NSTA of the A tile and
// NSTB of the B tile: buffer_load ... lds moves each 16-byte chunk from HBM
// straight into LDS (no VGPR staging), bounds-checked by the buffer
// descriptor (rows past the tile's valid rows read as zero), while the MFMAs
// run on a stage that has landed; each operand has all but one of its stages
// in flight. Fragments are read with ds_read_b128 one K-substep ahead of the
// MFMAs that use them; each step is laid out by hand (one read and one load
// after each MFMA).
//
// Method sources: "论文精读：In-Place Test-Time Training" reading notes —
// "In-Place 设计" (gated MLP), "Chunk-Wise 更新机制" (update equation),
// "LM-Aligned 目标函数" (target equation); iplexlaw explainer of In-Place
// Test-Time Training, §3 (apply, then update) and §6 (exclusive prefix over
// chunk deltas).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_device.h"
#include "ttt_launch.h"

namespace tttk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;      // small kernels
constexpr int kMaxStages = 6;      // LDS stages of one operand (all but one in flight)
constexpr int kRsrcWord3 = 0x00020000;
enum { kRowMajor = 0, kSlab = 1 };  // LDS / HBM layouts of a GEMM operand (see Operand)
constexpr int kCpolNt = 2, kCpolSc1 = 16;  // cache-policy bits of buffer instructions

struct Bf16Mma {
  static __device__ __forceinline__ f32x16 mma(const uint4& a, const uint4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

struct F16Mma {
  static __device__ __forceinline__ f32x16 mma(const uint4& a, const uint4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// LDS tile of `rows` x BK 16-bit elements, 2 * BK bytes per row, CPR = BK / 8
// 16-byte chunks per row. Chunk kc of row r sits at physical chunk
// kc ^ swz(r), chosen so that any 8 consecutive rows read at one logical
// chunk fall on 8 distinct 16-byte bank groups of the 128-byte bank line
// (one ds_read_b128 pass): with 128-byte rows the 8 rows need 8 distinct
// chunk positions; with 64-byte rows, rows 2i and 2i + 1 share a bank line
// at opposite halves, so the 4 even (and the 4 odd) rows need 4 distinct
// positions. swz depends on row % 32 only, so a lane's permutation is the
// same for every 32-row fragment it reads and each read is one per-lane
// register plus an immediate offset.
template <int BK>
struct Swz {
  static_assert(BK == 32 || BK == 64, "BK");
  static constexpr int CPR = BK / 8;   // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;  // rows per 1 KB direct-to-LDS block
  static __device__ __forceinline__ int swz(int row) {
    return BK == 64 ? (row ^ ((row >> 3) & 3)) & 7 : (row >> 1) & 3;
  }
  static __device__ __forceinline__ int off(int row, int kc) {
    return row * BK + ((kc ^ swz(row)) << 3);
  }
};

// A slab operand keeps its HBM image in LDS: piece kc of row r at element
// (r / 32) * 2048 + (kc / 2) * 512 + ((kc % 2) * 32 + r % 32) * 8. A
// fragment read (32 consecutive rows from a multiple of 32, lanes 32-63 at
// kc + 1 with kc even) is then one contiguous, conflict-free 1 KB.
__device__ __forceinline__ int slab_off(int row, int kc) {
  return (row >> 5) * 2048 + (kc >> 1) * 512 + ((kc & 1) * 32 + (row & 31)) * 8;
}

template <int BK, int LAY>
__device__ __forceinline__ uint4 lds_frag(const u16* lds, int row, int kc) {
  return *reinterpret_cast<const uint4*>(lds + (LAY == kSlab ? slab_off(row, kc)
                                                             : Swz<BK>::off(row, kc)));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor of `bytes` bytes at `base` (raw, no stride): reads at
// offsets >= bytes return zero.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  // The descriptor must sit in SGPRs: every lane holds the same value.
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = kRsrcWord3;
  return r;
}

// Direct-to-LDS loads, written as inline asm so that the compiler does not
// track them: it would otherwise wait for every such load before any later
// LDS read, which serialises the pipeline. They have no register results;
// completion is tracked only by the explicit vmcnt waits in the pipeline.
// M0 holds the LDS byte address of lane 0; one wait state separates the M0
// write from the load. The compiler warns that M0 is a reserved register in
// the clobber list; no compiler-generated code in these kernels reads or
// writes M0 (every M0 access in their assembly is one of these loads'), so
// there is nothing for the clobber to protect.
__device__ __forceinline__ void lds_dma_b128(const u32x4& rsrc, uint32_t lds_addr,
                                             uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}

// LDS byte address of p, which must be the same in every lane of the wave
// (it becomes M0).
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// A GEMM operand in HBM as the core reads it: the tile's rows of K step kt
// (BK elements) start at byte kt * step_bytes from base. Row-major (kRowMajor):
// the 16-byte piece kc (K elements 8kc .. 8kc + 7) of row r is at
// r * row_bytes + kc * 16 from there. Slab (kSlab, the sb layout of
// ttt_launch.h, BK = 64): the step is one contiguous slab of rows * 128
// bytes, with piece kc of row r at (r / 32) * 4096 + (kc / 2) * 1024 +
// ((kc % 2) * 32 + r % 32) * 16. Reads at or past `bytes` from base return
// zero.
struct Operand {
  const u16* base;
  uint32_t row_bytes, step_bytes, bytes;
};

// Row-major [rows][ld] with K contiguous; rows at or past rows_valid read as
// zero.
template <int BK>
__device__ __forceinline__ Operand row_major(const u16* base, int64_t ld, int rows_valid) {
  int64_t bytes = rows_valid > 0 ? (int64_t)rows_valid * ld * 2 : 0;
  if (bytes > 0xffffffffLL) bytes = 0xffffffffLL;
  return {base, (uint32_t)(ld * 2), (uint32_t)(BK * 2), (uint32_t)bytes};
}

// Blocked [nk][rows][BK]: each K step of the tile is one contiguous slab.
template <int BK>
__device__ __forceinline__ Operand blocked(const u16* base, int rows, int nk) {
  int64_t bytes = (int64_t)nk * rows * (BK * 2);
  if (bytes > 0xffffffffLL) bytes = 0xffffffffLL;
  return {base, (uint32_t)(BK * 2), (uint32_t)(rows * BK * 2), (uint32_t)bytes};
}

// The SR-row slab row of an sb<SR> matrix at m (K columns) that starts at
// row r0 (a multiple of SR), from column k0 (a multiple of 64) on; the GEMM
// tile is the SR rows and steps 64 columns at a time.
template <int SR>
__device__ __forceinline__ Operand slab_blocked(const u16* m, int64_t K, int r0, int64_t k0) {
  int64_t bytes = (K - k0) / 64 * (SR * 128);
  if (bytes > 0xffffffffLL) bytes = 0xffffffffLL;
  return {m + sb_offset<SR>(r0, k0, K), 4096u, (uint32_t)(SR * 128), (uint32_t)bytes};
}

// One operand tile of ROWS rows, loaded in blocks of RPB rows (1 KB): one
// direct-to-LDS load (64 lanes x 16 bytes) fills block b. Row-major: lane l
// the 16 bytes at physical chunk l % CPR of row RPB * b + l / CPR, which is
// that row's logical chunk (l % CPR) ^ swz(row). Slab: lane l the 16 bytes
// at 1024 b + 16 l of the slab, copied as they are. Every wave issues
// NI = ceil(blocks / waves) loads per K step, load i of wave w covering block
// (waves * i + w) mod blocks; when the blocks do not divide evenly the extra
// loads repeat a block, writing the same bytes to the same place. The
// per-lane byte offsets are fixed; the K step enters as the scalar offset.
// The LDS side is all scalar: the stage's 32-bit LDS byte address plus the
// wave's block offsets, so that setting M0 for a load is one scalar add
// (no per-load conversion of a generic pointer, which cost two
// readfirstlanes and a null check per load, issued ahead of the MFMAs).
template <int ROWS, int BK, int LAY, int NW>
struct DmaTile {
  using S = Swz<BK>;
  static constexpr int NB = ROWS / S::RPB;
  static constexpr int NI = (NB + NW - 1) / NW;
  static constexpr uint32_t kBlockBytes = S::RPB * BK * 2;  // 1 KB
  static_assert(ROWS % S::RPB == 0, "rows");
  static_assert(LAY == kRowMajor || (BK == 64 && ROWS % 32 == 0), "slab tiles");
  uint32_t voff[NI];
  uint32_t loff[NI];  // wave-uniform: LDS byte offset of load i within a stage
  uint32_t step_bytes;
  u32x4 rsrc;
  // wave must be the same in every lane of the wave (a scalar).
  __device__ __forceinline__ void init(const Operand& op, int wave, int lane) {
    rsrc = make_rsrc(op.base, op.bytes);
    step_bytes = op.step_bytes;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int block = (NW * i + wave) % NB;
      loff[i] = (uint32_t)block * kBlockBytes;
      const int row = block * S::RPB + lane / S::CPR;
      const int kc = (lane % S::CPR) ^ S::swz(row);
      voff[i] = LAY == kSlab ? (uint32_t)block * 1024 + lane * 16
                             : (uint32_t)row * op.row_bytes + kc * 16;
    }
  }
  // The scalar byte offset of K step kt.
  __device__ __forceinline__ uint32_t soff(int kt) const {
    return __builtin_amdgcn_readfirstlane((uint32_t)kt * step_bytes);
  }
  // Load i of K step kt (scalar offset so) into the stage at LDS byte
  // address lds_stage.
  __device__ __forceinline__ void issue_one(uint32_t lds_stage, uint32_t so, int i) const {
    lds_dma_b128(rsrc, lds_stage + loff[i], voff[i], so);
  }
  // All loads of K step kt.
  __device__ __forceinline__ void issue(uint32_t lds_stage, int kt) const {
    const uint32_t so = soff(kt);
#pragma unroll
    for (int i = 0; i < NI; ++i) issue_one(lds_stage, so, i);
  }
};

// The LDS of a GEMM workgroup: NST stages of the A tile (BM * BK elements)
// and NST of the B tile (BN * BK) (the epilogues reuse the whole array once
// the core has returned).
#define TTT_GEMM_LDS(var, BM_, BN_, BK_, NST_)                                  \
  static_assert((NST_) >= 2 && (NST_) <= kMaxStages, "stages");                 \
  __shared__ __attribute__((aligned(16))) u16 var[(NST_) * ((BM_) + (BN_)) * (BK_)];
// The same with NSTA stages of the A tile and NSTB of the B tile.
#define TTT_GEMM_LDS_AB(var, BM_, BN_, BK_, NSTA_, NSTB_)                       \
  static_assert((NSTA_) >= 2 && (NSTB_) >= 2 && (NSTA_) <= kMaxStages && (NSTB_) <= kMaxStages, \
                "stages");                                                              \
  __shared__ __attribute__((aligned(16))) u16 var[((NSTA_) * (BM_) + (NSTB_) * (BN_)) * (BK_)];

// Waits until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order) and all of its LDS reads have
// returned, then joins the workgroup barrier. This replaces __syncthreads()
// in the pipeline: that one carries a release fence, which waits for every
// outstanding load, including the stages meant to stay in flight. The
// "memory" clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Maps the linear workgroup id to (batch, tile_m, tile_n). Workgroups are
// handed to the 8 XCDs in turn, so ids are first renumbered so that each XCD
// runs one contiguous range of tiles; within a range, tiles go in groups of
// group_m rows of tiles, M fastest, so that the workgroups resident on one
// XCD share A and B slices through its L2.
struct TileIdx {
  int b, tm, tn;
};

// Position p of a range of `count` workgroups that starts at a multiple of
// 8 renumbered so that the workgroups of one XCD form one contiguous range
// (workgroup ids go to the XCDs in turn, so p & 7 is the XCD).
__device__ __forceinline__ int xcd_contiguous(int p, int count) {
  const int xcd = p & 7, idx = p >> 3;
  const int per = count >> 3, rem = count & 7;
  return xcd * per + min(xcd, rem) + idx;
}

// The workgroup id renumbered so that the workgroups of one XCD form one
// contiguous range of ids.
__device__ __forceinline__ int xcd_contiguous_id() {
  return xcd_contiguous(blockIdx.x, gridDim.x);
}

// Tile coordinates of the linear tile id lin: batch-major, then groups of
// group_m tile rows, M fastest within a group.
__device__ __forceinline__ TileIdx tile_coords(int lin, int tiles_m, int tiles_n, int group_m) {
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

__device__ __forceinline__ TileIdx tile_index(int tiles_m, int tiles_n, int group_m) {
  return tile_coords(xcd_contiguous_id(), tiles_m, tiles_n, group_m);
}

// A K-step hook: called with the accumulators at the start of a K step,
// returns whether it issued stores, and then issued exactly kStores vector
// memory instructions in every wave (the pipeline's waits count them).
struct NoHook {
  static constexpr int kStores = 0;
  __device__ __forceinline__ bool operator()(int, f32x16*) const { return false; }
};

// Waits as wait_and_barrier<BASE + c * STEP> for a runtime c in [0, C].
template <int BASE, int STEP, int C>
__device__ __forceinline__ void wait_and_barrier_var(int c) {
  if constexpr (C == 0) {
    wait_and_barrier<BASE>();
  } else {
    if (c == C)
      wait_and_barrier<BASE + C * STEP>();
    else
      wait_and_barrier_var<BASE, STEP, C - 1>(c);
  }
}

template <int TM, int TN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[TM][TN]) {
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n) acc[m][n] = f32x16{};
}

// Wave layout of a BM x BN GEMM tile: WGM x WGN waves (WGM * WGN = NW), each
// owning TM x TN MFMA tiles of 32 x 32.
template <int BM, int BN, int WGM, int NW>
struct Layout {
  static constexpr int NWAVES = NW;
  static constexpr int WGN = NW / WGM;
  static constexpr int TM = BM / (32 * WGM);
  static constexpr int TN = BN / (32 * WGN);
  static_assert(TM >= 1 && TN >= 1 && TM * 32 * WGM == BM && TN * 32 * WGN == BN, "layout");
};

// The GEMM core. acc[m * TN + n] is the 32x32 MFMA tile (m, n) of this wave
// (wave w = (wm, wn) with wm = w / WGN, wn = w % WGN); its register r holds
// output row wm*TM*32 + m*32 + 8*(r/4) + 4*(lane/32) + r%4 and column
// wn*TN*32 + n*32 + lane%32.
// SPLITB: the B tile is BN/2 rows of B0 followed by BN/2 rows of B1 (the
// gate and up projections); wave wn then owns the same TN/2 * 32 columns of
// each, in acc[.][0, TN/2) (B0) and acc[.][TN/2, TN) (B1).
// hook(kt, acc) runs at the start of K step kt, when acc holds steps < kt;
// from step 1 on, after that step's loads of the shorter-distance operand
// (issued right after the previous barrier) and before its spread loads of
// the other operand, so that its stores need to be complete only R steps
// later (the waits in between allow for them).
// nk is the number of BK-wide K steps. lds holds NSTA stages of the A tile
// (BM * BK elements each) followed by NSTB stages of the B tile (BN * BK);
// the A loads run NSTA - 1 steps ahead and the B loads NSTB - 1, so the LDS
// left after two stages of each can buy the operand that misses more an
// extra step of latency. Step kt reads K block (kt + k0) mod
// nk (k0 in [0, nk)): tiles that share an operand slab but start at
// different k0 reach it at different times, so one of them misses in L2 and
// the others then hit, instead of all waiting on the same miss. A hook
// needs k0 = 0.
template <int NW, int BM, int BN, int WGM, int BK, int NSTA, int NSTB, class Op, bool SPLITB,
          int ALAY, int BLAY, class Hook>
__device__ __forceinline__ void gemm_core_ab(const Operand& A, const Operand& B0,
                                             const Operand& B1, int nk, f32x16* acc, u16* lds,
                                             const Hook& hook, int k0 = 0) {
  using Lay = Layout<BM, BN, WGM, NW>;
  constexpr int TM = Lay::TM, TN = Lay::TN, WGN = Lay::WGN;
  constexpr int BROWS = SPLITB ? BN / 2 : BN;
  constexpr int KSUB = BK / 16;  // MFMA K-substeps per stage
  static_assert(NSTA >= 2 && NSTB >= 2 && NSTA <= kMaxStages && NSTB <= kMaxStages && KSUB >= 2,
                "pipeline");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WGN, wn = w % WGN;
  if (nk <= 0) return;

  // The wave index as a scalar, so that the loads' LDS offsets are scalars.
  const int ws = __builtin_amdgcn_readfirstlane(w);
  DmaTile<BM, BK, ALAY, NW> ta;
  DmaTile<BROWS, BK, BLAY, NW> tb0;
  DmaTile<SPLITB ? BN / 2 : 32, BK, BLAY, NW> tb1;  // unused unless SPLITB
  ta.init(A, ws, lane);
  tb0.init(B0, ws, lane);
  if constexpr (SPLITB) tb1.init(B1, ws, lane);

  u16* const ldsb = lds + NSTA * BM * BK;
  auto stage_a = [&](int i) { return lds + i * (BM * BK); };
  auto stage_b = [&](int i) { return ldsb + i * (BN * BK); };
  // The same stages as LDS byte addresses, for the loads.
  const uint32_t lds0 = lds_addr_of(lds);
  auto addr_a = [&](int i) { return lds0 + (uint32_t)(i * (BM * BK * 2)); };
  auto addr_b = [&](int i) { return lds0 + (uint32_t)((NSTA * BM + i * BN) * BK * 2); };
  auto kblock = [&](int kt) {
    kt += k0;
    return kt >= nk ? kt - nk : kt;
  };
  auto issue_a = [&](int st, int kt) { ta.issue(addr_a(st), kblock(kt)); };
  auto issue_b = [&](int st, int kt) {
    tb0.issue(addr_b(st), kblock(kt));
    if constexpr (SPLITB) tb1.issue(addr_b(st) + (uint32_t)((BN / 2) * BK * 2), kblock(kt));
  };

  // Rows of this lane's fragments within the A and B stages.
  int arow[TM], brow[TN];
#pragma unroll
  for (int m = 0; m < TM; ++m) arow[m] = wm * TM * 32 + m * 32 + (lane & 31);
#pragma unroll
  for (int n = 0; n < TN; ++n) {
    if constexpr (SPLITB) {
      constexpr int H = TN / 2;
      brow[n] =
          (n < H ? wn * H * 32 + n * 32 : BN / 2 + wn * H * 32 + (n - H) * 32) + (lane & 31);
    } else {
      brow[n] = wn * TN * 32 + n * 32 + (lane & 31);
    }
  }
  const int khalf = lane >> 5;

  // Software pipeline. While stage kt is read, the A loads of stages up to
  // kt + RA and the B loads up to kt + RB are in flight; each refill goes
  // into the stage read at kt - 1, which the barrier ending step kt - 1
  // released. A stage holds KSUB 16-wide substeps: the fragments of substep
  // s + 1 are read between the MFMAs of substep s, and the MFMAs of the last
  // substep run after the barrier, between the reads of the next stage's
  // first substep.
  constexpr int RA = NSTA - 1, RB = NSTB - 1;  // load distances in stages
  uint4 fa[2][TM], fb[2][TN];
  auto load_sub = [&](const u16* sa, const u16* sb, int sub, int set) {
#pragma unroll
    for (int m = 0; m < TM; ++m) fa[set][m] = lds_frag<BK, ALAY>(sa, arow[m], 2 * sub + khalf);
#pragma unroll
    for (int n = 0; n < TN; ++n) fb[set][n] = lds_frag<BK, BLAY>(sb, brow[n], 2 * sub + khalf);
  };
  constexpr int NPA = DmaTile<BM, BK, ALAY, NW>::NI;
  constexpr int NPB =
      SPLITB ? 2 * DmaTile<BN / 2, BK, BLAY, NW>::NI : DmaTile<BN, BK, BLAY, NW>::NI;
  constexpr int NPS = NPA + NPB;
  // Each step issues the loads of the operand with the shorter distance
  // first (A first when they agree). Stage kt + 1 is complete once the last
  // of its loads is: those of the shorter-distance operand, issued at step
  // kt + 1 - min(RA, RB). Issued after them: that step's loads of the other
  // operand when the distances differ, and every load of the min(RA, RB) - 1
  // steps that follow.
  constexpr int R = RA < RB ? RA : RB;
  constexpr int WAIT = (RA > RB ? NPA : (RB > RA ? NPB : 0)) + (R - 1) * NPS;
  constexpr int NSH = Hook::kStores;
  static_assert(WAIT + NPS + R * NSH <= 63, "outstanding operations exceed the vmcnt range");
  // Bit i of `stored`: the hook stored at step kt - i. The waits of step kt
  // let the stores of steps kt - R + 1 .. kt (issued after the loads of
  // stage kt + 1) stay in flight.
  unsigned stored = 0;
  // Loads and reads past the last stage are unconditional (clamped to the
  // last stage, in bounds, into released stages; reads of stale LDS) so a
  // step's MFMA section stays one basic block; nothing uses their results.
  // kt + 1 is taken mod the stage counts, so u (kt mod U) is compile-time.
  constexpr int U = NSTA == NSTB ? NSTA : NSTA * NSTB;

  // The step is laid out by hand, in the order the waves issue it: after
  // every MFMA one fragment read for the next substep and one load, with
  // scheduling fences in between, so that neither the loads nor the reads
  // bunch up between MFMAs and the MFMAs ahead of the stage barrier stay
  // ahead of it (the barrier's LDS wait is then covered). The loads of step
  // kt + 1 (A stage kt + 1 + RA, B stage kt + 1 + RB) go out right after the
  // barrier of step kt, which released their stages, between the MFMAs of
  // its last substep; the hook's stores of step kt + 1 follow them.
  constexpr int NPB0 = DmaTile<BROWS, BK, BLAY, NW>::NI;
  // Load j (in issue order) of the loads of step kt: A stage kt + RA and B
  // stage kt + RB, the shorter-distance operand's first.
  auto issue_load = [&](int u, int kt, int j) {
    const int ra = (u + RA) % NSTA, rb = (u + RB) % NSTB;
    auto a_load = [&](int i) { ta.issue_one(addr_a(ra), ta.soff(kblock(min(kt + RA, nk - 1))), i); };
    auto b_load = [&](int i) {
      const int kb = kblock(min(kt + RB, nk - 1));
      if (i < NPB0)
        tb0.issue_one(addr_b(rb), tb0.soff(kb), i);
      else if constexpr (SPLITB)
        tb1.issue_one(addr_b(rb) + (uint32_t)((BN / 2) * BK * 2), tb1.soff(kb), i - NPB0);
    };
    if constexpr (RA > RB) {
      if (j < NPB) b_load(j); else a_load(j - NPB);
    } else {
      if (j < NPA) a_load(j); else b_load(j - NPA);
    }
  };
  // Fragment read r (A fragments first, then B) of substep sub of the stage
  // (sa, sb) into set.
  auto read_frag = [&](const u16* sa, const u16* sb, int sub, int set, int r) {
    if (r < TM)
      fa[set][r] = lds_frag<BK, ALAY>(sa, arow[r], 2 * sub + khalf);
    else
      fb[set][r - TM] = lds_frag<BK, BLAY>(sb, brow[r - TM], 2 * sub + khalf);
  };
  // The MFMAs of fragment set `set`, each followed by one read of substep
  // rsub of (sa, sb) into rset and, while nload remain, one load of step
  // lkt (lu = lkt mod U). sub >= 0: this is substep sub of step skt
  // (su = skt mod U), which also issues that step's spread loads.
  // When the distances differ, the loads of step kt of the longer-distance
  // operand do not go out after the barrier with the others: they are
  // spread over the MFMAs of step kt's first KSUB - 1 substeps, one every
  // SPREAD MFMAs. Their stages were released by the barrier ending step
  // kt - 1. They follow the shorter-distance operand's loads of step kt and
  // the hook's stores of step kt, so what a step's wait allows in flight
  // (those stores and these loads) is the same set as with all loads in one
  // burst. In one burst the waves stalled on issuing them (with 4 waves, one
  // per SIMD, the MFMA units were 60% busy with the loads and 72% without);
  // spread, gate/up, the target, the apply and the update run 3-5% faster.
  constexpr int NFIRST = (RA > RB ? NPB : NPA);
  constexpr int NSECOND = NPS - NFIRST;
  constexpr bool SPREADING = RA != RB;
  constexpr int SLOTS = (KSUB - 1) * TM * TN;
  constexpr int SPREAD =
      SPREADING && NSECOND > 0 ? (SLOTS / NSECOND > 0 ? SLOTS / NSECOND : 1) : 1;
  auto mma_sub_sched = [&](int set, const u16* sa, const u16* sb, int rsub, int rset, int lu,
                           int lkt, int nload, int sub = -1, int su = 0, int skt = 0) {
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      acc[i] = Op::mma(fa[set][i / TN], fb[set][i % TN], acc[i]);
      if (i < TM + TN) read_frag(sa, sb, rsub, rset, i);
      if (i < nload) issue_load(lu, lkt, i);
      if constexpr (SPREADING) {
        if (sub >= 0) {
          const int slot = sub * TM * TN + i;
          if (slot % SPREAD == 0 && slot / SPREAD < NSECOND)
            issue_load(su, skt, NFIRST + slot / SPREAD);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = TM * TN; i < TM + TN; ++i) read_frag(sa, sb, rsub, rset, i);
#pragma unroll
    for (int i = TM * TN; i < nload; ++i) issue_load(lu, lkt, i);
  };
  auto step = [&](int u, int kt) {
    const u16* ca = stage_a(u % NSTA);
    const u16* cb = stage_b(u % NSTB);
    if constexpr (NSH > 0) {
      asm volatile("" ::: "memory");  // the hook's stores go after the loads
      stored = (stored << 1) | (kt > 0 && hook(kt, acc) ? 1u : 0u);
    }
#pragma unroll
    for (int sub = 0; sub + 1 < KSUB; ++sub)
      mma_sub_sched(sub & 1, ca, cb, sub + 1, (sub + 1) & 1, 0, 0, 0, sub, u, kt);
    // Stage kt + 1 landed everywhere; stage kt released.
    if constexpr (NSH > 0)
      wait_and_barrier_var<WAIT, NSH, R>(__builtin_popcount(stored & ((1u << R) - 1)));
    else
      wait_and_barrier<WAIT>();
    mma_sub_sched((KSUB - 1) & 1, stage_a((u + 1) % NSTA), stage_b((u + 1) % NSTB), 0, 0,
                  (u + 1) % U, kt + 1, SPREADING ? NFIRST : NPS);
  };

  hook(0, acc);
  // The loads of the steps before step 0, in the steady state's order.
  constexpr int RMAX = RA > RB ? RA : RB;
#pragma unroll
  for (int j = -RMAX; j < 0; ++j) {
    if constexpr (RA > RB) {
      if (j + RB >= 0) issue_b(j + RB, min(j + RB, nk - 1));
      issue_a(j + RA, min(j + RA, nk - 1));
    } else {
      if (j + RA >= 0) issue_a(j + RA, min(j + RA, nk - 1));
      if (j + RB >= 0) issue_b(j + RB, min(j + RB, nk - 1));
    }
  }
  wait_and_barrier<WAIT>();
  load_sub(stage_a(0), stage_b(0), 0, 0);
  // Step 0's loads; each later step's go out after the previous barrier.
#pragma unroll
  for (int j = 0; j < (SPREADING ? NFIRST : NPS); ++j) issue_load(0, 0, j);
  for (int kt = 0; kt < nk; kt += U) {
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (kt + i < nk) step(i, kt + i);
  }
  // Drain the trailing loads before the caller reuses LDS.
  wait_and_barrier<0>();
}

// Output coordinates of register group q (registers 4q..4q+3) of MFMA tile
// (m, n): four consecutive rows starting at row(), one column col().
template <class L>
struct Frag {
  int wm, wn, lane;
  // opaque: the thread index goes through an empty asm statement, so that
  // the coordinates, and the addresses derived from them, are computed where
  // they are used instead of being kept live across the K loop (for the
  // update's hooks, which run inside it).
  __device__ __forceinline__ explicit Frag(bool opaque = false) {
    int t = threadIdx.x;
    if (opaque) asm volatile("" : "+v"(t));
    const int w = t >> 6;
    wm = w / L::WGN;
    wn = w % L::WGN;
    lane = t & 63;
  }
  __device__ __forceinline__ int row(int m, int q) const {
    return wm * L::TM * 32 + m * 32 + 8 * q + 4 * (lane >> 5);
  }
  __device__ __forceinline__ int col(int n) const { return wn * L::TN * 32 + n * 32 + (lane & 31); }
};

// Stores one 32x32 MFMA accumulator tile `a` of this wave, as 16-bit
// values, into an sb<SR> matrix m (K columns) transposed: tile row R
// (R = 8q + 4(lane / 32) + e for register 4q + e) goes to column k_base + R
// (k_base a multiple of 32), and the lane's tile column to matrix row r.
// Lanes l and l ^ 32 hold the two halves of every 8 consecutive tile rows;
// each gives the other the half it does not keep, so that lane l < 32 ends
// with rows 16p .. 16p + 7 and lane l + 32 with rows 16p + 8 .. 16p + 15,
// and each of the two store instructions writes one contiguous 1 KB block
// (32 consecutive matrix rows from a multiple of 32). cvt(x, y) packs two
// values; sink(element offset, value, ok) stores the lanes with ok (all
// lanes must call this).
template <int SR, class Cvt, class Sink>
__device__ __forceinline__ void store_tile_sb(int64_t K, int r, int64_t k_base, const f32x16& a,
                                              const Cvt& cvt, bool ok, const Sink& sink) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t lo0 = cvt(a[8 * p + 0], a[8 * p + 1]), lo1 = cvt(a[8 * p + 2], a[8 * p + 3]);
    const uint32_t hi0 = cvt(a[8 * p + 4], a[8 * p + 5]), hi1 = cvt(a[8 * p + 6], a[8 * p + 7]);
    // q = 2p is (lo0, lo1), q = 2p + 1 is (hi0, hi1). Lane h = 0 keeps q = 2p
    // and sends q = 2p + 1; lane h = 1 keeps q = 2p + 1 and sends q = 2p.
    const uint32_t s0 = h ? lo0 : hi0, s1 = h ? lo1 : hi1;
    const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32), r1 = (uint32_t)__shfl_xor((int)s1, 32);
    const uint4 v = h ? make_uint4(r0, r1, hi0, hi1) : make_uint4(lo0, lo1, r0, r1);
    sink(sb_offset<SR>(r, k_base + 16 * p + 8 * h, K), v, ok);
  }
}

// 16-byte streaming (non-temporal) stores, for outputs that the next
// kernel reads: keeping them from displacing the operand stream in the
// caches made gate/up 9% faster.
__device__ __forceinline__ void store_stream(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Streaming 16-byte stores of the lanes with ok into m.
struct StreamSink {
  u16* m;
  __device__ __forceinline__ void operator()(int64_t off, const uint4& v, bool ok) const {
    if (ok) store_stream(m + off, v);
  }
};

struct CvtF16 {
  float scale;
  __device__ __forceinline__ uint32_t operator()(float x, float y) const {
    return pack_f16(x * scale, y * scale);
  }
};
struct CvtBf16 {
  float scale;
  __device__ __forceinline__ uint32_t operator()(float x, float y) const {
    return pack_bf16(x * scale, y * scale);
  }
};

// K-step rotation of the tile at absolute tile coordinates (tm, tn) when the
// workgroups resident on one XCD cover GM tile rows x 32 / GM tile columns
// (tile_index with group_m = GM): offsets that differ along both directions
// stagger every shared A and B slab.
template <int GM>
__device__ __forceinline__ int k_rotation(int tm, int tn, int nk) {
  static_assert(GM >= 1 && 32 % GM == 0, "group");
  return ((tm % GM) + (tn % (32 / GM))) % nk;
}

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

__global__ __launch_bounds__(64 * K1_NW) void gate_up_kernel(
    const u16* __restrict__ H, const u16* __restrict__ Wgp, const u16* __restrict__ Wup,
    u16* __restrict__ Z, u16* __restrict__ ZT, Dims g, int tiles_m, int tiles_n) {
  using L = Layout<K1_BM, K1_BN, K1_WGM, K1_NW>;
  constexpr int NG = L::TN / 2;  // gate tiles per wave (and as many up tiles)
  static_assert(NG >= 1 && L::TN == 2 * NG, "gate and up tiles pair up");
  TTT_GEMM_LDS_AB(lds, K1_BM, K1_BN, K1_BK, K1_NSTA, K1_NSTB)
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
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
      for (int r = 0; r < 16; ++r) z[r] = silu(acc[m][n][r]) * acc[m][n + NG][r];
      if (ZT != nullptr)
        store_tile_sb<kZtSlab>(g.T_pad, j, t0 + fr.wm * WROWS + m * 32, z, CvtF16{1.0f}, j < f,
                               StreamSink{ZT + ti.b * sb_elems<kZtSlab>(f, g.T_pad)});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = fr.wm * WROWS + m * 32 + 8 * q + 4 * (fr.lane >> 5);  // tile row
        u16* sZ = lds + row * K1_LDZ + jl;
#pragma unroll
        for (int e = 0; e < 4; ++e) sZ[e * K1_LDZ] = bf16_rne(z[4 * q + e]);
      }
    }
  if (Z == nullptr) return;
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
}

// ------------------------------------------------------ target GEMM (K2)
// M = tokens (256), N = output channels (256), K = d; fp16 operands.
// Y's stages run one step deeper than W_target's (160 KB of LDS): 5% faster.
constexpr int K2_NW = 8, K2_BM = 256, K2_BN = 256, K2_WGM = 2, K2_BK = 64, K2_NSTA = 3,
              K2_NSTB = 2;

__global__ __launch_bounds__(64 * K2_NW) void target_kernel(
    const u16* __restrict__ Y, const u16* __restrict__ WtT, u16* __restrict__ VT,
    u16* __restrict__ Vtok, u16* __restrict__ Vrow, float vscale, Dims g, int tiles_m,
    int tiles_n) {
  using L = Layout<K2_BM, K2_BN, K2_WGM, K2_NW>;
  TTT_GEMM_LDS_AB(lds, K2_BM, K2_BN, K2_BK, K2_NSTA, K2_NSTB)
  const TileIdx ti = tile_index(tiles_m, tiles_n, 4);
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
#pragma unroll
  for (int m = 0; m < L::TM; ++m)
#pragma unroll
    for (int n = 0; n < L::TN; ++n) {
      const int c = c0 + fr.col(n);
      if (VT != nullptr)
        store_tile_sb<kVtSlab>(g.T_pad, c, t0 + fr.wm * L::TM * 32 + m * 32, acc[m][n],
                               CvtF16{vscale}, c < d,
                               StreamSink{VT + ti.b * sb_elems<kVtSlab>(d, g.T_pad)});
      if (Vtok != nullptr && c < d) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t0 + fr.row(m, q);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t + e < g.T)
              Vtok[((int64_t)ti.b * g.T + t + e) * d + c] = bf16_rne(acc[m][n][4 * q + e] * vscale);
        }
      }
    }
  if (Vrow == nullptr) return;
  // Token-major fp16 vscale * V ([B][T_pad][ld_y]) through LDS, 128 tile
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
            for (int e = 0; e < 4; ++e) sv[e * LDV] = f16_rne(acc[m][n][4 * q + e] * vscale);
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
// norm_factor * sqrt(sum of chunk i's npair partials), summed in a fixed
// order.
__global__ __launch_bounds__(kThreads) void clip_scale_kernel(const float* __restrict__ partial,
                                                             float* __restrict__ scale, int npair,
                                                             int n, float norm_factor,
                                                             float clip) {
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
  float out_scale;
  uint32_t bytes;
  __device__ __forceinline__ void operator()(u16* dst, const f32x16* acc) const {
    const Frag<L> fr(OPQ);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int)bytes, kRsrcWord3);
    const uint32_t drop = bytes;
    auto sink = [&](int64_t off, const uint4& v, bool ok) {
      const u32x4 w = {v.x, v.y, v.z, v.w};
      __builtin_amdgcn_raw_buffer_store_b128(w, rsrc, ok ? (int)(off * 2) : (int)drop, 0,
                                             kCpolNt | kCpolSc1);
    };
#pragma unroll
    for (int m = 0; m < L::TM; ++m)
#pragma unroll
      for (int n = 0; n < L::TN; ++n) {
        const int jb = j0 + fr.wm * L::TM * 32 + m * 32;  // first d_ff index of the tile
        const int c = c0 + fr.col(n);
        store_tile_sb<kSnapSlab>(f, c, jb, acc[m * L::TN + n], CvtBf16{out_scale},
                                 c < d && jb < f, sink);
      }
  }
};

// acc = acc_scale * W for the wave's part of a [d_ff tile] x [d_model tile]
// state block, W element (c, j) at W + c * ld + j (bf16 or fp32). BATCHED:
// the loads are unconditional (lanes outside the matrix read element 0 and
// drop it), so that they are issued back to back and waited for once; this
// needs registers for all of them, so inside the K loop (the packed
// update's reset) the per-element conditional form is used instead.
template <class L, bool F32, bool BATCHED = true, bool OPQ = false>
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
template <class L, bool F32, bool PACKED>
struct ChunkSnapshots {
  static constexpr int kStores = SnapshotStore<L, PACKED>::kStores;
  SnapshotStore<L, PACKED> store;
  StateLoad<L, F32, false, PACKED> reset;
  u16* snap;  // this sequence's snapshots, or null
  int64_t chunk_stride;
  int steps_per_chunk;
  StepBits bits;  // PACKED: this launch's steps
  int n_chunks;   // PACKED: snapshot slots (table values are clamped to them)
  __device__ __forceinline__ bool operator()(int kt, f32x16* acc) const {
    int slot;
    if constexpr (PACKED) {
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
template <int BN, bool WINIT_F32, bool PACKED>
__device__ __forceinline__ void update_tile(
    u16* lds, StepBits bits, int b, int j0, int c0, const u16* __restrict__ ZT,
    const u16* __restrict__ VT, const void* __restrict__ Winit, int64_t winit_bstride,
    int64_t winit_ld, float acc_scale, u16* __restrict__ snap, int64_t snap_bstride,
    float* __restrict__ Wf, u16* __restrict__ shadow, const Dims& g, int tok_begin, int nk,
    int steps_per_chunk, int n_chunks) {
  using C = UpdCfg<BN>;
  using L = Layout<K3_BM, BN, C::WGM, K3_NW>;
  constexpr int TM = L::TM, TN = L::TN, NSTA = C::NSTA, NSTB = C::NSTB;
  static_assert((NSTA * K3_BM + NSTB * BN) * K3_BK <= kUpdLdsElems, "stages fit");
  const int d = g.d, f = g.f;
  const Frag<L> fr;
  const int64_t chunk_stride = snap_elems(g);
  const float out_scale = 1.0f / acc_scale;

  const void* winit_b =
      WINIT_F32 ? (const void*)(static_cast<const float*>(Winit) + b * winit_bstride)
                : (const void*)(static_cast<const u16*>(Winit) + b * winit_bstride);
  const StateLoad<L, WINIT_F32> init{winit_b, winit_ld, j0, c0, d, f, acc_scale};
  const StateLoad<L, WINIT_F32, false, PACKED> reset{winit_b, winit_ld, j0, c0, d, f,
                                                     acc_scale};
  f32x16 acc[TM][TN];
  init(&acc[0][0]);

  const SnapshotStore<L, PACKED> snapshot{j0, c0, d, f, out_scale,
                                          (uint32_t)(chunk_stride * 2)};
  const ChunkSnapshots<L, WINIT_F32, PACKED> hook{
      snapshot, reset, snap ? snap + b * snap_bstride : nullptr, chunk_stride,
      steps_per_chunk, bits, n_chunks};
  // Rows past d_ff / d_model in the last slabs are never written; they only
  // feed output rows / columns that are not stored. A narrow tile reads the
  // first or second 128 rows of a 256-row V^T slab: 16 contiguous KB per K
  // step.
  static_assert(K3_BM == kZtSlab && kVtSlab == K3_WIDE && BN <= kVtSlab && K3_BK == 64,
                "update tile rows = slab rows");
  const Operand vt =
      slab_blocked<kVtSlab>(VT + b * sb_elems<kVtSlab>(d, g.T_pad), g.T_pad, c0, tok_begin);
  gemm_core_ab<K3_NW, K3_BM, BN, C::WGM, K3_BK, NSTA, NSTB, F16Mma, false, kSlab, kSlab>(
      slab_blocked<kZtSlab>(ZT + b * sb_elems<kZtSlab>(f, g.T_pad), g.T_pad, j0, tok_begin),
      vt, vt, nk, &acc[0][0], lds, hook);

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
  if (shadow != nullptr) snapshot(shadow + (int64_t)b * chunk_stride, &acc[0][0]);
}

// Workgroups [0, n_wide) take the wide tiles of regions [0, n_wide); the
// rest take the two narrow halves of each remaining region (regions in
// tile_coords order over regions_m x regions_n 256 x 256 regions per
// sequence, group 4).
template <bool WINIT_F32, bool PACKED>
__global__ __launch_bounds__(64 * K3_NW) void update_kernel(
    const u16* __restrict__ ZT, const u16* __restrict__ VT, const void* __restrict__ Winit,
    int64_t winit_bstride, int64_t winit_ld, float acc_scale, u16* __restrict__ snap,
    int64_t snap_bstride, float* __restrict__ Wf, u16* __restrict__ shadow, Dims g,
    int tok_begin, int nk, int steps_per_chunk, const BlockInfo* __restrict__ blocks,
    int n_chunks, int regions_m, int regions_n, int n_wide) {
  __shared__ __attribute__((aligned(16))) u16 lds[kUpdLdsElems];
  StepBits bits{0u, 0u, 0};
  // nk <= kMaxPackedSteps for a packed launch (checked on the host).
  if constexpr (PACKED) bits = load_step_bits(lds, blocks, tok_begin / K3_BK, nk, n_chunks);
  if ((int)blockIdx.x < n_wide) {
    const TileIdx t = tile_coords(xcd_contiguous(blockIdx.x, n_wide), regions_m, regions_n, 4);
    update_tile<K3_WIDE, WINIT_F32, PACKED>(
        lds, bits, t.b, t.tm * K3_BM, t.tn * K3_WIDE, ZT, VT, Winit, winit_bstride, winit_ld,
        acc_scale, snap, snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
        n_chunks);
    return;
  }
  // n_wide is a multiple of 8 whenever narrow tiles follow, so the XCD of a
  // workgroup is that of its position in the narrow range.
  const int id = xcd_contiguous(blockIdx.x - n_wide, gridDim.x - n_wide);
  const TileIdx t = tile_coords(n_wide + id / 2, regions_m, regions_n, 4);
  const int c0 = t.tn * K3_WIDE + (id & 1) * K3_NARROW;
  if (c0 >= g.d) return;  // uniform: the half of a region past d_model
  update_tile<K3_NARROW, WINIT_F32, PACKED>(
      lds, bits, t.b, t.tm * K3_BM, c0, ZT, VT, Winit, winit_bstride, winit_ld, acc_scale,
      snap, snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk, n_chunks);
}

// ------------------------------------------------------------ apply (K4)
// M = d_model (256), N = tokens (BN, which divides the chunk), K = d_ff.
// The tile's tokens all lie in one chunk i and read snapshot i.
// The XCD's resident apply tiles: 8 d_model tiles x 4 token tiles, which
// (with 256-token tiles) share one chunk's snapshot slabs.
constexpr int kApplyGroupM = 8;

template <int BN>
struct ApplyCfg {
  static constexpr int NW = 8;
  static constexpr int WGM =
      BN == 256 ? 2 : (BN == 128 ? 4 : 8);
  // With 256-token tiles, Z's stages run one step deeper than the
  // snapshot's (160 KB of LDS): 10% faster. Narrower tiles keep two each.
  static constexpr int BK = 64, NSTA = 2, NSTB = BN == 256 ? 3 : 2;
};

template <int BN, bool OUT_F32>
__global__ __launch_bounds__(64 * ApplyCfg<BN>::NW) void apply_kernel(
    const u16* __restrict__ Z, const u16* __restrict__ snap, int64_t snap_bstride,
    int64_t snap_cstride, void* __restrict__ O, Dims g, int tok_begin, int tok_end, int chunk,
    const ApplyTile* __restrict__ tiles, int n_chunks, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int BM = kSnapSlab, WGM = ApplyCfg<BN>::WGM, BK = ApplyCfg<BN>::BK,
                NSTA = ApplyCfg<BN>::NSTA, NSTB = ApplyCfg<BN>::NSTB;
  static_assert(BK == 64, "the snapshot slab is one K step");
  using L = Layout<BM, BN, WGM, ApplyCfg<BN>::NW>;
  TTT_GEMM_LDS_AB(lds, BM, BN, BK, NSTA, NSTB)
  const TileIdx ti = tile_index(tiles_m, tiles_n, kApplyGroupM);
  const int c0 = ti.tm * BM;
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
  const int d = g.d, f = g.f, T = g.T;
  f32x16 acc[L::TM][L::TN];
  zero_acc(acc);
  const Operand z =
      row_major<BK>(Z + ((int64_t)ti.b * T + t0) * g.ld_z, g.ld_z, min(BN, T - t0));
  // The rotation follows the absolute 256-token block, whatever the tile
  // width, so that every schedule and width sums each output in the same
  // order.
  const int nk = f / BK;
  gemm_core_ab<ApplyCfg<BN>::NW, BM, BN, WGM, BK, NSTA, NSTB, Bf16Mma, false, kSlab, kRowMajor>(
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

template <bool F32>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const void* __restrict__ src,
                                                             u16* __restrict__ dst, int rows,
                                                             int cols, int64_t ld_dst) {
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
    if (c < cols && r < rows) dst[(int64_t)c * ld_dst + r] = f16_rne(tile[tx][i]);
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

template <bool TAPS_F32>
__global__ __launch_bounds__(kThreads) void conv_kernel(const u16* __restrict__ X0,
                                                        const u16* __restrict__ X0n, int n_next,
                                                        const void* __restrict__ taps,
                                                        u16* __restrict__ Y, Dims g, int K,
                                                        int chunk, int pad_chunk,
                                                        const BlockInfo* __restrict__ blocks,
                                                        int64_t total) {
  // Neighbouring row windows overlap by K - 1 rows; keeping them on one XCD
  // lets the overlap come from that XCD's L2.
  const int64_t gid = (int64_t)xcd_contiguous_id() * kThreads + threadIdx.x;
  if (gid >= total) return;
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
#pragma unroll
  for (int r = 0; r < kConvRows; ++r)
    *reinterpret_cast<uint4*>(Y + ((int64_t)b * g.T_pad + t + r) * g.ld_y + c) =
        make_uint4(pack_f16(acc[r][0], acc[r][1]), pack_f16(acc[r][2], acc[r][3]),
                   pack_f16(acc[r][4], acc[r][5]), pack_f16(acc[r][6], acc[r][7]));
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

hipError_t launch_transpose_f16(const void* src, bool src_f32, uint16_t* dst, int rows, int cols,
                                int64_t ld_dst, hipStream_t s) {
  dim3 grid(ceil_div(cols, 64), ceil_div(rows, 64));
  if (src_f32)
    transpose_kernel<true><<<grid, kThreads, 0, s>>>(src, dst, rows, cols, ld_dst);
  else
    transpose_kernel<false><<<grid, kThreads, 0, s>>>(src, dst, rows, cols, ld_dst);
  return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* X0, const uint16_t* X0_next, int n_next,
                       const void* taps, bool taps_f32, uint16_t* Y, const Dims& g, int K,
                       int chunk, bool pad_chunk, const BlockInfo* blocks, hipStream_t s) {
  const int64_t total = (int64_t)g.B * (g.T_pad / kConvRows) * (g.d / 8);
  const int grid = ceil_div(total, kThreads);
  if (n_next == 0) X0_next = X0;  // never read
  if (taps_f32)
    conv_kernel<true><<<grid, kThreads, 0, s>>>(X0, X0_next, n_next, taps, Y, g, K, chunk,
                                                pad_chunk ? 1 : 0, blocks, total);
  else
    conv_kernel<false><<<grid, kThreads, 0, s>>>(X0, X0_next, n_next, taps, Y, g, K, chunk,
                                                 pad_chunk ? 1 : 0, blocks, total);
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
                          uint16_t* Z, uint16_t* ZT, const Dims& g, hipStream_t s) {
  const int tiles_m = g.T_pad / K1_BM, tiles_n = ceil_div(g.f, K1_BN / 2);
  gate_up_kernel<<<tiles_m * tiles_n * g.B, 64 * K1_NW, 0, s>>>(H, Wgp, Wup, Z, ZT, g, tiles_m,
                                                              tiles_n);
  return hipGetLastError();
}

hipError_t launch_target(const uint16_t* Y, const uint16_t* WtT, uint16_t* VT, uint16_t* Vtok,
                         uint16_t* Vrow, float vscale, const Dims& g, hipStream_t s) {
  const int tiles_m = g.T_pad / K2_BM, tiles_n = ceil_div(g.d, K2_BN);
  target_kernel<<<tiles_m * tiles_n * g.B, 64 * K2_NW, 0, s>>>(Y, WtT, VT, Vtok, Vrow, vscale,
                                                             g, tiles_m, tiles_n);
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
                             hipStream_t s) {
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
                                                               n, norm_factor, clip);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n16 = vt_elems(g) / 8;
  vt_scale_kernel<<<ceil_div(n16, kThreads), kThreads, 0, s>>>(VT, scale, g, chunk, nchunks,
                                                               blocks, n16);
  return hipGetLastError();
}

template <bool F32, bool PACKED>
static void update_launch(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                          int64_t winit_bstride, int64_t winit_ld, float acc_scale,
                          uint16_t* snap, int64_t snap_bstride, float* Wf, uint16_t* shadow,
                          const Dims& g, int tok_begin, int nk, int steps_per_chunk,
                          const BlockInfo* blocks, int n_chunks, hipStream_t s) {
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
  update_kernel<F32, PACKED><<<grid, 64 * K3_NW, 0, s>>>(
      ZT, VT, Winit, winit_bstride, winit_ld, acc_scale, snap, snap_bstride, Wf, shadow, g,
      tok_begin, nk, steps_per_chunk, blocks, n_chunks, regions_m, regions_n, n_wide);
}

hipError_t launch_update(const uint16_t* ZT, const uint16_t* VT, const void* Winit,
                         bool winit_f32, int64_t winit_bstride, int64_t winit_ld,
                         float acc_scale, uint16_t* snap, int64_t snap_bstride, float* Wf,
                         uint16_t* shadow, const Dims& g, int tok_begin, int tok_count,
                         int chunk, const BlockInfo* blocks, int n_chunks, hipStream_t s) {
  // Token offsets and counts are whole K steps, so that the slab operands are
  // read from a slab boundary.
  const int nk = (tok_count + K3_BK - 1) / K3_BK, steps_per_chunk = chunk / K3_BK;
  if (blocks != nullptr) {
    if (nk > kMaxPackedSteps) return hipErrorInvalidValue;  // StepBits holds 2048 steps
    if (winit_f32)
      update_launch<true, true>(ZT, VT, Winit, winit_bstride, winit_ld, acc_scale, snap,
                                snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                blocks, n_chunks, s);
    else
      update_launch<false, true>(ZT, VT, Winit, winit_bstride, winit_ld, acc_scale, snap,
                                 snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                 blocks, n_chunks, s);
  } else {
    if (winit_f32)
      update_launch<true, false>(ZT, VT, Winit, winit_bstride, winit_ld, acc_scale, snap,
                                 snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                 nullptr, n_chunks, s);
    else
      update_launch<false, false>(ZT, VT, Winit, winit_bstride, winit_ld, acc_scale, snap,
                                  snap_bstride, Wf, shadow, g, tok_begin, nk, steps_per_chunk,
                                  nullptr, n_chunks, s);
  }
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
