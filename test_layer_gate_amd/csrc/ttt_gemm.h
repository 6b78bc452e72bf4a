// The MFMA GEMM core shared by the gfx950 kernel files (prefill and
// backward): C[M][N] = sum_k A[m][k] * B[n][k] with both operands
// K-contiguous in HBM, staged through LDS by direct-to-LDS buffer loads, and
// the helpers its kernels use (tile order, accumulator stores). Each kernel
// file includes it once; everything here is internal to that file.
//
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
#pragma once
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
// LDS / HBM layouts of a GEMM operand (see Operand; kSlabT: OperandT)
enum { kRowMajor = 0, kSlab = 1, kSlabT = 2 };
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

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// A B fragment of a kSlabT stage: two LDS transpose reads at the lane's byte
// offsets b0 (K values 0..3) and b1 (4..7) from the stage (slabt_tr_byte).
__device__ __forceinline__ uint4 lds_frag_tr(const u16* lds, uint32_t b0, uint32_t b1) {
  char* p = (char*)lds;
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + b0));
  const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + b1));
  const uint2 xu = __builtin_bit_cast(uint2, x), yu = __builtin_bit_cast(uint2, y);
  return make_uint4(xu.x, xu.y, yu.x, yu.y);
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

// A B operand read transposed from sb<256> matrices (kSlabT, BK = 64, tile
// of 256 columns): B[n][k] = M0[k][n] for the K steps kt < ksplit and
// M1[k - 64 ksplit][n] after them, both with K columns (slabt_* in
// ttt_launch.h give the layouts). base0 / base1 point at the tile's first
// column in slab row 0; reads at or past bytes0 / bytes1 from there return
// zero. The step offsets must stay below 2^31 bytes.
struct OperandT {
  const u16* base0;
  const u16* base1;
  uint32_t bytes0, bytes1;
  int ksplit;
  int64_t K;
};

template <int ROWS, int NW>
struct DmaTile<ROWS, 64, kSlabT, NW> {
  static constexpr int NB = ROWS / 8;  // 1 KB blocks: 16 columns x 32 rows each
  static constexpr int NI = (NB + NW - 1) / NW;
  uint32_t voff[NI];
  uint32_t loff[NI];
  u32x4 rsrc0, rsrc1;
  int ksplit;
  int64_t K;
  __device__ __forceinline__ void init(const OperandT& op, int wave, int lane) {
    rsrc0 = make_rsrc(op.base0, op.bytes0);
    rsrc1 = make_rsrc(op.base1, op.bytes1);
    ksplit = op.ksplit;
    K = op.K;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int block = (NW * i + wave) % NB;
      loff[i] = (uint32_t)block * 1024;
      voff[i] = slabt_piece_byte(block, lane);
    }
  }
  // The scalar byte offset of K step kt, with bit 31 set when it reads M1.
  __device__ __forceinline__ uint32_t soff(int kt) const {
    const bool second = kt >= ksplit;
    const uint32_t o = slabt_step_byte(second ? kt - ksplit : kt, K);
    return __builtin_amdgcn_readfirstlane(o | (second ? 0x80000000u : 0u));
  }
  __device__ __forceinline__ void issue_one(uint32_t lds_stage, uint32_t so, int i) const {
    lds_dma_b128((so >> 31) ? rsrc1 : rsrc0, lds_stage + loff[i], voff[i], so & 0x7fffffffu);
  }
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
// kReverse: the K steps run from the last K block to the first (a hook's
// step index kt then reads block nk - 1 - kt).
struct NoHook {
  static constexpr int kStores = 0;
  static constexpr bool kReverse = false;
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
// BLAY = kSlabT: B0 is an OperandT, read with LDS transpose reads (not with
// SPLITB).
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
          int ALAY, int BLAY, class Hook, class OpB = Operand>
__device__ __forceinline__ void gemm_core_ab(const Operand& A, const OpB& B0, const OpB& B1,
                                             int nk, f32x16* acc, u16* lds, const Hook& hook,
                                             int k0 = 0) {
  using Lay = Layout<BM, BN, WGM, NW>;
  constexpr int TM = Lay::TM, TN = Lay::TN, WGN = Lay::WGN;
  constexpr int BROWS = SPLITB ? BN / 2 : BN;
  constexpr int KSUB = BK / 16;  // MFMA K-substeps per stage
  static_assert(NSTA >= 2 && NSTB >= 2 && NSTA <= kMaxStages && NSTB <= kMaxStages && KSUB >= 2,
                "pipeline");
  static_assert(BLAY != kSlabT || (!SPLITB && BK == 64 && BN == 256), "transposed B tiles");
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
    if constexpr (Hook::kReverse) return nk - 1 - kt;
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
  // kSlabT: the lane's LDS byte offsets of the two transpose reads of each
  // B fragment in a stage's substep 0.
  uint32_t btr[BLAY == kSlabT ? TN : 1][2];
  if constexpr (BLAY == kSlabT) {
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) btr[n][rd] = slabt_tr_lane(lane, wn * TN * 32 + n * 32, rd);
  }
  auto b_frag = [&](const u16* sb, int n, int sub) {
    if constexpr (BLAY == kSlabT)
      return lds_frag_tr(sb, btr[n][0] + slabt_tr_sub(sub), btr[n][1] + slabt_tr_sub(sub));
    else
      return lds_frag<BK, BLAY>(sb, brow[n], 2 * sub + khalf);
  };

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
    for (int n = 0; n < TN; ++n) fb[set][n] = b_frag(sb, n, sub);
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
      fb[set][r - TM] = b_frag(sb, r - TM, sub);
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
    // q = 2p is (lo0, lo1), q = 2p + 1 is (hi0, hi1). v_permlane32_swap
    // trades lanes 32..63 of its first operand for lanes 0..31 of its
    // second: afterwards lane l < 32 holds its own q = 2p in the first and
    // lane l + 32's q = 2p in the second, and lane l + 32 holds lane l's
    // q = 2p + 1 in the first and its own in the second.
    const auto x0 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);
    const auto x1 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);
    sink(sb_offset<SR>(r, k_base + 16 * p + 8 * h, K), make_uint4(x0[0], x1[0], x0[1], x1[1]),
         ok);
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

}  // namespace
}  // namespace tttk
