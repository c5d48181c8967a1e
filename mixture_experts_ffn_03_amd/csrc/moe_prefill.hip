// Prefill experts: expert-grouped GEMM on gfx950 MFMA with FP4 weights decoded in
// registers (W4A16: bf16 activations, bf16 MFMA operands, fp32 accumulation).
//
// MoE constructor page (spark_model/layers/moe/init.rs): the sorted/grouped prefill path
// (sort by expert, grouped gate+up GEMM, SiLU*up, grouped down GEMM, unpermute-reduce,
// blend) and its tile work list built on the same stream; MoE module page
// (spark_model/layers/moe/mod.rs): the "original" [N, K/2] weight layout with its block
// scales, the NVFP4/MXFP4 formats (doc of experts_scale_kind) and the gather of sorted
// rows fused into the GEMM's A load (doc of moe_permute_tokens_k).
//
// Design (gfx950, v_mfma_f32_32x32x16_bf16):
// * A block of 4 waves (one per SIMD) computes an MT-row tile of one expert against
//   BROWS weight rows. Each wave owns RB 32-row blocks and CB 32-column blocks of
//   weight rows (gate+up: half of them gate and the same ones of up, so SwiGLU runs in
//   the epilogue on values held by the same lane; with one column block per wave, waves
//   0-1 hold gate and 2-3 up, paired through LDS in the epilogue), i.e. RB*CB independent
//   accumulators; each decoded B operand feeds RB MFMAs.
// * Both operands reach LDS by direct-to-LDS loads (global_load_lds_*: the activation
//   rows gathered by row_token, the FP4 weight rows and their scale bytes) into a ring
//   of K stages (three of 64 codes for most shapes; see launch_pre). Step c waits for stage c, synchronises the block once,
//   reads stage c's operands from LDS, issues stage c+2 into the slot freed by step c-1,
//   then runs the MFMAs of stage c.
//   Loads therefore have two steps to land, and no registers are spent on them.
// * A block takes at most 80 KB of LDS, so two blocks run on each CU; their barriers
//   and LDS waits fall at different times, and each fills the other's MFMA gaps.
// * The loads and their waits are explicit: the compiler's counter tracking cannot tell
//   a direct-to-LDS load apart from the LDS reads of other stages and would drain every
//   load before each read. No other vector-memory load is issued in the main loop, so
//   "at most one stage of loads in flight" means "this step's stage has landed".
// * LDS rows are swizzled in 16-byte slots (a_swz, b_swz) so that the rows served per
//   LDS cycle by one MFMA operand read fall in distinct banks; the load side picks the
//   source piece for its fixed slot.
// * The MFMA K order is permuted inside a stage (lane half h covers codes 32h..32h+31),
//   so each lane's B codes are 16 contiguous bytes of one weight row; A is read with the
//   same permutation.
// * E2M1 codes become exact bf16 operands in registers (MXFP4: scaled convert by the
//   E8M0 power of two; NVFP4: convert, times the E4M3 scale in fp32, pack).
// * Block ids are remapped so that each XCD (ids dispatched round-robin over the 8
//   XCDs) walks a contiguous run of (row tile, column tile) work, which keeps an A
//   tile and an expert's weight rows in that XCD's L2 while they are reused.
// * Down projections of FP4 weights with per-stage scales run as a persistent grid over
//   the tile list when it exceeds the resident slots (see k_pre_gemm's PERSIST form; build
//   flag MOE_PRE_PERSIST=0 gives one block per tile instead).
// * Build flag MOE_PRE_MX8 (off by default: measured slower, kept to reproduce the
//   measurement): MXFP4 weights fed natively to the block-scaled MFMA
//   (v_mfma_scale_f32_32x32x64_f8f6f4, the analogue of the pages' block-scaled FP4 MMA,
//   MoE constructor page) with the activations quantised to MXFP8 hi + lo pairs.
#include <type_traits>

#include "moe_device.h"
#include "moe_fp4.h"

namespace moe {

constexpr int kFp8MaxKb = 128;  // FP8 prefill: K up to 128 * 128 codes (block-scale table)

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint32_t (&d)[4]) {
  uint4 v = make_uint4(d[0], d[1], d[2], d[3]);
  return __builtin_bit_cast(bf16x8_t, v);
}

// One row's 32 columns of an MFMA output block as 16-bit values, lane half h holding
// columns 8g + 4h .. 8g + 4h + 3 (g = 0..3) packed in pk[g]: the two halves swap half of
// them (lane l with l + 32), so each lane stores 16 contiguous bytes and each store
// instruction writes 32 contiguous bytes of each of 32 rows (half 0: columns 0-7 and 16-23,
// half 1: 8-15 and 24-31). Both lanes of a pair must be active.
__device__ __forceinline__ void store_cols32_16bit(uint16_t* row, const uint32_t (&pk)[4][2],
                                                   int half) {
  const uint32_t s0 = half ? pk[0][0] : pk[1][0], s1 = half ? pk[0][1] : pk[1][1];
  const uint32_t s2 = half ? pk[2][0] : pk[3][0], s3 = half ? pk[2][1] : pk[3][1];
  const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32), r1 = (uint32_t)__shfl_xor((int)s1, 32);
  const uint32_t r2 = (uint32_t)__shfl_xor((int)s2, 32), r3 = (uint32_t)__shfl_xor((int)s3, 32);
  *reinterpret_cast<uint4*>(row + (half ? 8 : 0)) =
      half ? make_uint4(r0, r1, pk[1][0], pk[1][1]) : make_uint4(pk[0][0], pk[0][1], r0, r1);
  *reinterpret_cast<uint4*>(row + (half ? 24 : 16)) =
      half ? make_uint4(r2, r3, pk[3][0], pk[3][1]) : make_uint4(pk[2][0], pk[2][1], r2, r3);
}

// Build flag MOE_PRE_WAIT_SPLIT (off in the library; a diagnostic build): the one-block-per-tile
// grouped GEMM of the routed MXFP4 experts sums per wave the shader-clock cycles of each step
// spent in the stage-load wait, at the barrier, and in the whole K loop, into g_wait_split
// [gate+up, down][block][wave][loop, load wait, barrier, steps] (moe_debug_prefill_wait_split).
#ifndef MOE_PRE_WAIT_SPLIT
#define MOE_PRE_WAIT_SPLIT 0
#endif
#if MOE_PRE_WAIT_SPLIT
constexpr int kWaitSplitBlocks = 8192;
__device__ unsigned long long g_wait_split[2][kWaitSplitBlocks][4][4];
#endif

// The stage-load half of wait_stage: at most N loads of this wave in flight, LDS reads done.
template <int N>
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}
template <int NL, int NSS>
__device__ __forceinline__ void wait_loads_inflight(int r, bool ss) {
  if (r <= 0) {
    wait_loads<0>();
  } else if (r == 1) {
    if (ss) wait_loads<NL + NSS>(); else wait_loads<NL>();
  } else if (r == 2) {
    if (ss) wait_loads<2 * NL + NSS>(); else wait_loads<2 * NL>();
  } else {
    if (ss) wait_loads<3 * NL + NSS>(); else wait_loads<3 * NL>();
  }
}

// Wait until at most N vector-memory loads of this wave are in flight and its LDS reads
// have returned, then synchronise the block: every wave's loads of the stage have
// landed, and every read of the slot about to be refilled is done.
template <int N>
__device__ __forceinline__ void wait_stage() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// wait_stage with R (0..3) stages of NL loads still in flight, one of which (ss) also
// carries NSS super-stage scale loads
template <int NL, int NSS>
__device__ __forceinline__ void wait_inflight(int r, bool ss) {
  if (r <= 0) {
    wait_stage<0>();
  } else if (r == 1) {
    if (ss) wait_stage<NL + NSS>(); else wait_stage<NL>();
  } else if (r == 2) {
    if (ss) wait_stage<2 * NL + NSS>(); else wait_stage<2 * NL>();
  } else {
    if (ss) wait_stage<3 * NL + NSS>(); else wait_stage<3 * NL>();
  }
}

// Row swizzles of the 16-byte pieces in LDS. An MFMA operand read (ds_read_b128) has
// lane r read row r; every 16 consecutive lanes (one LDS cycle of 256 bytes), and every
// 8 of them, must land on distinct 16-byte bank groups. A rows of 8 pieces (128 bytes)
// XOR the piece with a permutation of row bits 0..3 that is distinct over any 8
// consecutive rows and over the 8 rows of each parity within 16; rows of 16 pieces use
// row bits 0..3 directly; rows of 4 pieces XOR with (row >> 1 ^ row >> 2) & 3, distinct over
// the rows that share banks in either grouping. B rows of 2 pieces (32 bytes) flip the piece by row bit 2 xor
// bit 3; of 4 pieces (64 bytes) by ((row >> 1) ^ (row >> 3)) & 3.
template <int PA>
__device__ __forceinline__ int a_swz(int row) {
  if (PA >= 16) return row & 15;
  if (PA == 8) return ((row >> 1) ^ ((row & 1) << 2)) & 7;
  return ((row >> 1) ^ (row >> 2)) & 3;  // 4 pieces (64-byte rows)
}
template <int PB>
__device__ __forceinline__ int b_swz(int row) {
  if (PB == 8) return (row >> 1) & 7;
  return PB == 2 ? ((row >> 2) ^ (row >> 3)) & 1 : ((row >> 1) ^ (row >> 3)) & 3;
}

// Scale word of a lane half: W (1, 2, 4 or 8) scale bytes, little-endian.
template <int W>
using ScaleWord = std::conditional_t<(W > 4), uint64_t, uint32_t>;
template <int W>
__device__ __forceinline__ ScaleWord<W> lds_scale(const uint8_t* p) {
  if constexpr (W == 8) return *reinterpret_cast<const uint64_t*>(p);
  if constexpr (W == 4) return *reinterpret_cast<const uint32_t*>(p);
  if constexpr (W == 2) return *reinterpret_cast<const uint16_t*>(p);
  return *p;
}

// Resolve this block's (row tile, column tile), remapped per XCD; false = no work.
__device__ __forceinline__ bool pre_resolve(const ExpertGemmArgs& a, int ncol_tiles, Tile& t,
                                            int& col_tile) {
  int nrow_tiles;
  if (a.src.tiles) {
    nrow_tiles = a.src.ntiles[0];
  } else {
    nrow_tiles = (a.src.implicit_rows + a.src.implicit_height - 1) / a.src.implicit_height;
  }
  const int real = nrow_tiles * ncol_tiles;
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  if (b >= real) return false;
  const int x = b % kXcds, j = b / kXcds, q = real / kXcds, r = real % kXcds;
  const int logical = x * q + (x < r ? x : r) + j;
  const int rt = logical / ncol_tiles;
  col_tile = logical % ncol_tiles;
  if (a.src.tiles) {
    t = a.src.tiles[rt];
  } else {
    const int r0 = rt * a.src.implicit_height;
    t.group = 0;
    t.row0 = a.src.implicit_row0 + r0;
    t.count = min(a.src.implicit_height, a.src.implicit_rows - r0);
    t.pad = 0;
  }
  return true;
}

// A float at a block-uniform address, through the scalar cache (the memory is read-only
// while the kernel runs): the wait for it is on the scalar counter, never on the
// vector-memory counter that tracks the stage loads.
__device__ __forceinline__ float load_uniform_f32(const float* p, int i) {
  typedef __attribute__((address_space(4))) const float cf32_t;
  return *((cf32_t*)p + __builtin_amdgcn_readfirstlane(i));
}

// Header (group, first row, row count) of a tile at a block-uniform index, through the
// scalar cache; the fields stay in scalar registers.
__device__ __forceinline__ Tile load_tile_header(const Tile* tiles, int i) {
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(4))) const i32x4_t ci32x4_t;
  const i32x4_t h = *(ci32x4_t*)(tiles + i);
  Tile t;
  t.group = __builtin_amdgcn_readfirstlane(h[0]);
  t.row0 = __builtin_amdgcn_readfirstlane(h[1]);
  t.count = __builtin_amdgcn_readfirstlane(h[2]);
  t.pad = 0;
  return t;
}

// Operand for MFMA step s (codes 8s..8s+7 of the lane's codes of the stage).
template <int FMT, typename W>
__device__ __forceinline__ bf16x8_t b_operand(const uint32_t q, const W sc_word, int s) {
  const int blk = FMT == 0 ? s / 2 : s / 4;  // 16- or 32-code block inside the lane's codes
  const uint32_t sb = (sc_word >> (8 * blk)) & 0xFFu;
  uint32_t d[4];
  mfma_operand_fp4x8<FMT>(q, sb, d);
  return as_bf16x8(d);
}

// Block = 4 waves (one per SIMD) in a WM x WN grid, with a ring of NSTG stage slots. Tile height MT = 32 * RB * WM;
// BROWS weight rows per block (gate+up: BROWS/2 gate rows and the same BROWS/2 up rows;
// down: BROWS output columns). A stage holds KC (64, 128 or 256) codes of K: the A tile (MT
// rows x 2*KC bytes of bf16) and the B tile (BROWS rows x KC/2 bytes of E2M1 codes).
// Scales come one of two ways:
// * SS = false: with each stage, per weight row one 4-byte LDS slot per 64 codes holding
//   their scale bytes (NVFP4 four, MXFP4 two), loaded as one dword or one ushort.
// * SS = true (scale rows a multiple of 16 bytes): 16 bytes per row at a time, covering
//   SUPER stages (256 codes NVFP4, 512 MXFP4), into one of two super-stage slots.
// Every shape in use keeps a block within 80 KB of LDS, so two blocks share a CU: the waves
// of one fill the SIMDs while the other waits at its barrier or on LDS. The 32-row tiles
// of the HBM-bound short groups take longer stages: 128 codes (64-byte pieces of each weight
// row), or 256 for MXFP4 (whole 128-byte lines, in a two-slot ring).
template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS>
struct PreShape {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;  // threads per block
  static constexpr int WN = NW / WM;
  static constexpr int MT = 32 * RB * WM;
  static constexpr int BROWS = 32 * CB * WN;
  static constexpr int NCOLS = GATEUP ? BROWS / 2 : BROWS;  // output columns per block
  static constexpr bool FP4 = FMT <= 1;
  static constexpr int STEPS = KC / 16;  // MFMA steps per stage (lane half: KC/2 codes)
  static constexpr int PA = KC / 8;      // 16-byte pieces per A row per stage (bf16)
  // B row bytes per stage: KC codes of 1/2 (FP4), 1 (FP8) or 2 (BF16) bytes
  static constexpr int B_ROW = FP4 ? KC / 2 : (FMT == 2 ? KC : 2 * KC);
  static constexpr int PB = B_ROW / 16;   // 16-byte pieces per B row per stage
  static constexpr int WPS = B_ROW / 4 / (2 * STEPS);  // B dwords per lane per MFMA step
  static constexpr int A_ROW = 16 * PA;
  static constexpr int SLOTS = KC / 64;                            // FP4 scale slots per row
  static constexpr int SROW = (SS || !FP4) ? 0 : 4 * SLOTS;        // scale bytes per row per stage
  static constexpr int SW = FMT == 0 ? KC / 32 : KC / 64;          // FP4 scale bytes per lane half
  static constexpr int A_BYTES = MT * A_ROW;
  static constexpr int B_BYTES = BROWS * B_ROW;
  static constexpr int S_BYTES = BROWS * SROW;
#if MOE_PRE_MX8
  // block-scaled MFMA variant: MXFP8 hi/lo activations (MXFP4 weights, 64-code stages)
  static constexpr bool MX8 = FMT == 1 && KC == 64 && !SS;
#else
  static constexpr bool MX8 = false;
#endif
  // activation scales: [row][2 blocks], one 4-byte LDS slot each (a 2-byte direct-to-LDS load
  // still fills a dword per lane)
  static constexpr int AS_BYTES = MX8 ? MT * 2 * 4 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES + AS_BYTES;
  static constexpr int NA = MT * PA / NT;        // 16-byte loads per lane (A)
  static constexpr int NB = BROWS * PB / NT;     // 16-byte loads per lane (B)
  static constexpr int NS = S_BYTES / 4 / NT;    // scale loads per lane (one per slot)
  static constexpr int NAS = MX8 ? MT * 2 / NT : 0;  // activation-scale loads per lane (2 bytes)
  static constexpr int NLOADS = NA + NB + NS + NAS;
  static constexpr int SUPER = (FMT == 0 ? 256 : 512) / KC;  // stages per 16 scale bytes
  // super-stage scale loads: one lane per row, issued by the first SS_WAVES waves
  static constexpr int SS_WAVES = SS ? (BROWS / 64 < NW ? BROWS / 64 : NW) : 0;
  static constexpr int NSS = SS ? BROWS / (SS_WAVES * 64) : 0;  // per lane of those waves
  static constexpr int SS_BYTES = SS ? 2 * BROWS * 16 : 0;       // two super-stage slots
  static constexpr int LEAD = NSTG - 1;  // stages in flight ahead of the one computed
  // FP8: the fp32 scales of the block's weight rows (gate and up, or down), one per
  // (128-row block, 128-code block), for K up to kFp8MaxKb * 128
  static constexpr int MATS = GATEUP ? 2 : 1;
  static constexpr int NBL = (NCOLS + 127) / 128;
  static constexpr int TAB_BYTES = FMT == 2 ? MATS * NBL * kFp8MaxKb * 4 : 0;
  static constexpr size_t SMEM = (size_t)NSTG * STAGE + SS_BYTES + TAB_BYTES;
  static constexpr int BLOCKS_PER_CU = SMEM <= 80 * 1024 ? 2 : 1;
  static_assert(FP4 ? (KC == 64 || KC == 128 || (KC == 256 && SS)) : KC == 32, "stage width");
  static_assert(!SS || FP4, "super-staged scales are FP4 only");
  static_assert(PB >= 2 && WPS * 2 * STEPS * 4 == B_ROW, "B row split over the lane halves");
  static_assert(NA * NT == MT * PA && NB * NT == BROWS * PB && NS * NT * 4 == S_BYTES,
                "a stage must split evenly over the block");
  static_assert(!SS || NSS * SS_WAVES * 64 == BROWS, "one super-stage load per row");
  // gate+up pairs column blocks inside a wave, or (one column block per wave, FP4) across
  // waves: waves 0 .. WN/2-1 hold gate columns, the others the same columns of up
  static_assert(CB % 2 == 0 || !GATEUP || (CB == 1 && WN == 4 && FP4), "gate+up pairs column blocks");
  static_assert(NSTG >= 2 && NSTG <= 5, "ring depth");
  static_assert(LEAD <= SUPER, "a super-stage slot is refilled only after its last read");
  static_assert((LEAD - 1) * NLOADS + NSS <= 63, "the loads in flight must fit the wait counter");
  static_assert(MT * (int)sizeof(int) <= STAGE, "the row map borrows the last stage slot");
  static_assert(SMEM * BLOCKS_PER_CU <= 160 * 1024, "the blocks of a CU must fit its LDS");
};

// waves per SIMD the register allocation must allow: two when two blocks share a CU
template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS>
constexpr int kPreWaves = PreShape<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>::BLOCKS_PER_CU;

// Persistent form (PERSIST): gridDim.x blocks (a multiple of kXcds, at most the resident
// slots) walk the work list of (row tile, column tile) items. The items are split into
// kXcds contiguous ranges, one per XCD; block b (dispatched to XCD b % kXcds) starts at
// item b / kXcds of its range and then takes the next unclaimed item of the range from
// that range's work counter. (Correctness does not depend on where a block runs: every
// item of a range is claimed exactly once by the blocks of that range; only L2 locality
// does.) The stage ring runs on across items: the next item is claimed at step 0 of the
// current one and published in LDS at step 1; at step nch - LEAD every wave reads it, the
// next tile's header and its load sources, and the next tile's first LEAD stages are
// issued during the current item's last LEAD steps, so neither the pipeline fill nor the
// epilogue leaves the CU idle (MoE constructor page: the grouped GEMM runs as a persistent
// grid over the compacted tile work list).
template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS>
constexpr int kPersistLds = PreShape<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>::SMEM + 16;

template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((
    amdgpu_waves_per_eu(kPreWaves<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>, 2)))
void k_pre_gemm(ExpertGemmArgs a) {
  using Sh = PreShape<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>;
  constexpr int NT = Sh::NT;
  constexpr int WN = Sh::WN, BROWS = Sh::BROWS, NCOLS = Sh::NCOLS, MT = Sh::MT;
  constexpr int NA = Sh::NA, NB = Sh::NB, NS = Sh::NS, NSS = Sh::NSS, SUPER = Sh::SUPER;
  constexpr int PA = Sh::PA, PB = Sh::PB, STEPS = Sh::STEPS, SLOTS = Sh::SLOTS;
  constexpr int LEAD = Sh::LEAD;
  static_assert(!PERSIST || (Sh::FP4 && !SS && !GATEUP && !Sh::MX8),
                "persistent form: FP4 down projections with per-stage scales");
  static_assert(!PERSIST || kPersistLds<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS> * Sh::BLOCKS_PER_CU <=
                                160 * 1024, "the claimed-item word must fit beside the ring");
  extern __shared__ __align__(16) uint8_t s_dyn[];
  uint8_t* s_ss = s_dyn + NSTG * Sh::STAGE;  // super-stage scale slots (SS)
  // source row of each A tile row; lives in the last stage slot, which the first load
  // into it (stage LEAD, issued after the first barrier of the main loop) overwrites
  int* s_tok = reinterpret_cast<int*>(s_dyn + LEAD * Sh::STAGE);
  int* s_claim = reinterpret_cast<int*>(s_dyn + Sh::SMEM);  // PERSIST: claimed item

  const int N = GATEUP ? a.I : a.H;  // rows of each weight matrix
  const int K = GATEUP ? a.H : a.I;  // a multiple of KC
  const int ncol_tiles = (N + NCOLS - 1) / NCOLS;
  Tile t;
  int ct;
  // PERSIST: this block's XCD, its range of items [wlo, wlo + wcnt), the XCD's blocks
  int wx = 0, wlo = 0, wcnt = 0, wnb = 0;
  if constexpr (PERSIST) {
    const int real = a.src.ntiles[0] * ncol_tiles;
    wx = blockIdx.x % kXcds;
    wnb = gridDim.x / kXcds;
    const int q = real / kXcds, rem = real % kXcds;
    wlo = wx * q + (wx < rem ? wx : rem);
    wcnt = q + (wx < rem ? 1 : 0);
    const int j = blockIdx.x / kXcds;
    if (j >= wcnt) return;
    t = load_tile_header(a.src.tiles, (wlo + j) / ncol_tiles);
    ct = (wlo + j) % ncol_tiles;
  } else {
    if (!pre_resolve(a, ncol_tiles, t, ct)) return;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, r = lane & 31;
  int e = t.group;
  int n0 = ct * NCOLS;
  const size_t row_bytes = (size_t)K * Sh::B_ROW / KC;
  const int sbytes = Sh::FP4 ? K / (FMT == 0 ? 16 : 32) : 0;
  // the two weight matrices (gate, up) or the one (down), by value: taking addresses of
  // the kernel argument's members would place the whole argument in private memory
  const uint8_t* const pk0 = GATEUP ? a.gate.packed : a.down.packed;
  const uint8_t* const pk1 = GATEUP ? a.up.packed : a.down.packed;
  const uint8_t* const sc0 = GATEUP ? a.gate.scales : a.down.scales;
  const uint8_t* const sc1 = GATEUP ? a.up.scales : a.down.scales;
  float* s_tab = reinterpret_cast<float*>(s_ss + Sh::SS_BYTES);  // FP8 block scales
  if (FMT == 2) {
    // [matrix][128-row block][128-code block] of the rows n0..n0+NCOLS-1 (0 past N)
    const int kb = (K + 127) / 128, nbg = (N + 127) / 128;
    for (int i = threadIdx.x; i < Sh::MATS * Sh::NBL * kb; i += NT) {
      const int m = i / (Sh::NBL * kb), rest = i % (Sh::NBL * kb);
      const int nb = n0 / 128 + rest / kb, kk = rest % kb;
      const float* tab = reinterpret_cast<const float*>(m ? sc1 : sc0);
      s_tab[(m * Sh::NBL + rest / kb) * kFp8MaxKb + kk] =
          nb < nbg ? tab[((size_t)e * nbg + nb) * kb + kk] : 0.0f;
    }
  }

  // gathered token (gate+up) or h row (down); rows past the tile's count repeat its
  // first row (results discarded). The persistent form (down only) computes the rows.
  if constexpr (!PERSIST) {
    for (int i = threadIdx.x; i < MT; i += NT) {
      const int ii = i < t.count ? i : 0;
      // an implicit list's row r holds token r - implicit_row0 (no dispatch output read)
      const int tok = a.src.tiles ? a.row_token[t.row0 + ii] : t.row0 + ii - a.src.implicit_row0;
      s_tok[i] = GATEUP ? tok : t.row0 + ii;
    }
    __syncthreads();
  }

  // Source address of each load of this lane for the tile (tt, column tile ctt) (fixed
  // across stages, + the stage's K offset). The i-th load of a wave fills LDS slots
  // (wave * n + i) * 64 + lane of its region; a slot holds the source piece that the
  // swizzle assigns to it.
  const uint16_t* asrc[NA];
  const uint16_t* assrc = nullptr;
  const uint8_t* bsrc[NB];
  const uint8_t* ssrc[NS > 0 ? NS : 1];
  const uint8_t* sssrc[NSS > 0 ? NSS : 1];
  auto set_sources = [&](const Tile& tt, int ctt) __attribute__((always_inline)) {
    const int te = tt.group, tn0 = ctt * NCOLS;
    // persistent form: the lane index behind an empty asm, so that the per-lane slot
    // arithmetic below is redone at each call instead of held in registers across the loop
    int lane = threadIdx.x & 63;
    if constexpr (PERSIST) asm volatile("" : "+v"(lane));
    // A: PA pieces of 16 bytes per row, slot = piece ^ a_swz(row)
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int slot = (wave * NA + i) * 64 + lane;
      const int row = slot / PA, piece = (slot % PA) ^ a_swz<PA>(row);
      const int src = PERSIST ? tt.row0 + (row < tt.count ? row : 0) : s_tok[row];
      const uint16_t* base = GATEUP ? a.x + (size_t)src * a.H : a.h + (size_t)src * a.h_stride;
#if MOE_PRE_MX8
      if (Sh::MX8)
        base = reinterpret_cast<const uint16_t*>(a.a8) + (size_t)src * (GATEUP ? a.H : a.h_stride);
#endif
      asrc[i] = base + piece * 8;
    }
    // MX8: one (row, 32-code block) activation-scale pair of the stage per lane
#if MOE_PRE_MX8
    if (Sh::MX8) {
      const int pi = (wave * 64 + lane) % (MT * 2);
      assrc = a.a8s + (size_t)s_tok[pi / 2] * (K / 32) + (pi % 2);
    }
#endif
    // weight row of B-tile row brow; rows past N read row 0 of the expert (not stored)
    auto wrow = [&](int brow, bool& second) -> size_t {
      int n;
      if (GATEUP) {
        second = brow >= BROWS / 2;
        n = tn0 + (second ? brow - BROWS / 2 : brow);
      } else {
        second = false;
        n = tn0 + brow;
      }
      return (size_t)te * N + (n < N ? n : 0);
    };
    // B: PB pieces of 16 bytes per row, slot = piece ^ b_swz(row)
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot = (wave * NB + i) * 64 + lane;
      const int brow = slot / PB, piece = (slot % PB) ^ b_swz<PB>(brow);
      bool m;
      const size_t rw = wrow(brow, m);
      bsrc[i] = (m ? pk1 : pk0) + rw * row_bytes + piece * 16;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      bool m;
      const int slot = (wave * NS + i) * 64 + lane;  // 4-byte slot u of its row: 64 codes
      constexpr int SL = SLOTS > 0 ? SLOTS : 1;  // (no such loads for FP8 / BF16)
      const size_t rw = wrow(slot / SL, m);
      ssrc[i] = (m ? sc1 : sc0) + rw * sbytes + (slot % SL) * (FMT == 0 ? 4 : 2);
    }
#pragma unroll
    for (int i = 0; i < NSS; ++i) {
      bool m;
      const int row = (wave * NSS + i) * 64 + lane;  // one lane per row (waves < SS_WAVES)
      const size_t rw = wrow(row < BROWS ? row : 0, m);
      sssrc[i] = (m ? sc1 : sc0) + rw * sbytes;
    }
  };
  set_sources(t, ct);

  // split z of a.ksplit takes K codes [kbase, kbase + K / ksplit) (a whole number of
  // super-stages when SS holds)
  const int kspan = K / a.ksplit;
  const int kbase = blockIdx.z * kspan;
  const int nch = kspan / KC;

  // Loads of stage c into ring slot `slot`: always NLOADS per lane, so the wait count is a
  // constant.
  auto issue = [&](int c, int slot) __attribute__((always_inline)) {
    const uint32_t abase = lds_addr(s_dyn + slot * Sh::STAGE);
    const uint32_t bbase = abase + Sh::A_BYTES, sbase = bbase + Sh::B_BYTES;
    const int k0 = kbase + c * KC;
    if (SS && c % SUPER == 0 && wave < Sh::SS_WAVES) {
      const int j = (kbase / KC + c) / SUPER;  // 16-byte piece of the scale rows
      const uint32_t ssbase = lds_addr(s_ss + ((c / SUPER) & 1) * BROWS * 16);
#pragma unroll
      for (int i = 0; i < NSS; ++i) {
        const int slot0 = (wave * NSS + i) * 64;
        dma16(sssrc[i] + 16 * j, __builtin_amdgcn_readfirstlane(ssbase + slot0 * 16));
      }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int slot0 = (wave * NA + i) * 64;
      dma16(asrc[i] + k0, __builtin_amdgcn_readfirstlane(abase + slot0 * 16));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot0 = (wave * NB + i) * 64;
      if (KC == 256)
        dma16_nt(bsrc[i] + (size_t)k0 * Sh::B_ROW / KC, __builtin_amdgcn_readfirstlane(bbase + slot0 * 16));
      else
        dma16(bsrc[i] + (size_t)k0 * Sh::B_ROW / KC, __builtin_amdgcn_readfirstlane(bbase + slot0 * 16));
    }
    if (Sh::MX8) {
      const uint32_t asbase = sbase + Sh::S_BYTES;
      dma2(assrc + k0 / 32, __builtin_amdgcn_readfirstlane(asbase + wave * 64 * 4));
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int slot0 = (wave * NS + i) * 64;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + slot0 * 4);
      if (FMT == 0) {
        dma4(ssrc[i] + k0 / 16, dst);
      } else {
        dma2(ssrc[i] + k0 / 32, dst);
      }
    }
  };

  // ring slot of the current tile's stage 0 (the persistent form carries the ring on
  // from tile to tile), and whether a next tile was claimed (persistent form, from step 2)
  int ring0 = 0;
  bool has_next = false;
  Tile tn{};
  int ctn = 0;
  // loads issued after the MFMA step of stage c: stage c + LEAD of this tile, or of the next
  auto issue_after = [&](int c) __attribute__((always_inline)) {
    const int n = c + LEAD;
    const int slot = (ring0 + n) % NSTG;
    if (n < nch) {
      issue(n, slot);
    } else if (PERSIST && has_next) {
      issue(n - nch, slot);
    }
  };

  f32x16_t acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16_t{};

  // B-tile rows of this wave's column blocks
  // (gate+up: column blocks 0..CB/2-1 are gate rows, CB/2.. the same rows of up)
  // XW: one column block per wave, gate in waves 0 and 1, up in waves 2 and 3 (paired in
  // the epilogue through LDS)
  constexpr bool XW = GATEUP && CB == 1;
  constexpr int CH = GATEUP ? (XW ? 1 : CB / 2) : CB;
  int brow0[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    brow0[cb] = XW ? wn * 32
                   : GATEUP ? (cb / CH) * (BROWS / 2) + wn * CH * 32 + (cb % CH) * 32
                            : wn * CB * 32 + cb * 32;
  }
  const int arow = wm * 32 * RB + r;  // + rb * 32
  const int bsw = b_swz<PB>(r);  // = b_swz(brow0[cb] + r): brow0 is a multiple of 32


  // MFMAs of stage c for the first NR row blocks: STEPS steps of K 16, lane half h
  // covering codes (KC/2)h..(KC/2)h+KC/2-1 of the stage (8 per step)
  auto stage_mma = [&](auto nr_c, int c) __attribute__((always_inline)) {
    constexpr int NR = decltype(nr_c)::value;
    if constexpr (NR == 0) {
      issue_after(c);
      return;
    }
    const uint8_t* sa = s_dyn + ((ring0 + c) % NSTG) * Sh::STAGE;
    const uint8_t* sbq = sa + Sh::A_BYTES;
    const uint8_t* ssc = sbq + Sh::B_BYTES;
    constexpr int WPS = Sh::WPS;
    uint32_t q[CB][STEPS * WPS];
    ScaleWord<Sh::SW> sc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int srow = brow0[cb] + r;
#pragma unroll
      for (int j = 0; j < PB / 2; ++j) {
        const int piece = (PB / 2) * half + j;
        const uint4 v = *reinterpret_cast<const uint4*>(sbq + srow * Sh::B_ROW + ((piece ^ bsw) << 4));
        q[cb][4 * j] = v.x; q[cb][4 * j + 1] = v.y; q[cb][4 * j + 2] = v.z; q[cb][4 * j + 3] = v.w;
      }
      if (Sh::FP4) {
        // this lane's scale bytes of the stage (blocks of its codes: NVFP4 KC/32, MXFP4 KC/64)
        const uint8_t* sp =
            SS ? s_ss + ((c / SUPER) & 1) * BROWS * 16 + srow * 16 + (c % SUPER) * 2 * Sh::SW +
                     half * Sh::SW
               : ssc + srow * Sh::SROW + (SLOTS == 2 ? 4 * half : half * Sh::SW);
        sc[cb] = lds_scale<Sh::SW>(sp);
      } else if (FMT == 2) {
        // the column block's 32 rows lie in one 128-row block; the stage in one 128-code block
        const int m = GATEUP ? cb / CH : 0;
        const int nbl = ((GATEUP ? brow0[cb] - m * (BROWS / 2) : brow0[cb])) / 128;
        sc[cb] = __float_as_uint(s_tab[(m * Sh::NBL + nbl) * kFp8MaxKb + (kbase + c * KC) / 128]);
      } else {
        sc[cb] = 0u;
      }
    }
#if MOE_PRE_MX8
    if constexpr (Sh::MX8) {
      // block-scaled MFMA, K = 64: weights (E2M1, lane half h: codes 32h..32h+31, one E8M0
      // scale) first; activations second as an MXFP8 hi and lo pair, lane half h holding
      // codes 16h..16h+15 and 32+16h..47+16h (pieces h, 4+h of hi; 2+h, 6+h of lo), with
      // the E8M0 scales of block h
      const uint8_t* sas = ssc + Sh::S_BYTES;
      typedef int v8i_t __attribute__((ext_vector_type(8)));
      v8i_t wq[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        wq[cb] = v8i_t{(int)q[cb][0], (int)q[cb][1], (int)q[cb][2], (int)q[cb][3], 0, 0, 0, 0};
      issue_after(c);
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        const int row = arow + rb * 32;
        const uint8_t* rp = sa + row * Sh::A_ROW;
        const int sw = a_swz<PA>(row);
        const uint4 h0 = *reinterpret_cast<const uint4*>(rp + ((half ^ sw) << 4));
        const uint4 h1 = *reinterpret_cast<const uint4*>(rp + (((4 + half) ^ sw) << 4));
        const uint4 l0 = *reinterpret_cast<const uint4*>(rp + (((2 + half) ^ sw) << 4));
        const uint4 l1 = *reinterpret_cast<const uint4*>(rp + (((6 + half) ^ sw) << 4));
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sas + (row * 2 + half) * 4);
        const v8i_t vh{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        const v8i_t vl{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wq[cb], vh, acc[rb][cb], 4, 0, 0, (int)sc[cb], 0, (int)(s2 & 0xFFu));
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wq[cb], vl, acc[rb][cb], 4, 0, 0, (int)sc[cb], 0, (int)(s2 >> 8));
        }
      }
      return;
    }
#endif
    // A operands are read AHEAD steps before their MFMAs, in the order of use (LDS reads
    // return in order), so that LDS latency overlaps the MFMAs of the steps before; two
    // steps of RB x CB MFMAs cover it, and holding only AHEAD steps of operands leaves
    // registers to spare under the budget of two waves per SIMD
    constexpr int AHEAD = STEPS < 2 ? STEPS : 2;
    uint4 av[NR > 0 ? NR : 1][AHEAD];
    auto read_a = [&](int s) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        const int row = arow + rb * 32;
        av[rb][s % AHEAD] = *reinterpret_cast<const uint4*>(
            sa + row * Sh::A_ROW + (((STEPS * half + s) ^ a_swz<PA>(row)) << 4));
        __builtin_amdgcn_sched_barrier(0);  // keep the reads in the order they are used
      }
    };
#pragma unroll
    for (int s = 0; s < AHEAD; ++s) read_a(s);
    // the loads of stage c + LEAD go out while this stage's LDS reads are in flight
    issue_after(c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      bf16x8_t bo[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (Sh::FP4) {
          bo[cb] = b_operand<FMT>(q[cb][s], sc[cb], s);
        } else if (FMT == 2) {
          uint32_t d[4];
          mfma_operand_fp8x8(q[cb][2 * s], q[cb][2 * s + 1], __uint_as_float(sc[cb]), d);
          bo[cb] = as_bf16x8(d);
        } else {
          const uint32_t d[4] = {q[cb][4 * s], q[cb][4 * s + 1], q[cb][4 * s + 2], q[cb][4 * s + 3]};
          bo[cb] = as_bf16x8(d);
        }
      }
      bf16x8_t af[NR > 0 ? NR : 1];
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) af[rb] = __builtin_bit_cast(bf16x8_t, av[rb][s % AHEAD]);
      if (s + AHEAD < STEPS) read_a(s + AHEAD);
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[cb], af[rb], acc[rb][cb], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int i = 0; i < LEAD; ++i)
    if (i < nch) issue(i, i % NSTG);
#if MOE_PRE_WAIT_SPLIT
  unsigned long long ws_load = 0, ws_bar = 0, ws_steps = 0;
#endif
  auto kloop = [&](auto nr_c) __attribute__((always_inline)) {
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
      // may stay in flight: stages c+1 .. c+LEAD-1 (fewer near the end), one of which may
      // start a super-stage of scales (at most one: LEAD <= SUPER)
      int inflight = nch - 1 - c;
      inflight = inflight < LEAD - 1 ? inflight : LEAD - 1;
      bool ss = false;
      if (SS && wave < Sh::SS_WAVES) {
        const int next = (c / SUPER + 1) * SUPER;  // first super-stage start after c
        ss = next <= c + inflight;
      }
#if MOE_PRE_WAIT_SPLIT
      const unsigned long long t0 = __builtin_amdgcn_s_memtime();
      wait_loads_inflight<Sh::NLOADS, NSS>(inflight, ss);
      const unsigned long long t1 = __builtin_amdgcn_s_memtime();
      asm volatile("s_barrier" ::: "memory");
      const unsigned long long t2 = __builtin_amdgcn_s_memtime();
      ws_load += t1 - t0;
      ws_bar += t2 - t1;
      ws_steps += 1;
#else
      wait_inflight<Sh::NLOADS, NSS>(inflight, ss);
#endif
      stage_mma(nr_c, c);
    }
  };
  // persistent form: the same steps in two runs. Steps 0 .. nch - LEAD - 1 claim the next
  // tile (step 0 takes the item, step 1 publishes it in LDS); between the runs every wave
  // reads the claim, the next tile's header and its load sources; steps nch - LEAD .. nch - 1
  // then issue the next tile's first LEAD stages (nch >= LEAD + 3, checked by the launcher).
  // No next-tile state is carried from step to step.
  int claim = 0;
  auto kloop_persist = [&](auto nr_c) __attribute__((always_inline)) {
#pragma unroll 1
    for (int c = 0; c < nch - LEAD; ++c) {
      wait_inflight<Sh::NLOADS, NSS>(LEAD - 1, false);
      if (c == 0) {
        // claimed before this step's loads, so the next step's wait covers it; an
        // increment that wraps only at 2^32 - 1 (not an add, which the compiler would
        // spread over the wave and wait for at once)
        if (threadIdx.x == 0)
          claim = (int)__builtin_amdgcn_atomic_inc32(
              reinterpret_cast<unsigned*>(a.work + wx * kWorkCtrStride), 0xFFFFFFFFu,
              __ATOMIC_RELAXED, "agent");
      } else if (c == 1) {
        if (threadIdx.x == 0) *s_claim = claim;
      }
      stage_mma(nr_c, c);
    }
    // (the claim was written at step 1 and the barrier of step 2 has passed)
    const int jn = wnb + __builtin_amdgcn_readfirstlane(*s_claim);
    has_next = jn < wcnt;
    if (has_next) {
      tn = load_tile_header(a.src.tiles, (wlo + jn) / ncol_tiles);
      ctn = (wlo + jn) % ncol_tiles;
      set_sources(tn, ctn);
    }
#pragma unroll 1
    for (int c = nch - LEAD; c < nch; ++c) {
      int inflight = LEAD - 1;
      if (!has_next && nch - 1 - c < inflight) inflight = nch - 1 - c;
      wait_inflight<Sh::NLOADS, NSS>(inflight, false);
      stage_mma(nr_c, c);
    }
  };
  // row blocks of this wave that hold rows of the tile: a partly filled tile skips the
  // MFMAs of its empty 32-row blocks
  auto run_tile = [&](auto loop) __attribute__((always_inline)) {
    int nrb = (t.count - wm * 32 * RB + 31) / 32;
    nrb = nrb < 0 ? 0 : (nrb > RB ? RB : nrb);
    if (nrb >= RB) {
      loop(std::integral_constant<int, RB>{});
    } else if (nrb == 1) {
      loop(std::integral_constant<int, 1>{});
    } else if (nrb == 2) {  // (RB > 2 only)
      loop(std::integral_constant<int, (RB > 2 ? 2 : 1)>{});
    } else if (nrb == 3) {  // (RB > 3 only)
      loop(std::integral_constant<int, (RB > 3 ? 3 : 1)>{});
    } else {
      loop(std::integral_constant<int, 0>{});
    }
  };

  // epilogue. The weights are the MFMA's first operand, so block (rb, cb) holds
  // out[token][n] transposed: lane l owns token row wm*32*RB + rb*32 + l % 32 and, in
  // element v, column 8*(v/4) + 4*half + v%4 of the 32-column block, i.e. four runs of 4
  // consecutive columns: fp32 outputs are stored one run per write (16 bytes), 16-bit ones
  // (h, fp16 y) 8 columns per write after a swap between the lane halves
  // (store_cols32_16bit). Column blocks are 32-aligned and N is a multiple of 32, so a block
  // is wholly inside N or wholly outside.
  auto epilogue = [&]() __attribute__((always_inline)) {
    if (!PERSIST && a.ksplit > 1) {  // (the persistent form never splits K)
      // split K: the raw fp32 sums of this split, [split][row][gate cols | up cols] or
      // [split][row][H] (rows relative to the implicit list); scales and SwiGLU come with
      // the reduce
      const int NO = GATEUP ? 2 * a.I : a.H;
      float* prow0 = a.part + (size_t)blockIdx.z * a.src.implicit_rows * NO;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int col = XW ? n0 + (wn & 1) * 32
                           : GATEUP ? n0 + wn * CH * 32 + (cb % CH) * 32 : n0 + wn * CB * 32 + cb * 32;
        if (col >= N) continue;
        const int ocol = XW ? (wn >= 2 ? a.I + col : col) : (GATEUP && cb >= CH ? a.I + col : col);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = wm * 32 * RB + rb * 32 + r;
          if (i >= t.count) continue;
          float* prow = prow0 + (size_t)(t.row0 + i - a.src.implicit_row0) * NO + ocol + 4 * half;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x16_t& cc = acc[rb][cb];
            *reinterpret_cast<float4*>(prow + 8 * g4) =
                make_float4(cc[4 * g4], cc[4 * g4 + 1], cc[4 * g4 + 2], cc[4 * g4 + 3]);
          }
        }
      }
    } else if constexpr (XW) {
      // up waves hand their sums to the gate waves of the same columns through LDS (the
      // stage ring is idle once every wave has left the K loop)
      const float gs_g = FMT == 0 ? a.gate.global[e] : 1.0f;
      const float gs_u = FMT == 0 ? a.up.global[e] : 1.0f;
      float* s_u = reinterpret_cast<float*>(s_dyn);
      __syncthreads();
      if (wn >= 2) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int v = 0; v < 16; ++v) s_u[(((wn - 2) * RB + rb) * 16 + v) * 64 + lane] = acc[rb][0][v];
      }
      __syncthreads();
      const int nb = n0 + (wn & 1) * 32;
      if (wn < 2 && nb < N) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = wm * 32 * RB + rb * 32 + r;
          if (i >= t.count) continue;
          uint32_t pk[4][2];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int v = 4 * g4 + j;
              const float g = acc[rb][0][v] * gs_g;
              const float u = s_u[((wn * RB + rb) * 16 + v) * 64 + lane] * gs_u;
              hv[j] = silu(g) * u;
            }
            pk[g4][0] = pack_bf16x2(hv[0], hv[1]);
            pk[g4][1] = pack_bf16x2(hv[2], hv[3]);
          }
          store_cols32_16bit(a.h + (size_t)(t.row0 + i) * a.h_stride + nb, pk, half);
        }
      }
    } else if (GATEUP) {
      const float gs_g = FMT == 0 ? a.gate.global[e] : 1.0f;
      const float gs_u = FMT == 0 ? a.up.global[e] : 1.0f;
#pragma unroll
      for (int cg = 0; cg < CH; ++cg) {
        const int nb = n0 + wn * CH * 32 + cg * 32;
        if (nb >= N) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = wm * 32 * RB + rb * 32 + r;
          if (i >= t.count) continue;
          uint32_t pk[4][2];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float g = acc[rb][cg][4 * g4 + j] * gs_g;
              const float u = acc[rb][CH + cg][4 * g4 + j] * gs_u;
              hv[j] = silu(g) * u;
            }
            pk[g4][0] = pack_bf16x2(hv[0], hv[1]);
            pk[g4][1] = pack_bf16x2(hv[2], hv[3]);
          }
          store_cols32_16bit(a.h + (size_t)(t.row0 + i) * a.h_stride + nb, pk, half);
        }
      }
    } else {
      // y is fp32, or fp16 for routed prefill rows (y_half): the blend reads it once, and
      // fp16's 11-bit significand keeps its rounding an eighth of a bf16 one (bf16 would add
      // up to half a bf16 ulp of every expert output to the layer's error)
      const float gs = FMT == 0 ? load_uniform_f32(a.down.global, e) : 1.0f;
      float* y = reinterpret_cast<float*>(a.y);
      uint16_t* y16 = reinterpret_cast<uint16_t*>(a.y);
      bool range = false;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int nb = n0 + wn * CB * 32 + cb * 32;
        if (nb >= N) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = wm * 32 * RB + rb * 32 + r;
          if (i >= t.count) continue;
          const size_t off = (size_t)(t.row0 + i) * a.H + nb + 4 * half;
          const f32x16_t& c = acc[rb][cb];
          if (a.y_half) {
            // round to fp16; a value that rounds past +-65504 (or is not finite) is rare, so
            // the saturating conversion runs only for a lane that produced one
            uint32_t pk[4][2], nf = 0;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              pk[g4][0] = pack_f16x2(c[4 * g4] * gs, c[4 * g4 + 1] * gs);
              pk[g4][1] = pack_f16x2(c[4 * g4 + 2] * gs, c[4 * g4 + 3] * gs);
              nf |= f16x2_nonfinite_bits(pk[g4][0]) | f16x2_nonfinite_bits(pk[g4][1]);
            }
            if (nf) {
              range = true;
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                pk[g4][0] = pack_f16x2_sat(c[4 * g4] * gs, c[4 * g4 + 1] * gs);
                pk[g4][1] = pack_f16x2_sat(c[4 * g4 + 2] * gs, c[4 * g4 + 3] * gs);
              }
            }
            store_cols32_16bit(y16 + (size_t)(t.row0 + i) * a.H + nb, pk, half);
          } else {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const float v0 = c[4 * g4] * gs, v1 = c[4 * g4 + 1] * gs;
              const float v2 = c[4 * g4 + 2] * gs, v3 = c[4 * g4 + 3] * gs;
              *reinterpret_cast<float4*>(y + off + 8 * g4) = make_float4(v0, v1, v2, v3);
            }
          }
        }
      }
      // a value beyond the fp16 range was saturated: flag it (rare; one lane of the wave)
      if (a.y_half && __builtin_amdgcn_ballot_w64(range) != 0ull && (threadIdx.x & 63) == 0 &&
          a.err_word)
        atomicOr(a.err_word, MOE_DEVERR_Y_RANGE);
    }
  };

  if constexpr (PERSIST) {
    for (;;) {
      run_tile(kloop_persist);
      epilogue();
      if (!has_next) break;
      t = tn;
      ct = ctn;
      e = t.group;
      n0 = ct * NCOLS;
      ring0 = (ring0 + nch) % NSTG;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16_t{};
    }
  } else {
#if MOE_PRE_WAIT_SPLIT
    const unsigned long long ts = __builtin_amdgcn_s_memtime();
#endif
    run_tile(kloop);
#if MOE_PRE_WAIT_SPLIT
    const unsigned long long te = __builtin_amdgcn_s_memtime();
    const int bid = blockIdx.y * gridDim.x + blockIdx.x;
    if (FMT == 1 && a.src.tiles && blockIdx.z == 0 && (threadIdx.x & 63) == 0 && bid < kWaitSplitBlocks) {
      unsigned long long* d = g_wait_split[GATEUP ? 0 : 1][bid][threadIdx.x >> 6];
      d[0] = te - ts;
      d[1] = ws_load;
      d[2] = ws_bar;
      d[3] = ws_steps;
    }
#endif
    epilogue();
  }
}

// Sum of the K splits of a shared-expert GEMM, in split order, then the epilogue of the
// unsplit kernel: gate+up x global scales, SiLU(gate) * up to bf16 h; down x global scale
// to fp32 y. One thread per 4 consecutive outputs of a row.
template <bool GATEUP>
__global__ __launch_bounds__(256) void k_splitk_reduce(ExpertGemmArgs a) {
  const int NC = GATEUP ? a.I : a.H;  // output columns
  const int NO = GATEUP ? 2 * a.I : a.H;  // partial-sum columns
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  const int rows = a.src.implicit_rows;
  if (q >= rows * (NC / 4)) return;
  const int r = q / (NC / 4), n = (q % (NC / 4)) * 4;
  const size_t split = (size_t)rows * NO;
  const float* p = a.part + (size_t)r * NO + n;
  float4 g = *reinterpret_cast<const float4*>(p);
  float4 u = GATEUP ? *reinterpret_cast<const float4*>(p + a.I) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z = 1; z < a.ksplit; ++z) {
    const float4 gz = *reinterpret_cast<const float4*>(p + z * split);
    g.x += gz.x; g.y += gz.y; g.z += gz.z; g.w += gz.w;
    if (GATEUP) {
      const float4 uz = *reinterpret_cast<const float4*>(p + z * split + a.I);
      u.x += uz.x; u.y += uz.y; u.z += uz.z; u.w += uz.w;
    }
  }
  const int row = a.src.implicit_row0 + r;
  if (GATEUP) {
    const float gs_g = a.gate.fmt == 0 ? a.gate.global[0] : 1.0f;
    const float gs_u = a.up.fmt == 0 ? a.up.global[0] : 1.0f;
    const float h0 = silu(g.x * gs_g) * (u.x * gs_u), h1 = silu(g.y * gs_g) * (u.y * gs_u);
    const float h2 = silu(g.z * gs_g) * (u.z * gs_u), h3 = silu(g.w * gs_g) * (u.w * gs_u);
    *reinterpret_cast<uint2*>(a.h + (size_t)row * a.h_stride + n) =
        make_uint2(pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
  } else {
    const float gs = a.down.fmt == 0 ? a.down.global[0] : 1.0f;
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + (size_t)row * a.H + n) =
        make_float4(g.x * gs, g.y * gs, g.z * gs, g.w * gs);
  }
}

// Compute units of the current device (cached per device).
static int device_cus() {
  constexpr int kMaxDev = 64;
  static int cus[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// K splits for a GEMM over an implicit row list (the shared expert) whose blocks would
// not fill the resident slots: the largest split that keeps each split a whole number of
// `unit` codes and at least MOE_SPLIT_MIN_STAGES stages, the grid within twice the slots,
// and the partial sums within the workspace's share.
#ifndef MOE_SPLIT_MIN_STAGES
#define MOE_SPLIT_MIN_STAGES 4
#endif
static int pick_ksplit(const ExpertGemmArgs& a, int K, int KC, int unit, int blocks, int slots,
                       int nout) {
  if (a.src.tiles || !a.part || blocks >= slots) return 1;
  const size_t per = (size_t)a.src.implicit_rows * nout * sizeof(float);
  int best = 1;
  for (int ks = 2; ks <= kMaxKsplit; ++ks) {
    if (K % (ks * unit) != 0 || K / ks / KC < MOE_SPLIT_MIN_STAGES) continue;
    if ((long long)blocks * ks > 2LL * slots || per * ks > a.part_bytes) continue;
    best = ks;
  }
  return best;
}

// The persistent form (down projections of FP4 weights with per-stage scales, over the
// device tile list): when the tile grid exceeds the resident block slots and each tile
// has enough stages for the claim of the next one to land first.
#ifndef MOE_PRE_PERSIST
#define MOE_PRE_PERSIST 1
#endif
template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS>
constexpr bool kCanPersist = MOE_PRE_PERSIST && !GATEUP && !SS && FMT <= 1 &&
                             !PreShape<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>::MX8;

template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS, bool PERSIST>
static hipError_t set_lds_limit() {
  using Sh = PreShape<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>;
  const int bytes = PERSIST ? kPersistLds<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS> : (int)Sh::SMEM;
  // one attribute call per instantiation and process (a function-local static: thread-safe)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_pre_gemm<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS, PERSIST>),
      hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return attr;
}

template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP, bool SS>
static hipError_t launch_pre_ss(const ExpertGemmArgs& a0, hipStream_t s) {
  using Sh = PreShape<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>;
  const int N = GATEUP ? a0.I : a0.H;
  const int K = GATEUP ? a0.H : a0.I;
  const int ncol = (N + Sh::NCOLS - 1) / Sh::NCOLS;
  const int slots = device_cus() * Sh::BLOCKS_PER_CU;
  ExpertGemmArgs a = a0;
  // FP8 / BF16 blocks keep the whole K (the FP8 block-scale table is per block)
  a.ksplit = Sh::FP4 ? pick_ksplit(a, K, KC, SS ? KC * Sh::SUPER : KC, ncol * a.tile_bound, slots,
                                   GATEUP ? 2 * a.I : a.H)
                     : 1;
  if constexpr (kCanPersist<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>) {
    const int grid = slots / kXcds * kXcds;
    if (a.work && a.src.tiles && a.ksplit == 1 && K / KC >= Sh::LEAD + 3 && grid > 0 &&
        (long long)ncol * a.tile_bound > grid) {
      const hipError_t attr = set_lds_limit<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS, true>();
      if (attr != hipSuccess) return attr;
      constexpr int lds = kPersistLds<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS>;
      auto kern = k_pre_gemm<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS, true>;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(Sh::NT), lds, s, a);
      return hipGetLastError();
    }
  }
  const hipError_t attr = set_lds_limit<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS, false>();
  if (attr != hipSuccess) return attr;
  auto kern = k_pre_gemm<FMT, KC, NSTG, RB, WM, CB, GATEUP, SS, false>;
  hipLaunchKernelGGL(kern, dim3(ncol, a.tile_bound, a.ksplit), dim3(Sh::NT), Sh::SMEM, s, a);
  if (a.ksplit > 1) {
    const int nc = GATEUP ? a.I : a.H;
    const int threads = a.src.implicit_rows * (nc / 4);
    hipLaunchKernelGGL(k_splitk_reduce<GATEUP>, dim3((threads + 255) / 256), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// Super-staged scales when each scale row is a whole number of 16-byte pieces.
template <int FMT, int KC, int NSTG, int RB, int WM, int CB, bool GATEUP>
static hipError_t launch_pre_shape(const ExpertGemmArgs& a, hipStream_t s) {
  const int K = GATEUP ? a.H : a.I;
  if (K % KC != 0) return hipErrorInvalidValue;
  if constexpr (FMT >= 2) {
    if (FMT == 2 && (K + 127) / 128 > kFp8MaxKb) return hipErrorInvalidValue;
    return launch_pre_ss<FMT, KC, NSTG, RB, WM, CB, GATEUP, false>(a, s);
  } else {
    const int sbytes = K / (FMT == 0 ? 16 : 32);
#if MOE_PRE_MX8
    if constexpr (FMT == 1 && KC == 64) return launch_pre_ss<FMT, KC, NSTG, RB, WM, CB, GATEUP, false>(a, s);
#endif
    if (sbytes % 16 == 0) return launch_pre_ss<FMT, KC, NSTG, RB, WM, CB, GATEUP, true>(a, s);
    if constexpr (KC == 256) return hipErrorInvalidValue;  // (super-staged scales only)
    else return launch_pre_ss<FMT, KC, NSTG, RB, WM, CB, GATEUP, false>(a, s);
  }
}

// Tile height MT -> stage width KC and block shape (row blocks per wave RB, waves along M
// WM, column blocks per wave CB): FP4 128 = 64-code stages, 4 x 1 x 2 (128 x 256 weight
// rows; each wave all 128 rows, so a decoded B operand feeds four MFMAs); FP4 64 = 64-code
// stages, 2 x 1 x 2 (64 x 256); FP4 32 = 128-code stages, 1 x 1 x 2 (32 x 256: twice the
// blocks of 32 x 512, which balanced worse), except MXFP4 with K a multiple of 512 and
// NVFP4 with K a multiple of 256: 256-code stages in a two-slot ring, 1 x 1 x 1 (32 x 128). K that is not a multiple of 128
// takes 64-code stages, 1 x 1 x 4 (32 x 512), at height 32.
#ifndef MOE_PRE_NSTG
#define MOE_PRE_NSTG 3
#endif
template <bool GATEUP>
static hipError_t launch_pre(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  const int fmt = GATEUP ? a.gate.fmt : a.down.fmt;
  const int K = GATEUP ? a.H : a.I;
  constexpr int NS3 = MOE_PRE_NSTG;
  if (fmt == 0) {
    if (mt == 32) {
      // K a multiple of 256: 256-code stages reading whole weight lines, as for MXFP4 below
      if (K % 256 == 0) return launch_pre_shape<0, 256, 2, 1, 1, 1, GATEUP>(a, s);
      return K % 128 == 0 ? launch_pre_shape<0, 128, 3, 1, 1, 2, GATEUP>(a, s)
                          : launch_pre_shape<0, 64, 3, 1, 1, 4, GATEUP>(a, s);
    }
    if (mt == 64) return launch_pre_shape<0, 64, 3, 2, 1, 2, GATEUP>(a, s);
    return launch_pre_shape<0, 64, NS3, 4, 1, 2, GATEUP>(a, s);
  }
  // MXFP4 at 32-row tiles with K a multiple of 512: 256-code stages, so each stage reads
  // whole 128-byte lines of the weight rows (with 128-code stages the second half of every
  // line was fetched again one stage later: 1.42x the weight bytes at the hash layer's
  // gate+up). Gate+up pairs gate and up columns across waves to keep the block at 68 KB.
  if (mt == 32 && fmt == 1 && K % 512 == 0)
    return launch_pre_shape<1, 256, 2, 1, 1, 1, GATEUP>(a, s);
  if (mt == 32 && fmt == 1) {
    return K % 128 == 0 ? launch_pre_shape<1, 128, 3, 1, 1, 2, GATEUP>(a, s)
                        : launch_pre_shape<1, 64, 3, 1, 1, 4, GATEUP>(a, s);
  }
  if (fmt == 1) {
    if (mt == 64) return launch_pre_shape<1, 64, 3, 2, 1, 2, GATEUP>(a, s);
    return launch_pre_shape<1, 64, NS3, 4, 1, 2, GATEUP>(a, s);
  }
  // FP8 / BF16 weights: 32-code stages; 32-row tiles run in the 64-row shape (its second
  // row block idle)
  if (fmt == 2) {
    if (mt <= 64) return launch_pre_shape<2, 32, 3, 1, 2, 4, GATEUP>(a, s);
    return launch_pre_shape<2, 32, 3, 2, 2, 4, GATEUP>(a, s);
  }
  if (mt <= 64) return launch_pre_shape<3, 32, 3, 1, 2, 4, GATEUP>(a, s);
  return launch_pre_shape<3, 32, 3, 2, 2, 4, GATEUP>(a, s);
}

#if MOE_PRE_MX8
// Block-scaled MFMA variant: each 32-value block of a bf16 row as an MXFP8 (E4M3 + E8M0) hi
// value and an
// MXFP8 lo value of the residual x - hi. Scale 2^(floor(log2 amax) - 7) (the block's amax
// lands in [128, 256), inside E4M3's range). Output row: per block 32 hi bytes then 32 lo.
__global__ __launch_bounds__(256) void k_quant_mx8(const uint16_t* src, int rows, int K, int stride,
                                                  uint8_t* dst, uint16_t* scales) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int nb = K / 32;
  if (i >= rows * nb) return;
  const int r = i / nb, b = i % nb;
  const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)r * stride + b * 32);
  float x[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * q + 2 * j] = bf16_to_f32(d[j] & 0xFFFFu);
      x[8 * q + 2 * j + 1] = bf16_to_f32(d[j] >> 16);
    }
  }
  auto scale_byte = [](float amax) -> int {
    if (!(amax > 0.f)) return 0;
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;  // floor(log2), normals
    const int e = ex - 7;
    return e + 127 < 0 ? 0 : (e + 127 > 254 ? 254 : e + 127);
  };
  auto pow2 = [](int e) { return __uint_as_float((uint32_t)(e + 127) << 23); };  // e in [-126, 127]
  uint32_t packed[2][8];
  int sb[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
    sb[pass] = scale_byte(amax);
    const int e = sb[pass] - 127;
    // x * 2^-e in two exact power-of-two steps (2^-e alone may not be a normal float)
    const float m1 = pow2(-e / 2), m2 = pow2(-e - (-e / 2));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int w = 0;
      w = __builtin_amdgcn_cvt_pk_fp8_f32((x[4 * j] * m1) * m2, (x[4 * j + 1] * m1) * m2, w, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32((x[4 * j + 2] * m1) * m2, (x[4 * j + 3] * m1) * m2, w, true);
      packed[pass][j] = (uint32_t)w;
    }
    if (pass == 0) {  // residual of the hi values
      const float u1 = pow2(e / 2), u2 = pow2(e - e / 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int w = (int)packed[0][j];
        const float hv[4] = {__builtin_amdgcn_cvt_f32_fp8(w, 0), __builtin_amdgcn_cvt_f32_fp8(w, 1),
                             __builtin_amdgcn_cvt_f32_fp8(w, 2), __builtin_amdgcn_cvt_f32_fp8(w, 3)};
#pragma unroll
        for (int t = 0; t < 4; ++t) x[4 * j + t] -= (hv[t] * u1) * u2;
      }
    }
  }
  uint4* o = reinterpret_cast<uint4*>(dst + (size_t)r * stride * 2 + b * 64);
  o[0] = make_uint4(packed[0][0], packed[0][1], packed[0][2], packed[0][3]);
  o[1] = make_uint4(packed[0][4], packed[0][5], packed[0][6], packed[0][7]);
  o[2] = make_uint4(packed[1][0], packed[1][1], packed[1][2], packed[1][3]);
  o[3] = make_uint4(packed[1][4], packed[1][5], packed[1][6], packed[1][7]);
  scales[(size_t)r * nb + b] = (uint16_t)(sb[0] | (sb[1] << 8));
}

hipError_t launch_quant_mx8(const uint16_t* src, int rows, int K, int stride, uint8_t* dst,
                            uint16_t* scales, hipStream_t s) {
  const int n = rows * (K / 32);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_mx8, dim3((n + 255) / 256), dim3(256), 0, s, src, rows, K, stride,
                     dst, scales);
  return hipGetLastError();
}
#endif

hipError_t launch_prefill_gate_up(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<true>(a, mt, s);
}

hipError_t launch_prefill_down(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<false>(a, mt, s);
}

}  // namespace moe

#if MOE_PRE_WAIT_SPLIT
// Diagnostic build only (not declared in the public header): copy g_wait_split to `host`
// (2 x 8192 x 4 x 4 uint64) and clear it.
extern "C" int moe_debug_prefill_wait_split(void* host) {
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(moe::g_wait_split), sizeof(moe::g_wait_split), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return -4;
  static unsigned long long zero[2][moe::kWaitSplitBlocks][4][4];
  return hipMemcpyToSymbol(HIP_SYMBOL(moe::g_wait_split), zero, sizeof(zero), 0,
                           hipMemcpyHostToDevice) == hipSuccess ? 0 : -4;
}
#endif
