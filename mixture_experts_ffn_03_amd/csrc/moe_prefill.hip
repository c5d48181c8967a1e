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
//   BROWS weight rows. Each wave owns RB 32-row blocks and four 32-column blocks of
//   weight rows (gate+up: two of gate and the same two of up, so SwiGLU runs in the
//   epilogue on values held by the same lane), i.e. 4*RB independent accumulators.
// * Both operands reach LDS by direct-to-LDS loads (global_load_lds_*: the activation
//   rows gathered by row_token, the FP4 weight rows and their scale bytes) into a ring
//   of three 128-wide K stages. Step c waits for stage c, synchronises the block once,
//   issues stage c+2 into the slot freed by step c-1, then runs the MFMAs of stage c.
//   Loads therefore have two steps to land, and no registers are spent on them.
// * The loads and their waits are explicit: the compiler's counter tracking cannot tell
//   a direct-to-LDS load apart from the LDS reads of other stages and would drain every
//   load before each read. No other vector-memory load is issued in the main loop, so
//   "at most one stage of loads in flight" means "this step's stage has landed".
// * LDS rows are swizzled in 16-byte slots (A: slot = piece ^ (row & 15); B: slot =
//   piece ^ ((row >> 1 ^ row >> 3) & 3)) so that the rows read by one MFMA operand load
//   fall in distinct banks; the load side picks the source piece for its fixed slot.
// * The MFMA K order is permuted inside a stage (lane half h covers codes 64h..64h+63),
//   so each lane's B codes are 32 contiguous bytes of one weight row; A is read with the
//   same permutation.
// * E2M1 codes become exact bf16 operands in registers (MXFP4: scaled convert by the
//   E8M0 power of two; NVFP4: convert, times the E4M3 scale in fp32, pack).
// * Block ids are remapped so that each XCD (ids dispatched round-robin over the 8
//   XCDs) walks a contiguous run of (row tile, column tile) work, which keeps an A
//   tile and an expert's weight rows in that XCD's L2 while they are reused.
#include <type_traits>

#include "moe_device.h"

namespace moe {

constexpr int kKc = 128;  // K codes per stage
constexpr int kStages = 3;
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint32_t (&d)[4]) {
  uint4 v = make_uint4(d[0], d[1], d[2], d[3]);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// Direct-to-LDS loads: every lane reads SIZE bytes at its own global address; the wave
// writes them to LDS at m0 + lane * SIZE (m0 = the wave-uniform base). Their wait is
// issued by hand (wait_stage).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}

// Wait until at most N vector-memory loads of this wave are in flight and its LDS reads
// have returned, then synchronise the block: every wave's loads of the stage have
// landed, and every read of the slot about to be refilled is done.
template <int N>
__device__ __forceinline__ void wait_stage() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

__device__ __forceinline__ int b_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

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

// Operand for MFMA step s (codes 8s..8s+7 of the lane's codes of the stage).
template <int FMT>
__device__ __forceinline__ bf16x8_t b_operand(const uint32_t q, const uint32_t sc_word, int s) {
  const int blk = FMT == 0 ? s / 2 : s / 4;  // 16- or 32-code block inside the lane's codes
  const uint32_t sb = (sc_word >> (8 * blk)) & 0xFFu;
  uint32_t d[4];
  mfma_operand_fp4x8<FMT>(q, sb, d);
  return as_bf16x8(d);
}

// Block = 4 waves in a WM x WN grid. Tile height MT = 32 * RB * WM; BROWS weight rows per
// block (gate+up: BROWS/2 gate rows and the same BROWS/2 up rows; down: BROWS output
// columns). A stage holds the A tile (MT rows x 256 bytes) and the B tile (BROWS rows x 64
// bytes). Scales come one of two ways:
// * SS = false: with each stage, BROWS rows x two 4-byte slots (NVFP4 4 bytes each, MXFP4
//   2 bytes each; the 64-code tail uses the first slot). Each row's few bytes are a
//   separate memory request.
// * SS = true (scale rows a multiple of 16 bytes): 16 bytes per row at a time, covering
//   SUPER stages (4 MXFP4, 2 NVFP4), into one of two super-stage slots; a quarter or half
//   as many requests.
template <int FMT, int RB, int WM, int NW, int CB, bool GATEUP, bool SS>
struct PreShape {
  static constexpr int NT = NW * 64;  // threads per block
  static constexpr int WN = NW / WM;
  static constexpr int MT = 32 * RB * WM;
  static constexpr int BROWS = 32 * CB * WN;
  static constexpr int NCOLS = GATEUP ? BROWS / 2 : BROWS;  // output columns per block
  static constexpr int SROW = SS ? 0 : 8;  // LDS bytes per row of scales per stage
  static constexpr int A_BYTES = MT * 256;
  static constexpr int B_BYTES = BROWS * 64;
  static constexpr int S_BYTES = BROWS * SROW;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int NA = MT * 16 / NT;      // 16-byte loads per lane (A)
  static constexpr int NB = BROWS * 4 / NT;    // 16-byte loads per lane (B)
  // scale loads: 4 bytes (NVFP4) or 2 bytes (MXFP4, whose rows may be only 2-aligned) per
  // lane, each landing in a 4-byte LDS slot (sub-dword direct-to-LDS loads keep a 4-byte
  // lane stride)
  static constexpr int SUNIT = FMT == 0 ? 4 : 2;
  static constexpr int NS = S_BYTES / 4 / NT;  // scale loads per lane
  static constexpr int NLOADS = NA + NB + NS;
  static constexpr int SUPER = FMT == 0 ? 2 : 4;              // stages per super-stage
  // super-stage scale loads: one lane per row, issued by the first SS_WAVES waves
  static constexpr int SS_WAVES = SS ? (BROWS / 64 < NW ? BROWS / 64 : NW) : 0;
  static constexpr int NSS = SS ? BROWS / (SS_WAVES * 64) : 0;  // per lane of those waves
  static constexpr int SS_BYTES = SS ? 2 * BROWS * 16 : 0;   // two super-stage slots
  static constexpr size_t SMEM = (size_t)kStages * STAGE + SS_BYTES + MT * sizeof(int);
  static_assert(NA * NT == MT * 16 && NB * NT == BROWS * 4 && NS * NT * 4 == S_BYTES,
                "a stage must split evenly over the block");
  static_assert(!SS || NSS * SS_WAVES * 64 == BROWS, "one super-stage load per row");
  static_assert(CB % 2 == 0 || !GATEUP, "gate+up pairs column blocks");
  static_assert(NLOADS + NSS <= 31, "two stages of loads must fit the wait counter");
  static_assert(SMEM <= 160 * 1024, "three stages must fit the 160 KB of LDS");
};

template <int FMT, int RB, int WM, int NW, int CB, bool GATEUP, bool SS>
__global__ __launch_bounds__(NW * 64) void k_pre_gemm(ExpertGemmArgs a) {
  using Sh = PreShape<FMT, RB, WM, NW, CB, GATEUP, SS>;
  constexpr int NT = Sh::NT;
  constexpr int WN = Sh::WN, BROWS = Sh::BROWS, NCOLS = Sh::NCOLS, MT = Sh::MT;
  constexpr int NA = Sh::NA, NB = Sh::NB, NS = Sh::NS, NSS = Sh::NSS, SUPER = Sh::SUPER;
  extern __shared__ __align__(16) uint8_t s_dyn[];
  uint8_t* s_ss = s_dyn + kStages * Sh::STAGE;  // super-stage scale slots (SS)
  int* s_tok = reinterpret_cast<int*>(s_ss + Sh::SS_BYTES);

  const int N = GATEUP ? a.I : a.H;  // rows of each weight matrix
  const int K = GATEUP ? a.H : a.I;
  const int ncol_tiles = (N + NCOLS - 1) / NCOLS;
  Tile t;
  int ct;
  if (!pre_resolve(a, ncol_tiles, t, ct)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, r = lane & 31;
  const int e = t.group;
  const int n0 = ct * NCOLS;
  const size_t row_bytes = (size_t)K / 2;
  const int sbytes = K / (FMT == 0 ? 16 : 32);
  const WeightDesc& w0 = GATEUP ? a.gate : a.down;
  const WeightDesc& w1 = GATEUP ? a.up : a.down;

  // source row of each A tile row: gathered token (gate+up) or h row (down); rows past
  // the tile's count repeat its first row (results discarded)
  for (int i = threadIdx.x; i < MT; i += NT) {
    const int ii = i < t.count ? i : 0;
    s_tok[i] = GATEUP ? a.row_token[t.row0 + ii] : t.row0 + ii;
  }
  __syncthreads();

  // Source address of each load of this lane (fixed across stages, + the stage's K
  // offset). The i-th load of a wave fills LDS slots (wave * n + i) * 64 + lane of its
  // region; a slot holds the source piece that the swizzle assigns to it.
  const uint16_t* asrc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int slot = (wave * NA + i) * 64 + lane;
    const int row = slot >> 4, piece = (slot & 15) ^ (row & 15);
    const uint16_t* base = GATEUP ? a.x + (size_t)s_tok[row] * a.H
                                  : a.h + (size_t)s_tok[row] * a.h_stride;
    asrc[i] = base + piece * 8;
  }
  // weight row of B-tile row brow; rows past N read row 0 of the expert (not stored)
  auto wrow = [&](int brow, const WeightDesc*& w) -> size_t {
    int n;
    if (GATEUP) {
      w = brow < BROWS / 2 ? &w0 : &w1;
      n = n0 + (brow < BROWS / 2 ? brow : brow - BROWS / 2);
    } else {
      w = &w0;
      n = n0 + brow;
    }
    return (size_t)e * N + (n < N ? n : 0);
  };
  const uint8_t* bsrc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int slot = (wave * NB + i) * 64 + lane;
    const int brow = slot >> 2, piece = (slot & 3) ^ b_swz(brow);
    const WeightDesc* w;
    const size_t rw = wrow(brow, w);
    bsrc[i] = w->packed + rw * row_bytes + piece * 16;
  }
  const uint8_t* ssrc[NS > 0 ? NS : 1];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int slot = (wave * NS + i) * 64 + lane;  // 4-byte LDS slots, two per row
    const WeightDesc* w;
    const size_t rw = wrow(slot >> 1, w);
    ssrc[i] = w->scales + rw * sbytes + (slot & 1) * Sh::SUNIT;
  }

  const uint8_t* sssrc[NSS > 0 ? NSS : 1];
#pragma unroll
  for (int i = 0; i < NSS; ++i) {
    const WeightDesc* w;
    const int row = (wave * NSS + i) * 64 + lane;  // one lane per row (waves < SS_WAVES)
    const size_t rw = wrow(row < BROWS ? row : 0, w);
    sssrc[i] = w->scales + rw * sbytes;
  }

  const int nfull = K / kKc;
  const int nch = nfull + (K % kKc ? 1 : 0);  // the last stage may be a 64-code tail

  // Loads of stage c: always NLOADS per lane, so the wait count is a constant. In the
  // 64-code tail, pieces past K re-read pieces below K (their slots are not read).
  auto issue = [&](int c) {
    const uint32_t abase = lds_addr(s_dyn + (c % kStages) * Sh::STAGE);
    const uint32_t bbase = abase + Sh::A_BYTES, sbase = bbase + Sh::B_BYTES;
    const int k0 = c * kKc;
    const bool tail = c == nfull;
    if (SS && c % SUPER == 0 && wave < Sh::SS_WAVES) {
      const int j = c / SUPER;
      const uint32_t ssbase = lds_addr(s_ss + (j & 1) * BROWS * 16);
#pragma unroll
      for (int i = 0; i < NSS; ++i) {
        const int slot0 = (wave * NSS + i) * 64;
        dma16(sssrc[i] + 16 * j, __builtin_amdgcn_readfirstlane(ssbase + slot0 * 16));
      }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int slot0 = (wave * NA + i) * 64, slot = slot0 + lane, row = slot >> 4;
      const int piece = (slot & 15) ^ (row & 15);
      dma16(asrc[i] + k0 - (tail ? (piece & 8) * 8 : 0),
            __builtin_amdgcn_readfirstlane(abase + slot0 * 16));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot0 = (wave * NB + i) * 64, slot = slot0 + lane;
      const int piece = (slot & 3) ^ b_swz(slot >> 2);
      dma16(bsrc[i] + k0 / 2 - (tail ? (piece & 2) * 16 : 0),
            __builtin_amdgcn_readfirstlane(bbase + slot0 * 16));
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      // a row's second half re-reads its first in the tail (half as many scale bytes)
      const int slot0 = (wave * NS + i) * 64;
      const int back = tail ? ((slot0 + lane) & 1) * Sh::SUNIT : 0;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + slot0 * 4);
      if (FMT == 0) {
        dma4(ssrc[i] + k0 / 16 - back, dst);
      } else {
        dma2(ssrc[i] + k0 / 32 - back, dst);
      }
    }
  };

  f32x16_t acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16_t{};

  // B-tile rows of this wave's column blocks
  // (gate+up: column blocks 0..CB/2-1 are gate rows, CB/2.. the same rows of up)
  constexpr int CH = GATEUP ? CB / 2 : CB;
  int brow0[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    brow0[cb] = GATEUP ? (cb / CH) * (BROWS / 2) + wn * CH * 32 + (cb % CH) * 32
                       : wn * CB * 32 + cb * 32;
  }
  const int arow = wm * 32 * RB + r;  // + rb * 32
  const int bsw = b_swz(r);            // = b_swz(brow0[cb] + r): brow0 is a multiple of 32

  // row blocks of this wave that hold rows of the tile: a partly filled tile skips the
  // MFMAs of its empty 32-row blocks (the other waves of the same SIMD then run alone)
  int nrb = (t.count - wm * 32 * RB + 31) / 32;
  nrb = nrb < 0 ? 0 : (nrb > RB ? RB : nrb);

  // MFMAs of one stage for the first NR row blocks (STEPS = 8, or 4 in the 64-code tail
  // where lane half h covers codes 32h..32h+31)
  auto stage_mma = [&](auto nr_c, auto steps_c, int c) {
    constexpr int NR = decltype(nr_c)::value, STEPS = decltype(steps_c)::value;
    if constexpr (NR == 0) return;
    const bool tail = STEPS == 4;
    const uint8_t* sa = s_dyn + (c % kStages) * Sh::STAGE;
    const uint8_t* sbq = sa + Sh::A_BYTES;
    const uint8_t* ssc = sbq + Sh::B_BYTES;
    uint32_t q[CB][8], sc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int srow = brow0[cb] + r;
      const uint8_t* row = sbq + srow * 64;
      if (tail) {
        const uint4 v0 = *reinterpret_cast<const uint4*>(row + ((half ^ bsw) << 4));
        q[cb][0] = v0.x; q[cb][1] = v0.y; q[cb][2] = v0.z; q[cb][3] = v0.w;
        q[cb][4] = q[cb][5] = q[cb][6] = q[cb][7] = 0;
        sc[cb] = FMT == 0 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ssc + srow * 8 + 2 * half)
                          : (uint32_t)ssc[srow * 8 + half];
        continue;
      }
      const uint4 v0 = *reinterpret_cast<const uint4*>(row + (((2 * half) ^ bsw) << 4));
      const uint4 v1 = *reinterpret_cast<const uint4*>(row + (((2 * half + 1) ^ bsw) << 4));
      q[cb][0] = v0.x; q[cb][1] = v0.y; q[cb][2] = v0.z; q[cb][3] = v0.w;
      q[cb][4] = v1.x; q[cb][5] = v1.y; q[cb][6] = v1.z; q[cb][7] = v1.w;
      if (SS) {
        const uint8_t* sp = s_ss + ((c / SUPER) & 1) * BROWS * 16 + srow * 16;
        sc[cb] = FMT == 0 ? *reinterpret_cast<const uint32_t*>(sp + (c & 1) * 8 + 4 * half)
                          : (uint32_t)*reinterpret_cast<const uint16_t*>(sp + (c & 3) * 4 + 2 * half);
      } else {
        sc[cb] = FMT == 0 ? *reinterpret_cast<const uint32_t*>(ssc + srow * 8 + 4 * half)
                          : (uint32_t)*reinterpret_cast<const uint16_t*>(ssc + srow * 8 + 4 * half);
      }
    }
    // every A operand of the stage is read up front, in the order of use, so that LDS
    // latency overlaps the MFMAs instead of stalling each step (LDS reads return in order)
    uint4 av[NR > 0 ? NR : 1][STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        const int row = arow + rb * 32;
        const int piece = tail ? 4 * half + s : 8 * half + s;
        av[rb][s] = *reinterpret_cast<const uint4*>(sa + row * 256 + ((piece ^ (row & 15)) << 4));
        __builtin_amdgcn_sched_barrier(0);  // keep the reads in the order they are used
      }
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      bf16x8_t bo[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) bo[cb] = b_operand<FMT>(q[cb][s], sc[cb], s);
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av[rb][s]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bo[cb], acc[rb][cb], 0, 0, 0);
      }
    }
  };
  issue(0);
  if (nch > 1) issue(1);
  // full stages, then the 64-code tail stage (if any) after the loop, so that the
  // accumulators have a single definition inside the loop
  auto kloop = [&](auto nr_c) {
#pragma unroll 1
    for (int c = 0; c < nfull; ++c) {
      // in flight: the loads of stage c+1 (with a super-stage of scales if it starts one)
      if (c + 1 >= nch) {
        wait_stage<0>();
      } else if (SS && (c + 1) % SUPER == 0 && wave < Sh::SS_WAVES) {
        wait_stage<Sh::NLOADS + NSS>();
      } else {
        wait_stage<Sh::NLOADS>();
      }
      if (c + 2 < nch) issue(c + 2);
      stage_mma(nr_c, std::integral_constant<int, 8>{}, c);
    }
    if (nch > nfull) {
      wait_stage<0>();
      stage_mma(nr_c, std::integral_constant<int, 4>{}, nfull);
    }
  };
  if (nrb >= RB) {
    kloop(std::integral_constant<int, RB>{});
  } else if (nrb == 1) {
    kloop(std::integral_constant<int, 1>{});
  } else {
    kloop(std::integral_constant<int, 0>{});
  }

  // epilogue: lane holds column j = lane % 32 of each 32x32 block, rows 8*(v/4)+4*half+v%4
  if (GATEUP) {
    const float gs_g = FMT == 0 ? a.gate.global[e] : 1.0f;
    const float gs_u = FMT == 0 ? a.up.global[e] : 1.0f;
#pragma unroll
    for (int cg = 0; cg < CH; ++cg) {
      const int n = n0 + wn * CH * 32 + cg * 32 + r;
      if (n >= N) continue;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = wm * 32 * RB + rb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (i < t.count) {
            const float g = acc[rb][cg][v] * gs_g;
            const float u = acc[rb][CH + cg][v] * gs_u;
            const float hval = silu(g) * u;
            a.h[(size_t)(t.row0 + i) * a.h_stride + n] = f32_to_bf16(hval);
          }
        }
      }
    }
  } else {
    const float gs = FMT == 0 ? a.down.global[e] : 1.0f;
    uint16_t* y = reinterpret_cast<uint16_t*>(a.y);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = n0 + wn * CB * 32 + cb * 32 + r;
      if (n >= N) continue;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = wm * 32 * RB + rb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (i < t.count) y[(size_t)(t.row0 + i) * a.H + n] = f32_to_bf16(acc[rb][cb][v] * gs);
        }
      }
    }
  }
}

template <int FMT, int RB, int WM, int NW, int CB, bool GATEUP, bool SS>
static hipError_t launch_pre_ss(const ExpertGemmArgs& a, hipStream_t s) {
  using Sh = PreShape<FMT, RB, WM, NW, CB, GATEUP, SS>;
  const int N = GATEUP ? a.I : a.H;
  const int ncol = (N + Sh::NCOLS - 1) / Sh::NCOLS;
  auto kern = k_pre_gemm<FMT, RB, WM, NW, CB, GATEUP, SS>;
  static bool attr_set = false;  // one attribute call per instantiation and process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Sh::SMEM);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(ncol, a.tile_bound), dim3(Sh::NT), Sh::SMEM, s, a);
  return hipGetLastError();
}

// Super-staged scales when each scale row is a whole number of 16-byte pieces.
template <int FMT, int RB, int WM, int NW, int CB, bool GATEUP>
static hipError_t launch_pre_shape(const ExpertGemmArgs& a, hipStream_t s) {
  const int K = GATEUP ? a.H : a.I;
  const int sbytes = K / (FMT == 0 ? 16 : 32);
  if (sbytes % 16 == 0) return launch_pre_ss<FMT, RB, WM, NW, CB, GATEUP, true>(a, s);
  return launch_pre_ss<FMT, RB, WM, NW, CB, GATEUP, false>(a, s);
}

// Tile height MT -> block shape (row blocks per wave RB, waves along M WM, waves NW,
// column blocks per wave CB): 128 = RB 2 x WM 2 with 8 waves of 2 column blocks (two waves
// per SIMD), 64 = 1 x 2 (4 waves of 4), 32 = 1 x 1 (4 waves of 4).
#ifndef MOE_PRE_NW128
#define MOE_PRE_NW128 8
#endif
template <bool GATEUP>
static hipError_t launch_pre(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  const int fmt = GATEUP ? a.gate.fmt : a.down.fmt;
  constexpr int NW = MOE_PRE_NW128, CB = 16 / NW;
  if (fmt == 0) {
    if (mt == 32) return launch_pre_shape<0, 1, 1, 4, 4, GATEUP>(a, s);
    if (mt == 64) return launch_pre_shape<0, 1, 2, 4, 4, GATEUP>(a, s);
    return launch_pre_shape<0, 2, 2, NW, CB, GATEUP>(a, s);
  }
  if (mt == 32) return launch_pre_shape<1, 1, 1, 4, 4, GATEUP>(a, s);
  if (mt == 64) return launch_pre_shape<1, 1, 2, 4, 4, GATEUP>(a, s);
  return launch_pre_shape<1, 2, 2, NW, CB, GATEUP>(a, s);
}

hipError_t launch_prefill_gate_up(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<true>(a, mt, s);
}

hipError_t launch_prefill_down(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<false>(a, mt, s);
}

}  // namespace moe
