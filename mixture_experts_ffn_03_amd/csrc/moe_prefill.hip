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
// * A block of 8 waves computes an MT-row tile of one expert: MT gathered token rows times
//   COLS weight rows (gate+up kernel: COLS gate rows and the same COLS up rows, so SwiGLU
//   runs in the epilogue on values that sit in the same lane and register). Waves form a
//   WM x WN grid; each owns 32*RB rows and two 32-column blocks (64 fp32 accumulators
//   per lane for RB = 2), which keeps 2 waves per SIMD resident.
// * The waves share the A tile, gathered from the activations by row_token and staged in
//   LDS (rows padded by 16 bytes so the 32 rows an MFMA operand reads fall in distinct
//   banks), double-buffered so that each 128-wide K chunk needs a single barrier.
// * Each lane reads its B fragment straight from HBM: 32 contiguous bytes (64 codes) of
//   one weight row per 128-wide K chunk, so the weight stream needs no LDS. The MFMA K
//   order is permuted inside a chunk (lane half h covers codes 64h..64h+63) and the A
//   fragments are read from LDS with the same permutation.
// * E2M1 codes become exact bf16 operands in registers (MXFP4: scaled convert by the
//   E8M0 power of two; NVFP4: convert, times the E4M3 scale in fp32, pack).
// * Global loads (A and B) for chunk c+1 are issued before the MFMAs of chunk c.
// * Block ids are remapped so that each XCD (ids dispatched round-robin over the 8
//   XCDs) walks a contiguous run of (row tile, column tile) work, which keeps an A
//   tile and an expert's weight rows in that XCD's L2 while they are reused.
#include "moe_device.h"

namespace moe {

constexpr int kKc = 128;           // K per chunk
constexpr int kLdsRow = kKc * 2 + 16;  // bytes per LDS row of the A tile (padded)
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint32_t (&d)[4]) {
  uint4 v = make_uint4(d[0], d[1], d[2], d[3]);
  return __builtin_bit_cast(bf16x8_t, v);
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

// B fragment of one 32-row column block for a chunk of KCH (128 or 64) codes: lane
// (row j = lane % 32, half h = lane / 32) holds codes [KCH/2 * h, KCH/2 * (h + 1)) of
// the chunk, i.e. KCH/16 dwords, plus their scale bytes.
template <int FMT, int KCH>
struct BFrag {
  uint32_t q[KCH / 16];
  uint32_t sc;
};

// Loads are unconditional: callers clamp rows and chunks to valid addresses (results for
// clamped rows are discarded), so the compiler can count outstanding loads and wait only
// for the ones a step consumes.
template <int FMT, int KCH>
__device__ __forceinline__ void load_b(const uint8_t* packed_row, const uint8_t* scale_row,
                                       int k0, int half, BFrag<FMT, KCH>& f) {
  const uint8_t* p = packed_row + k0 / 2 + half * (KCH / 4);
#pragma unroll
  for (int i = 0; i < KCH / 64; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[i];
    f.q[4 * i + 0] = v.x;
    f.q[4 * i + 1] = v.y;
    f.q[4 * i + 2] = v.z;
    f.q[4 * i + 3] = v.w;
  }
  // scale bytes of the lane's KCH/2 codes: NVFP4 KCH/32 bytes, MXFP4 KCH/64 bytes
  if (FMT == 0) {
    const uint8_t* s = scale_row + k0 / 16 + half * (KCH / 32);
    f.sc = KCH == 128 ? *reinterpret_cast<const uint32_t*>(s)
                      : (uint32_t)*reinterpret_cast<const uint16_t*>(s);
  } else {
    const uint8_t* s = scale_row + k0 / 32 + half * (KCH / 64);
    f.sc = KCH == 128 ? (uint32_t)*reinterpret_cast<const uint16_t*>(s) : (uint32_t)s[0];
  }
}

// Operand for MFMA step s (codes 8s..8s+7 of the lane's half chunk).
template <int FMT>
__device__ __forceinline__ bf16x8_t b_operand(const uint32_t q, const uint32_t sc_word, int s) {
  const int blk = FMT == 0 ? s / 2 : s / 4;  // 16- or 32-code block inside the lane's codes
  const uint32_t sb = (sc_word >> (8 * blk)) & 0xFFu;
  uint32_t d[4];
  mfma_operand_fp4x8<FMT>(q, sb, d);
  return as_bf16x8(d);
}

// Gathered A rows of one chunk -> registers (16-byte pieces spread over the NT threads of
// the block), then -> LDS.
template <int MT, int KCH, int NT>
struct AStage {
  static constexpr int kPieces = MT * (KCH / 8);
  static constexpr int kPerThread = (kPieces + NT - 1) / NT;
  // one vector value (not an array of structs) so it stays in registers across the loop
  typedef uint32_t vec_t __attribute__((ext_vector_type(4 * kPerThread)));
  vec_t v;
};

// Source rows of this thread's A pieces (fixed across chunks): gathered activation rows
// (gate+up) or the expert's h rows (down); rows past the tile's count read row 0.
template <int MT, int KCH, int NT, bool GATEUP>
__device__ __forceinline__ void a_rows(const ExpertGemmArgs& a, const Tile& t, const int* s_tok,
                                       const uint16_t* (&src)[AStage<MT, KCH, NT>::kPerThread]) {
  constexpr int kRowPieces = KCH / 8;
#pragma unroll
  for (int i = 0; i < AStage<MT, KCH, NT>::kPerThread; ++i) {
    const int p = (threadIdx.x + NT * i) % AStage<MT, KCH, NT>::kPieces;  // spare threads repeat
    int row = p / kRowPieces;
    row = row < t.count ? row : 0;
    src[i] = GATEUP ? a.x + (size_t)s_tok[row] * a.H : a.h + (size_t)(t.row0 + row) * a.h_stride;
    src[i] += (p % kRowPieces) * 8;
  }
}

template <int MT, int KCH, int NT>
__device__ __forceinline__ void load_a(const uint16_t* const (&src)[AStage<MT, KCH, NT>::kPerThread],
                                       int k0, AStage<MT, KCH, NT>& st) {
#pragma unroll
  for (int i = 0; i < AStage<MT, KCH, NT>::kPerThread; ++i) {
    const uint4 x = *reinterpret_cast<const uint4*>(src[i] + k0);
    st.v[4 * i + 0] = x.x;
    st.v[4 * i + 1] = x.y;
    st.v[4 * i + 2] = x.z;
    st.v[4 * i + 3] = x.w;
  }
}

template <int MT, int KCH, int NT>
__device__ __forceinline__ void store_a(uint8_t* s_a, const AStage<MT, KCH, NT>& st) {
  constexpr int kRowPieces = KCH / 8;
#pragma unroll
  for (int i = 0; i < AStage<MT, KCH, NT>::kPerThread; ++i) {
    const int p = threadIdx.x + NT * i;
    if (AStage<MT, KCH, NT>::kPieces % NT == 0 || p < AStage<MT, KCH, NT>::kPieces) {
      const int row = p / kRowPieces, c = p % kRowPieces;
      *reinterpret_cast<uint4*>(s_a + row * kLdsRow + c * 16) =
          make_uint4(st.v[4 * i], st.v[4 * i + 1], st.v[4 * i + 2], st.v[4 * i + 3]);
    }
  }
}

// MFMAs of one chunk for one wave: RB row blocks x 2 column blocks x KCH/16 steps.
// s_a points at the wave's first A row in LDS.
template <int FMT, int RB, int KCH>
__device__ __forceinline__ void mma_chunk(const uint8_t* s_a, const BFrag<FMT, KCH> (&bf)[2],
                                          f32x16_t (&acc)[RB][2], int lane) {
  const int half = lane >> 5, r = lane & 31;
#pragma unroll
  for (int s = 0; s < KCH / 16; ++s) {
    const bf16x8_t b0 = b_operand<FMT>(bf[0].q[s], bf[0].sc, s);
    const bf16x8_t b1 = b_operand<FMT>(bf[1].q[s], bf[1].sc, s);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // A[i][k] for the same permuted k: lane half h, step s -> chunk codes KCH/2*h + 8s
      const uint4 av = *reinterpret_cast<const uint4*>(
          s_a + (rb * 32 + r) * kLdsRow + (half * (KCH / 2) + 8 * s) * 2);
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
      acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b0, acc[rb][0], 0, 0, 0);
      acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b1, acc[rb][1], 0, 0, 0);
    }
  }
}

// Block = 8 waves in a WM x WN grid; each wave owns RB 32-row blocks of the tile's rows and
// two 32-column blocks of weight rows (gate+up: the same rows of gate and of up). Tile
// height MT = 32 * RB * WM. The A tile is double-buffered in LDS: chunk c+1 is loaded into
// registers while chunk c's MFMAs run and is written to the other buffer afterwards, so
// each chunk needs one barrier.
constexpr int kPreThreads = 512;
constexpr int kPreWaves = kPreThreads / 64;

template <int FMT, int RB, int WM, bool GATEUP>
struct PreShape {
  static constexpr int WN = kPreWaves / WM;
  static constexpr int MT = 32 * RB * WM;
  static constexpr int COLS = GATEUP ? WN * 32 : WN * 64;  // weight rows per matrix per block
};

template <int FMT, int RB, int WM, bool GATEUP>
__global__ __launch_bounds__(kPreThreads) void k_pre_gemm(ExpertGemmArgs a) {
  using Sh = PreShape<FMT, RB, WM, GATEUP>;
  constexpr int MT = Sh::MT, WN = Sh::WN, COLS = Sh::COLS, NT = kPreThreads;
  extern __shared__ __align__(16) uint8_t s_dyn[];
  uint8_t* s_a0 = s_dyn;
  uint8_t* s_a1 = s_dyn + MT * kLdsRow;
  int* s_tok = reinterpret_cast<int*>(s_dyn + 2 * MT * kLdsRow);

  const int N = GATEUP ? a.I : a.H;   // rows of each weight matrix
  const int K = GATEUP ? a.H : a.I;
  const int ncol_tiles = (N + COLS - 1) / COLS;
  Tile t;
  int ct;
  if (!pre_resolve(a, ncol_tiles, t, ct)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, r = lane & 31;
  const int e = t.group;
  int ncol[2];
  if (GATEUP) {
    ncol[0] = ct * COLS + wn * 32;  // gate rows; column block 1 = the same up rows
    ncol[1] = ncol[0];
  } else {
    ncol[0] = ct * COLS + wn * 64;
    ncol[1] = ncol[0] + 32;
  }
  const bool valid0 = ncol[0] < N, valid1 = ncol[1] < N;
  const size_t row_bytes = (size_t)K / 2;
  const int sbytes = K / (FMT == 0 ? 16 : 32);
  const WeightDesc& w0 = GATEUP ? a.gate : a.down;
  const WeightDesc& w1 = GATEUP ? a.up : a.down;
  // column blocks past N read row r of the expert instead (their results are not stored)
  const size_t r0 = (size_t)e * N + (valid0 ? ncol[0] : 0) + r;
  const size_t r1 = (size_t)e * N + (valid1 ? ncol[1] : 0) + r;
  const uint8_t* p0 = w0.packed + r0 * row_bytes;
  const uint8_t* p1 = w1.packed + r1 * row_bytes;
  const uint8_t* q0 = w0.scales + r0 * sbytes;
  const uint8_t* q1 = w1.scales + r1 * sbytes;
  const int arow0 = wm * 32 * RB;  // first A row of this wave

  if (GATEUP) {
    for (int i = threadIdx.x; i < MT; i += NT) s_tok[i] = i < t.count ? a.row_token[t.row0 + i] : 0;
    __syncthreads();
  }

  f32x16_t acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    acc[rb][0] = f32x16_t{};
    acc[rb][1] = f32x16_t{};
  }

  const int nfull = K / kKc;
  if (nfull > 0) {
    // Pipeline: B fragments rotate through three register slots, A stages through LDS.
    // Step c runs chunk c's MFMAs, writes A(c+1) (already in registers) to the other LDS
    // buffer, then issues the loads of A(c+2) and B(c+3) before the step's barrier. The
    // barrier keeps those loads ahead of the next steps, whose MFMAs hide their latency.
    // Past the last chunk the loads re-read it (unconditional loads, unused data).
    AStage<MT, kKc, NT> st;
    const uint16_t* asrc[AStage<MT, kKc, NT>::kPerThread];
    a_rows<MT, kKc, NT, GATEUP>(a, t, s_tok, asrc);
    const int klast = (nfull - 1) * kKc;
    BFrag<FMT, kKc> b0[2], b1[2], b2[2];
    load_a<MT, kKc, NT>(asrc, 0, st);
    load_b<FMT, kKc>(p0, q0, 0, half, b0[0]);
    load_b<FMT, kKc>(p1, q1, 0, half, b0[1]);
    load_b<FMT, kKc>(p0, q0, min(kKc, klast), half, b1[0]);
    load_b<FMT, kKc>(p1, q1, min(kKc, klast), half, b1[1]);
    load_b<FMT, kKc>(p0, q0, min(2 * kKc, klast), half, b2[0]);
    load_b<FMT, kKc>(p1, q1, min(2 * kKc, klast), half, b2[1]);
    store_a<MT, kKc, NT>(s_a0, st);
    load_a<MT, kKc, NT>(asrc, min(kKc, klast), st);
    __syncthreads();
    // A macro rather than a lambda: a captured register array would be demoted to scratch.
#define MOE_PRE_STEP(C, CUR)                                                               \
  {                                                                                       \
    mma_chunk<FMT, RB, kKc>((((C) & 1) ? s_a1 : s_a0) + arow0 * kLdsRow, CUR, acc, lane); \
    store_a<MT, kKc, NT>(((C) & 1) ? s_a0 : s_a1, st);                                    \
    load_a<MT, kKc, NT>(asrc, min(((C) + 2) * kKc, klast), st);                           \
    const int k3 = min(((C) + 3) * kKc, klast);                                           \
    load_b<FMT, kKc>(p0, q0, k3, half, CUR[0]);                                           \
    load_b<FMT, kKc>(p1, q1, k3, half, CUR[1]);                                           \
    __syncthreads();                                                                      \
  }
    // unrolled by three so the three B slots rotate by renaming, not by register copies
    // (a copy of a slot whose loads are in flight would wait for them)
#pragma unroll 1
    for (int c = 0; c < nfull; c += 3) {
      MOE_PRE_STEP(c, b0);
      if (c + 1 < nfull) MOE_PRE_STEP(c + 1, b1);
      if (c + 2 < nfull) MOE_PRE_STEP(c + 2, b2);
    }
#undef MOE_PRE_STEP
  }
  if (K % kKc) {  // 64-code tail (K % 64 == 0); both buffers are free after the last barrier
    const int k0 = nfull * kKc;
    AStage<MT, 64, NT> st;
    const uint16_t* asrc[AStage<MT, 64, NT>::kPerThread];
    a_rows<MT, 64, NT, GATEUP>(a, t, s_tok, asrc);
    BFrag<FMT, 64> tb[2];
    load_a<MT, 64, NT>(asrc, k0, st);
    load_b<FMT, 64>(p0, q0, k0, half, tb[0]);
    load_b<FMT, 64>(p1, q1, k0, half, tb[1]);
    store_a<MT, 64, NT>(s_a0, st);
    __syncthreads();
    mma_chunk<FMT, RB, 64>(s_a0 + arow0 * kLdsRow, tb, acc, lane);
  }

  // epilogue: lane holds column j = lane % 32 of each 32x32 block, rows 8*(v/4)+4*half+v%4
  if (GATEUP) {
    if (!valid0) return;
    const float gs_g = FMT == 0 ? a.gate.global[e] : 1.0f;
    const float gs_u = FMT == 0 ? a.up.global[e] : 1.0f;
    const int n = ncol[0] + r;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = arow0 + rb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
        if (i < t.count) {
          const float g = acc[rb][0][v] * gs_g;
          const float u = acc[rb][1][v] * gs_u;
          const float hval = g / (1.0f + expf(-g)) * u;
          a.h[(size_t)(t.row0 + i) * a.h_stride + n] = f32_to_bf16(hval);
        }
      }
    }
  } else {
    const float gs = FMT == 0 ? a.down.global[e] : 1.0f;
    uint16_t* y = reinterpret_cast<uint16_t*>(a.y);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (!(cb ? valid1 : valid0)) continue;
      const int n = ncol[cb] + r;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = arow0 + rb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (i < t.count) y[(size_t)(t.row0 + i) * a.H + n] = f32_to_bf16(acc[rb][cb][v] * gs);
        }
      }
    }
  }
}

template <int FMT, int RB, int WM, bool GATEUP>
static hipError_t launch_pre_shape(const ExpertGemmArgs& a, hipStream_t s) {
  using Sh = PreShape<FMT, RB, WM, GATEUP>;
  const int N = GATEUP ? a.I : a.H;
  const int ncol = (N + Sh::COLS - 1) / Sh::COLS;
  const size_t smem = 2 * (size_t)Sh::MT * kLdsRow + Sh::MT * sizeof(int);
  auto kern = k_pre_gemm<FMT, RB, WM, GATEUP>;
  static bool attr_set = false;  // one attribute call per instantiation and process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(ncol, a.tile_bound), dim3(kPreThreads), smem, s, a);
  return hipGetLastError();
}

// Tile height MT -> (row blocks per wave, waves along M): 128 = 2 x 2, 64 = 2 x 1, 32 = 1 x 1.
template <bool GATEUP>
static hipError_t launch_pre(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  const int fmt = GATEUP ? a.gate.fmt : a.down.fmt;
  if (fmt == 0) {
    if (mt == 32) return launch_pre_shape<0, 1, 1, GATEUP>(a, s);
    if (mt == 64) return launch_pre_shape<0, 2, 1, GATEUP>(a, s);
    return launch_pre_shape<0, 2, 2, GATEUP>(a, s);
  }
  if (mt == 32) return launch_pre_shape<1, 1, 1, GATEUP>(a, s);
  if (mt == 64) return launch_pre_shape<1, 2, 1, GATEUP>(a, s);
  return launch_pre_shape<1, 2, 2, GATEUP>(a, s);
}

hipError_t launch_prefill_gate_up(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<true>(a, mt, s);
}

hipError_t launch_prefill_down(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<false>(a, mt, s);
}

}  // namespace moe
