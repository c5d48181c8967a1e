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
// * A block computes an MT x 256 output tile of one expert: MT gathered token rows and
//   256 weight rows (gate+up kernel: 128 gate rows and the same 128 up rows, so SwiGLU
//   runs in the epilogue on values that sit in the same lane and register).
// * The 4 waves split N (64 weight rows each) and share the A tile, which is gathered
//   from the activations by row_token and staged in LDS (rows padded by 16 bytes so the
//   32 rows an MFMA operand reads fall in distinct banks).
// * Each lane reads its B fragment straight from HBM: 32 contiguous bytes (64 codes) of
//   one weight row per 128-wide K chunk, so the weight stream needs no LDS. The MFMA K
//   order is permuted inside a chunk (lane half h covers codes 64h..64h+63) and the A
//   fragments are read from LDS with the same permutation.
// * E2M1 codes become exact bf16 operands in registers (MXFP4: scaled convert by the
//   E8M0 power of two; NVFP4: convert, times the E4M3 scale in fp32, pack).
// * Global loads for chunk c+1 are issued before the MFMAs of chunk c.
// * Block ids are remapped so that each XCD (ids dispatched round-robin over the 8
//   XCDs) walks a contiguous run of (row tile, column tile) work, which keeps an A
//   tile and an expert's weight rows in that XCD's L2 while they are reused.
#include "moe_device.h"

namespace moe {

constexpr int kPreCols = 256;      // weight rows per block tile
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

template <int FMT, int KCH>
__device__ __forceinline__ void load_b(const uint8_t* packed_row, const uint8_t* scale_row,
                                       int k0, int half, bool valid, BFrag<FMT, KCH>& f) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < KCH / 16; ++i) f.q[i] = 0;
    f.sc = 0;
    return;
  }
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

// Gathered A rows of one chunk -> registers (each thread 16-byte pieces), then -> LDS.
template <int MT, int KCH>
struct AStage {
  static constexpr int kPieces = MT * (KCH / 8);                  // 16-byte pieces
  static constexpr int kPerThread = (kPieces + 255) / 256;
  uint4 v[kPerThread];
};

template <int MT, int KCH, bool GATEUP>
__device__ __forceinline__ void load_a(const ExpertGemmArgs& a, const Tile& t, const int* s_tok,
                                       int k0, AStage<MT, KCH>& st) {
  constexpr int kRowPieces = KCH / 8;
#pragma unroll
  for (int i = 0; i < AStage<MT, KCH>::kPerThread; ++i) {
    const int p = threadIdx.x + 256 * i;
    const int row = p / kRowPieces, c = p % kRowPieces;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (p < AStage<MT, KCH>::kPieces && row < t.count) {
      const uint16_t* src = GATEUP ? a.x + (size_t)s_tok[row] * a.H
                                   : a.h + (size_t)(t.row0 + row) * a.h_stride;
      v = *reinterpret_cast<const uint4*>(src + k0 + c * 8);
    }
    st.v[i] = v;
  }
}

template <int MT, int KCH>
__device__ __forceinline__ void store_a(uint8_t* s_a, const AStage<MT, KCH>& st) {
  constexpr int kRowPieces = KCH / 8;
#pragma unroll
  for (int i = 0; i < AStage<MT, KCH>::kPerThread; ++i) {
    const int p = threadIdx.x + 256 * i;
    if (p < AStage<MT, KCH>::kPieces) {
      const int row = p / kRowPieces, c = p % kRowPieces;
      *reinterpret_cast<uint4*>(s_a + row * kLdsRow + c * 16) = st.v[i];
    }
  }
}

// MFMAs of one chunk: RB row blocks x 2 column blocks x KCH/16 steps.
template <int FMT, int MT, int KCH>
__device__ __forceinline__ void mma_chunk(const uint8_t* s_a, const BFrag<FMT, KCH> (&bf)[2],
                                          f32x16_t (&acc)[MT / 32][2], int lane) {
  constexpr int RB = MT / 32;
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

template <int FMT, int MT, bool GATEUP>
__global__ __launch_bounds__(256) void k_pre_gemm(ExpertGemmArgs a) {
  constexpr int RB = MT / 32;
  __shared__ __align__(16) uint8_t s_a[MT * kLdsRow];
  __shared__ int s_tok[MT];

  const int N = GATEUP ? a.I : a.H;   // rows of each weight matrix
  const int K = GATEUP ? a.H : a.I;
  const int ncol_tiles = GATEUP ? (N + 127) / 128 : (N + kPreCols - 1) / kPreCols;
  Tile t;
  int ct;
  if (!pre_resolve(a, ncol_tiles, t, ct)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, r = lane & 31;
  const int e = t.group;
  // this wave's two 32-row column blocks
  int ncol[2];
  if (GATEUP) {
    ncol[0] = ct * 128 + wave * 32;  // gate rows; column block 1 = the same up rows
    ncol[1] = ncol[0];
  } else {
    ncol[0] = ct * kPreCols + wave * 64;
    ncol[1] = ncol[0] + 32;
  }
  const bool valid0 = ncol[0] < N, valid1 = ncol[1] < N;
  const size_t row_bytes = (size_t)K / 2;
  const int sbytes = K / (FMT == 0 ? 16 : 32);
  const WeightDesc& w0 = GATEUP ? a.gate : a.down;
  const WeightDesc& w1 = GATEUP ? a.up : a.down;
  const uint8_t* p0 = w0.packed + ((size_t)e * N + ncol[0] + r) * row_bytes;
  const uint8_t* p1 = w1.packed + ((size_t)e * N + ncol[1] + r) * row_bytes;
  const uint8_t* q0 = w0.scales + ((size_t)e * N + ncol[0] + r) * sbytes;
  const uint8_t* q1 = w1.scales + ((size_t)e * N + ncol[1] + r) * sbytes;

  if (GATEUP) {
    for (int i = threadIdx.x; i < MT; i += 256)
      s_tok[i] = i < t.count ? a.row_token[t.row0 + i] : 0;
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
    AStage<MT, kKc> st;
    BFrag<FMT, kKc> cur[2], nxt[2];
    load_a<MT, kKc, GATEUP>(a, t, s_tok, 0, st);
    load_b<FMT, kKc>(p0, q0, 0, half, valid0, cur[0]);
    load_b<FMT, kKc>(p1, q1, 0, half, valid1, cur[1]);
    for (int c = 0; c < nfull; ++c) {
      store_a<MT, kKc>(s_a, st);
      __syncthreads();
      if (c + 1 < nfull) {
        const int k1 = (c + 1) * kKc;
        load_a<MT, kKc, GATEUP>(a, t, s_tok, k1, st);
        load_b<FMT, kKc>(p0, q0, k1, half, valid0, nxt[0]);
        load_b<FMT, kKc>(p1, q1, k1, half, valid1, nxt[1]);
      }
      mma_chunk<FMT, MT, kKc>(s_a, cur, acc, lane);
      __syncthreads();
      cur[0] = nxt[0];
      cur[1] = nxt[1];
    }
  }
  if (K % kKc) {  // 64-code tail (K % 64 == 0)
    const int k0 = nfull * kKc;
    AStage<MT, 64> st;
    BFrag<FMT, 64> tb[2];
    load_a<MT, 64, GATEUP>(a, t, s_tok, k0, st);
    load_b<FMT, 64>(p0, q0, k0, half, valid0, tb[0]);
    load_b<FMT, 64>(p1, q1, k0, half, valid1, tb[1]);
    store_a<MT, 64>(s_a, st);
    __syncthreads();
    mma_chunk<FMT, MT, 64>(s_a, tb, acc, lane);
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
        const int i = rb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
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
          const int i = rb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (i < t.count) y[(size_t)(t.row0 + i) * a.H + n] = f32_to_bf16(acc[rb][cb][v] * gs);
        }
      }
    }
  }
}

template <bool GATEUP>
static hipError_t launch_pre(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  const int N = GATEUP ? a.I : a.H;
  const int ncol = GATEUP ? (N + 127) / 128 : (N + kPreCols - 1) / kPreCols;
  const dim3 grid(ncol, a.tile_bound), block(256);
  const int fmt = GATEUP ? a.gate.fmt : a.down.fmt;
#define MOE_PRE(F, M) hipLaunchKernelGGL((k_pre_gemm<F, M, GATEUP>), grid, block, 0, s, a)
  if (fmt == 0) {
    if (mt == 32) MOE_PRE(0, 32);
    else if (mt == 64) MOE_PRE(0, 64);
    else MOE_PRE(0, 128);
  } else {
    if (mt == 32) MOE_PRE(1, 32);
    else if (mt == 64) MOE_PRE(1, 64);
    else MOE_PRE(1, 128);
  }
#undef MOE_PRE
  return hipGetLastError();
}

hipError_t launch_prefill_gate_up(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<true>(a, mt, s);
}

hipError_t launch_prefill_down(const ExpertGemmArgs& a, int mt, hipStream_t s) {
  return launch_pre<false>(a, mt, s);
}

}  // namespace moe
