// Decode experts: HBM-streaming GEMV over FP4 weights for few tokens per expert.
//
// MoE module page (spark_model/layers/moe/mod.rs): the module doc's gate+up and
// SiLU+down expert launches and the [N, K/2] packed weight layout with [N, K/16]
// scales ("original" layout, docs of unified_layout / hybrid_layout); the NVFP4 and
// MXFP4 block formats (doc of experts_scale_kind).
//
// Design (gfx950): the grid is (block of output rows, expert tile); one tile is a run of
// at most kDecodeTile tokens routed to one expert, so every weight byte of an active
// expert is streamed from HBM once per tile whatever the batch. Each lane streams 16-byte
// chunks (32 E2M1 codes) of a row with 128-bit loads; a group of LPR lanes covers one row
// and a wave covers several rows, which keeps many independent loads in flight. Codes are decoded in
// registers to exact bf16 with the gfx950 scaled convert (scale 1.0), dotted with the
// bf16 activations by v_dot2_f32_bf16, and each 16- or 32-code block partial is
// multiplied by its fp32 block scale. The scale bytes travel with the codes in the same
// load round trip, and tile records carry their token ids, so a block waits on memory
// twice: for its tile record, then for weights, scales and activations together. Rows
// per pass shrink as tokens per tile grow, keeping register use within 256 VGPRs so that
// 2 waves share each SIMD and hide HBM latency. The per-row sums are reduced across the lane group
// by a transposing butterfly (no LDS), then gate/up pairs are combined into
// SiLU(gate) * up (gate+up kernel) or written as the expert output (down kernel).
#include "moe_device.h"

namespace moe {

constexpr int kGateRowsPerWave = 8;   // gate rows (and as many up rows) per wave
constexpr int kDownRowsPerWave = 16;  // down rows per wave
constexpr int kDecWaves = 4;

__device__ __forceinline__ bool resolve_tile(const TileSource& src, const int32_t* row_token,
                                             int idx, Tile& t) {
  if (src.tiles) {
    if (idx >= src.ntiles[0]) return false;
    t = src.tiles[idx];
    return true;
  }
  const int r0 = idx * src.implicit_height;
  if (r0 >= src.implicit_rows) return false;
  t.group = 0;
  t.row0 = src.implicit_row0 + r0;
  t.count = min(src.implicit_height, src.implicit_rows - r0);
  t.pad = 0;
#pragma unroll
  for (int q = 0; q < kTileTok; ++q) t.tok[q] = q < t.count ? row_token[t.row0 + q] : 0;
  return true;
}

// Scale bytes of one 32-code chunk: NVFP4 two E4M3 codes (16-code blocks), MXFP4 one E8M0.
template <int FMT>
__device__ __forceinline__ uint32_t load_chunk_scales(const uint8_t* row_scales, int c) {
  if (FMT == 0) return *reinterpret_cast<const uint16_t*>(row_scales + 2 * c);
  return row_scales[c];
}

// Dot of one 16-byte chunk (32 codes) with TT activation chunks: codes are decoded to exact
// bf16 (scale 1), dotted by v_dot2_f32_bf16, and each 16- or 32-code block partial is
// multiplied by its fp32 block scale.
template <int FMT, int TT>
__device__ __forceinline__ void chunk_dot(const uint4& w, uint32_t sc,
                                          const uint32_t (&xv)[TT][16], float (&acc)[TT]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  if (FMT == 0) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float part[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) part[t] = 0.f;
#pragma unroll
      for (int d = 2 * blk; d < 2 * blk + 2; ++d) {
        uint32_t b[4];
        fp4x8_to_bf16(wd[d], 1.0f, b);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < TT; ++t) part[t] = dot2_bf16(b[j], xv[t][4 * d + j], part[t]);
      }
      const float s = blk ? e4m3_byte_to_f32<1>(sc) : e4m3_byte_to_f32<0>(sc);
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = fmaf(part[t], s, acc[t]);
    }
  } else {
    float part[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) part[t] = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t b[4];
      fp4x8_to_bf16(wd[d], 1.0f, b);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < TT; ++t) part[t] = dot2_bf16(b[j], xv[t][4 * d + j], part[t]);
    }
    const float s = e8m0_to_f32(sc);
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = fmaf(part[t], s, acc[t]);
  }
}

template <int TT>
__device__ __forceinline__ void load_act_chunk(const uint16_t* base, const int (&row)[TT],
                                               int stride, int c, uint32_t (&xv)[TT][16]) {
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const uint4* p = reinterpret_cast<const uint4*>(base + (size_t)row[t] * stride + c * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = p[q];
      xv[t][4 * q + 0] = v.x;
      xv[t][4 * q + 1] = v.y;
      xv[t][4 * q + 2] = v.z;
      xv[t][4 * q + 3] = v.w;
    }
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Rows per pass: enough for every lane group of the wave to own a row, and few enough
// that weights, activations and sums fit 256 VGPRs (2 waves per SIMD, 8 per CU, each
// with 16 row loads of 16 bytes per lane in flight: about 128 KB per CU).
template <int TT, int LPR, int BASE>
struct RowSet {
  static constexpr int G = kWave / LPR;
  static constexpr int R0 = TT == 4 ? BASE / 2 : BASE;
  static constexpr int R = R0 > G ? R0 : G;
};

// ----------------------------------------------------------------------------- gate+up
template <int FMT, int TT, int LPR>
__device__ __forceinline__ void gate_up_body(const ExpertGemmArgs& a, const Tile& tile) {
  constexpr int G = kWave / LPR;
  constexpr int GR = RowSet<TT, LPR, kGateRowsPerWave>::R;  // gate rows per pass
  constexpr int NI = GR / G;
  constexpr int NV = 2 * NI * TT;
  static_assert(NV <= LPR, "one reduced value per lane expected");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  const int H = a.H, I = a.I;
  const int e = tile.group;
  const int nchunk = H / 32;
  const size_t row_bytes = (size_t)H / 2;
  const int sbytes = H / (FMT == 0 ? 16 : 32);
  const uint8_t* gp = a.gate.packed + (size_t)e * I * row_bytes;
  const uint8_t* upp = a.up.packed + (size_t)e * I * row_bytes;
  const uint8_t* gs = a.gate.scales + (size_t)e * I * sbytes;
  const uint8_t* us = a.up.scales + (size_t)e * I * sbytes;
  const float gsg = FMT == 0 ? a.gate.global[e] : 1.0f;
  const float gsu = FMT == 0 ? a.up.global[e] : 1.0f;

  int row[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) row[t] = tile.tok[t < tile.count ? t : 0];

  const int nwave0 = blockIdx.x * (kDecWaves * kGateRowsPerWave) + wave * kGateRowsPerWave;
#pragma unroll 1
  for (int r0 = 0; r0 < kGateRowsPerWave; r0 += GR) {
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.f;
#pragma unroll 1
    for (int c = sub; c < nchunk; c += LPR) {
      uint4 wv[NI][2];
      uint32_t sv[NI][2];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = nwave0 + r0 + grp + G * i;
        if (n < I) {
          wv[i][0] = *reinterpret_cast<const uint4*>(gp + (size_t)n * row_bytes + c * 16);
          wv[i][1] = *reinterpret_cast<const uint4*>(upp + (size_t)n * row_bytes + c * 16);
          sv[i][0] = load_chunk_scales<FMT>(gs + (size_t)n * sbytes, c);
          sv[i][1] = load_chunk_scales<FMT>(us + (size_t)n * sbytes, c);
        } else {
          wv[i][0] = wv[i][1] = make_uint4(0, 0, 0, 0);
          sv[i][0] = sv[i][1] = 0;
        }
      }
      uint32_t xv[TT][16];
      load_act_chunk<TT>(a.x, row, H, c, xv);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
          float r[TT];
#pragma unroll
          for (int t = 0; t < TT; ++t) r[t] = 0.f;
          chunk_dot<FMT, TT>(wv[i][gu], sv[i][gu], xv, r);
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[((i * TT + t) << 1) | gu] += r[t];
        }
      }
    }
    group_reduce_transpose<NV, LPR>(acc, lane);
    // each lane holds one complete sum; gate/up partners differ in the lane bit of the
    // last halving step, duplicates in the bits below it
    constexpr int kPair = LPR / NV;
    const float other = shfl_xor_f(acc[0], kPair);
    const int idx = reduced_index<NV, LPR>(lane, 0);
    if ((idx & 1) == 0 && (sub & (kPair - 1)) == 0) {
      const int q = idx >> 1, i = q / TT, t = q % TT;
      const int n = nwave0 + r0 + grp + G * i;
      if (t < tile.count && n < I) {
        const float g = acc[0] * gsg, u = other * gsu;
        a.h[(size_t)(tile.row0 + t) * a.h_stride + n] = f32_to_bf16(silu(g) * u);
      }
    }
  }
}

template <int FMT, int LPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_dec_gate_up(ExpertGemmArgs a) {
  Tile tile;
  if (!resolve_tile(a.src, a.row_token, blockIdx.y, tile)) return;
  if (tile.count == 1) gate_up_body<FMT, 1, LPR>(a, tile);
  else if (tile.count == 2) gate_up_body<FMT, 2, LPR>(a, tile);
  else gate_up_body<FMT, 4, LPR>(a, tile);
}

// ----------------------------------------------------------------------------- down
template <int FMT, int TT, int LPR>
__device__ __forceinline__ void down_body(const ExpertGemmArgs& a, const Tile& tile) {
  constexpr int G = kWave / LPR;
  constexpr int DR = RowSet<TT, LPR, kDownRowsPerWave>::R;  // rows per pass
  constexpr int NI = DR / G;
  constexpr int NV = NI * TT;
  static_assert(NV <= LPR, "one reduced value per lane expected");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  const int H = a.H, I = a.I;
  const int e = tile.group;
  const int nchunk = I / 32;
  const size_t row_bytes = (size_t)I / 2;
  const int sbytes = I / (FMT == 0 ? 16 : 32);
  const uint8_t* dp = a.down.packed + (size_t)e * H * row_bytes;
  const uint8_t* ds = a.down.scales + (size_t)e * H * sbytes;
  const float gsd = FMT == 0 ? a.down.global[e] : 1.0f;

  int row[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) row[t] = tile.row0 + (t < tile.count ? t : 0);

  const int nwave0 = blockIdx.x * (kDecWaves * kDownRowsPerWave) + wave * kDownRowsPerWave;
#pragma unroll 1
  for (int r0 = 0; r0 < kDownRowsPerWave; r0 += DR) {
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.f;
#pragma unroll 1
    for (int c = sub; c < nchunk; c += LPR) {
      uint4 wv[NI];
      uint32_t sv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = nwave0 + r0 + grp + G * i;
        if (n < H) {
          wv[i] = *reinterpret_cast<const uint4*>(dp + (size_t)n * row_bytes + c * 16);
          sv[i] = load_chunk_scales<FMT>(ds + (size_t)n * sbytes, c);
        } else {
          wv[i] = make_uint4(0, 0, 0, 0);
          sv[i] = 0;
        }
      }
      uint32_t xv[TT][16];
      load_act_chunk<TT>(a.h, row, a.h_stride, c, xv);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float r[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) r[t] = 0.f;
        chunk_dot<FMT, TT>(wv[i], sv[i], xv, r);
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[i * TT + t] += r[t];
      }
    }
    group_reduce_transpose<NV, LPR>(acc, lane);
    constexpr int kDup = LPR / NV;
    const int idx = reduced_index<NV, LPR>(lane, 0);
    if ((sub & (kDup - 1)) == 0) {
      const int i = idx / TT, t = idx % TT;
      const int n = nwave0 + r0 + grp + G * i;
      if (t < tile.count && n < H)
        reinterpret_cast<float*>(a.y)[(size_t)(tile.row0 + t) * H + n] = acc[0] * gsd;
    }
  }
}

template <int FMT, int LPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_dec_down(ExpertGemmArgs a) {
  Tile tile;
  if (!resolve_tile(a.src, a.row_token, blockIdx.y, tile)) return;
  if (tile.count == 1) down_body<FMT, 1, LPR>(a, tile);
  else if (tile.count == 2) down_body<FMT, 2, LPR>(a, tile);
  else down_body<FMT, 4, LPR>(a, tile);
}

// Lanes per row for a row of `nchunk` 16-byte chunks: the widest group that divides the
// row exactly, else the widest group not wider than the row.
static int pick_lpr(int nchunk) {
  for (int l = 64; l >= 8; l >>= 1)
    if (nchunk % l == 0) return l;
  for (int l = 64; l >= 8; l >>= 1)
    if (l <= nchunk) return l;
  return 8;
}

#define MOE_DISPATCH_LPR(KERNEL, FMT, LPR, GRID, S, A)                                  \
  switch (LPR) {                                                                       \
    case 64: hipLaunchKernelGGL((KERNEL<FMT, 64>), GRID, dim3(256), 0, S, A); break;   \
    case 32: hipLaunchKernelGGL((KERNEL<FMT, 32>), GRID, dim3(256), 0, S, A); break;   \
    case 16: hipLaunchKernelGGL((KERNEL<FMT, 16>), GRID, dim3(256), 0, S, A); break;   \
    default: hipLaunchKernelGGL((KERNEL<FMT, 8>), GRID, dim3(256), 0, S, A); break;    \
  }

hipError_t launch_decode_gate_up(const ExpertGemmArgs& a, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  const int rows = kDecWaves * kGateRowsPerWave;
  const dim3 grid((a.I + rows - 1) / rows, a.tile_bound);
  const int lpr = pick_lpr(a.H / 32);
  if (a.gate.fmt == 0) { MOE_DISPATCH_LPR(k_dec_gate_up, 0, lpr, grid, s, a); }
  else { MOE_DISPATCH_LPR(k_dec_gate_up, 1, lpr, grid, s, a); }
  return hipGetLastError();
}

hipError_t launch_decode_down(const ExpertGemmArgs& a, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  const int rows = kDecWaves * kDownRowsPerWave;
  const dim3 grid((a.H + rows - 1) / rows, a.tile_bound);
  const int lpr = pick_lpr(a.I / 32);
  if (a.down.fmt == 0) { MOE_DISPATCH_LPR(k_dec_down, 0, lpr, grid, s, a); }
  else { MOE_DISPATCH_LPR(k_dec_down, 1, lpr, grid, s, a); }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- debug
// Decode one expert matrix to f32 [n, k] with the device routine of a path:
// path 1 (decode GEMV): E2M1 -> bf16 (scale 1) -> f32, times the fp32 block scale;
// path 2 (MFMA operand): the bf16 operand the grouped GEMM feeds its MFMAs.
// Both then times the NVFP4 global scale (one fp32 rounding).
__global__ void k_debug_dequant(WeightDesc w, int expert, int path, float* out) {
  const int dwords_per_row = w.k / 8;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= w.n * dwords_per_row) return;
  const int row = i / dwords_per_row, d = i % dwords_per_row;
  const size_t rbytes = (size_t)w.k / 2;
  const uint32_t q =
      reinterpret_cast<const uint32_t*>(w.packed + ((size_t)expert * w.n + row) * rbytes)[d];
  const int blk = w.fmt == 0 ? 16 : 32;
  const uint8_t sb = w.scales[((size_t)expert * w.n + row) * (w.k / blk) + (d * 8) / blk];
  const float g = w.fmt == 0 ? w.global[expert] : 1.0f;
  uint32_t b[4];
  float scale_after = 1.0f;
  if (path == 1) {
    fp4x8_to_bf16(q, 1.0f, b);
    scale_after = w.fmt == 0 ? e4m3_to_f32(sb) : e8m0_to_f32(sb);
  } else {
    mfma_operand_fp4x8(w.fmt, q, sb, b);
  }
  float* o = out + (size_t)row * w.k + d * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (bf16_to_f32(b[j] & 0xFFFFu) * scale_after) * g;
    o[2 * j + 1] = (bf16_to_f32(b[j] >> 16) * scale_after) * g;
  }
}

hipError_t launch_debug_dequant(const WeightDesc& w, int expert, int path, float* out,
                                hipStream_t s) {
  const int n = w.n * (w.k / 8);
  hipLaunchKernelGGL(k_debug_dequant, dim3((n + 255) / 256), dim3(256), 0, s, w, expert, path,
                     out);
  return hipGetLastError();
}

}  // namespace moe
