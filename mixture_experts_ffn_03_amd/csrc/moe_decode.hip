// Decode experts: HBM-streaming GEMV over FP4 weights for few tokens per expert.
//
// MoE module page (spark_model/layers/moe/mod.rs): the module doc's gate+up and
// SiLU+down expert launches and the [N, K/2] packed weight layout with [N, K/16]
// scales ("original" layout, docs of unified_layout / hybrid_layout); the NVFP4 and
// MXFP4 block formats (doc of experts_scale_kind).
//
// Design (gfx950): the grid is (block of output rows, expert tile); one tile is a run of
// at most kDecodeTile tokens routed to one expert, so every weight byte of an active
// expert is streamed from HBM once per tile whatever the batch. The tile's activation rows
// are first copied to LDS (bf16), so the streaming loop issues weight loads only. Each
// lane streams 16-byte chunks (32 E2M1 codes) of a row with 128-bit loads; a group of LPR
// lanes covers one row and a wave covers several rows per pass. The loop over (pass,
// chunk) is software-pipelined: the loads of the next step are in flight while the codes
// of the current one are decoded in registers to exact bf16 with the gfx950 scaled
// convert (scale 1.0), dotted with the activations by v_dot2_f32_bf16, and each 16- or
// 32-code block partial is multiplied by its fp32 block scale. The per-row sums of a pass
// are reduced across the lane group by a transposing butterfly (no LDS), then gate/up
// pairs are combined into SiLU(gate) * up (gate+up kernel) or written as the expert
// output (down kernel). Rows per pass shrink as tokens per tile grow, keeping register
// use within 256 VGPRs so that 2 waves share each SIMD; rows per wave (passes) grow when
// the grid would otherwise run several short rounds of blocks.
#include "moe_device.h"
#include "moe_select.h"

namespace moe {

constexpr int kGateRowsPerPass = 8;   // gate rows (and as many up rows) per wave pass
constexpr int kDownRowsPerPass = 16;  // down rows per wave pass
constexpr int kDecWaves = 4;

__device__ __forceinline__ bool resolve_tile(const TileSource& src, int idx, Tile& t) {
  if (src.tiles) {
    // both loads at once: idx is below the list's capacity (the grid's tile bound), so the
    // entry is readable even past the count
    const int n = src.ntiles[0];
    t = src.tiles[idx];
    return idx < n;
  }
  const int r0 = idx * src.implicit_height;
  if (r0 >= src.implicit_rows) return false;
  t.group = 0;
  t.row0 = src.implicit_row0 + r0;
  t.count = min(src.implicit_height, src.implicit_rows - r0);
  t.pad = 0;
#pragma unroll
  for (int q = 0; q < kTileTok; ++q) t.tok[q] = q < t.count ? r0 + q : 0;  // token = row - row0
  return true;
}

// Weights are streamed in 16-byte chunks: 32 FP4 codes, 16 FP8 codes or 8 bf16 values.
template <int FMT>
struct DecFmt {
  static constexpr int CPC = FMT <= 1 ? 32 : (FMT == 2 ? 16 : 8);  // codes per chunk
  static constexpr int XW = CPC / 2;  // activation dwords (bf16 pairs) per chunk
};

// Bytes of one weight row of K codes.
template <int FMT>
__device__ __forceinline__ size_t dec_row_bytes(int K) {
  return FMT <= 1 ? (size_t)K / 2 : (size_t)K * (FMT == 2 ? 1 : 2);
}

// Scale layout: FP4 rows of K/16 (NVFP4) or K/32 (MXFP4) bytes; FP8 one fp32 per 128 x 128
// block, [ceil(N/128), ceil(K/128)] per expert; BF16 none. `stride` is the FP4 row bytes or
// the FP8 block-row length ceil(K/128).
template <int FMT>
__device__ __forceinline__ int dec_scale_stride(int K) {
  return FMT == 0 ? K / 16 : FMT == 1 ? K / 32 : FMT == 2 ? (K + 127) / 128 : 0;
}
template <int FMT>
__device__ __forceinline__ size_t dec_scale_expert_bytes(int N, int K) {
  if (FMT <= 1) return (size_t)N * dec_scale_stride<FMT>(K);
  if (FMT == 2) return (size_t)((N + 127) / 128) * dec_scale_stride<FMT>(K) * 4;
  return 0;
}

// Scale word of chunk c of row n: NVFP4 two E4M3 codes (16-code blocks), MXFP4 one E8M0,
// FP8 the fp32 bits of the row's 128 x 128 block, BF16 nothing.
template <int FMT>
__device__ __forceinline__ uint32_t load_chunk_scales(const uint8_t* base, int n, int stride,
                                                      int c) {
  if (FMT == 0) return *reinterpret_cast<const uint16_t*>(base + (size_t)n * stride + 2 * c);
  if (FMT == 1) return base[(size_t)n * stride + c];
  if (FMT == 2)
    return reinterpret_cast<const uint32_t*>(base)[(size_t)(n >> 7) * stride + (c >> 3)];
  return 0u;
}

// Dot of one 16-byte chunk with TT activation chunks. FP4 and FP8 codes are decoded to
// exact bf16 (scale 1), dotted by v_dot2_f32_bf16, and each block partial is multiplied by
// its fp32 block scale (FP4: 16- or 32-code blocks; FP8: the chunk lies in one 128-block);
// bf16 weights are dotted directly.
template <int FMT, int TT>
__device__ __forceinline__ void chunk_dot(const uint4& w, uint32_t sc,
                                          const uint32_t (&xv)[TT][DecFmt<FMT>::XW],
                                          float (&acc)[TT]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  if (FMT == 3) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = dot2_bf16(wd[d], xv[t][d], acc[t]);
  } else if (FMT == 2) {
    float part[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) part[t] = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t b[2];
      fp8x4_to_bf16(wd[d], b);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < TT; ++t) part[t] = dot2_bf16(b[j], xv[t][2 * d + j], part[t]);
    }
    const float s = __uint_as_float(sc);
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = fmaf(part[t], s, acc[t]);
  } else if (FMT == 0) {
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

// Chunk c (2 * XW values) of the TT activation rows staged in LDS ([TT][K] bf16).
template <int TT, int XW>
__device__ __forceinline__ void lds_act_chunk(const uint16_t* s_x, int K, int c,
                                              uint32_t (&xv)[TT][XW]) {
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const uint4* p = reinterpret_cast<const uint4*>(s_x + (size_t)t * K + c * 2 * XW);
#pragma unroll
    for (int q = 0; q < XW / 4; ++q) {
      const uint4 v = p[q];
      xv[t][4 * q + 0] = v.x;
      xv[t][4 * q + 1] = v.y;
      xv[t][4 * q + 2] = v.z;
      xv[t][4 * q + 3] = v.w;
    }
  }
}

// Chunk c (2 * XW values) of the TT activation rows read straight from memory.
template <int TT, int XW>
__device__ __forceinline__ void global_act_chunk(const uint16_t* src, size_t stride,
                                                 const int (&rows)[TT], int c,
                                                 uint32_t (&xv)[TT][XW]) {
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)rows[t] * stride + c * 2 * XW);
#pragma unroll
    for (int q = 0; q < XW / 4; ++q) {
      const uint4 v = p[q];
      xv[t][4 * q + 0] = v.x;
      xv[t][4 * q + 1] = v.y;
      xv[t][4 * q + 2] = v.z;
      xv[t][4 * q + 3] = v.w;
    }
  }
}

// Copy the tile's activation rows (src rows rows[t], t < TT) into LDS [TT][K].
template <int TT>
__device__ __forceinline__ void stage_activations(const uint16_t* src, size_t stride,
                                                  const int (&rows)[TT], int K, uint16_t* s_x) {
  const int pieces = K / 8;  // 16-byte pieces per row
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const uint4* g = reinterpret_cast<const uint4*>(src + (size_t)rows[t] * stride);
    uint4* l = reinterpret_cast<uint4*>(s_x + (size_t)t * K);
    for (int c = threadIdx.x; c < pieces; c += blockDim.x) l[c] = g[c];
  }
  __syncthreads();
}

// Rows per pass: enough for every lane group of the wave to own a row, and few enough
// that two steps of weights, the activations and the sums fit 256 VGPRs (2 waves per SIMD).
template <int TT, int LPR, int BASE>
struct RowSet {
  static constexpr int G = kWave / LPR;
  static constexpr int R0 = TT == 4 ? BASE / 2 : BASE;
  static constexpr int R = R0 > G ? R0 : G;
};

// One pipeline step's weights: NI rows x M matrices (gate+up: 2, down: 1).
template <int NI, int M>
struct WStep {
  uint4 w[NI][M];
  uint32_t s[NI][M];
};

// Weight rows of one pipeline matrix set: packed codes and scales of up to two matrices
// (gate+up: 2, down: 1), passed by value so that nothing lives in memory.
struct WSrc {
  const uint8_t* p0;
  const uint8_t* p1;
  const uint8_t* s0;
  const uint8_t* s1;
};

// Loads of step `it` (pass it / nci, chunk-slot it % nci) of this lane; every address is
// clamped to a valid row and chunk (out-of-range results are discarded).
template <int FMT, int NI, int M, int G, int GR>
__device__ __forceinline__ void load_step(const WSrc src, size_t row_bytes, int sstride,
                                          int n_base, int nmax, int sub, int lpr, int nci,
                                          int nchunk, int it, WStep<NI, M>& st) {
  const int pass = it / nci, ci = it - pass * nci;
  const int c = min(sub + ci * lpr, nchunk - 1);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = min(n_base + pass * GR + G * i, nmax);
    st.w[i][0] = load_weights16(src.p0 + (size_t)n * row_bytes + c * 16);
    st.s[i][0] = load_chunk_scales<FMT>(src.s0, n, sstride, c);
    if (M > 1) {
      st.w[i][M - 1] = load_weights16(src.p1 + (size_t)n * row_bytes + c * 16);
      st.s[i][M - 1] = load_chunk_scales<FMT>(src.s1, n, sstride, c);
    }
  }
}

// ----------------------------------------------------------------------------- gate+up
template <int FMT, int TT, int LPR, bool STAGED>
__device__ __forceinline__ void gate_up_body(const ExpertGemmArgs& a, const Tile& tile, int rpw,
                                             uint16_t* s_x) {
  constexpr int G = kWave / LPR;
  constexpr int GR = RowSet<TT, LPR, kGateRowsPerPass>::R;  // gate rows per pass
  constexpr int NI = GR / G;
  constexpr int NV = 2 * NI * TT;
  static_assert(NV <= LPR, "one reduced value per lane expected");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  const int H = a.H, I = a.I;
  const int e = tile.group;
  constexpr int XW = DecFmt<FMT>::XW;
  const int nchunk = H / DecFmt<FMT>::CPC;
  const size_t row_bytes = dec_row_bytes<FMT>(H);
  const int sstride = dec_scale_stride<FMT>(H);
  const size_t sexp = dec_scale_expert_bytes<FMT>(I, H);
  const WSrc src{a.gate.packed + (size_t)e * I * row_bytes, a.up.packed + (size_t)e * I * row_bytes,
                 a.gate.scales + e * sexp, a.up.scales + e * sexp};
  const float gsg = FMT == 0 ? a.gate.global[e] : 1.0f;
  const float gsu = FMT == 0 ? a.up.global[e] : 1.0f;

  const int nwave0 = blockIdx.x * (kDecWaves * rpw) + wave * rpw;
  const int nci = (nchunk + LPR - 1) / LPR;
  const int total = (rpw / GR) * nci;
  // the first weights are requested before the activations are staged (two round trips
  // in parallel instead of in sequence)
  WStep<NI, 2> s0, s1;
  const int nbase = nwave0 + grp;
  load_step<FMT, NI, 2, G, GR>(src, row_bytes, sstride, nbase, I - 1, sub, LPR, nci, nchunk, 0, s0);
  int rows[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) rows[t] = t < tile.count ? tile.tok[t] : tile.tok[0];
  // (a single step per wave has nothing to overlap: it reads the activations directly)
  if (STAGED) stage_activations<TT>(a.x, (size_t)H, rows, H, s_x);
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.f;

  // consume step it: dot products, and at the end of a pass the reduction and the store
  auto consume = [&](int it, const WStep<NI, 2>& st) {
    const int pass = it / nci, ci = it - pass * nci;
    const int c = sub + ci * LPR;
    if (c < nchunk) {
      uint32_t xv[TT][XW];
      if (STAGED) lds_act_chunk<TT, XW>(s_x, H, c, xv);
      else global_act_chunk<TT, XW>(a.x, (size_t)H, rows, c, xv);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
          float r[TT];
#pragma unroll
          for (int t = 0; t < TT; ++t) r[t] = 0.f;
          chunk_dot<FMT, TT>(st.w[i][gu], st.s[i][gu], xv, r);
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[((i * TT + t) << 1) | gu] += r[t];
        }
      }
    }
    if (ci == nci - 1) {
      group_reduce_transpose<NV, LPR>(acc, lane);
      // each lane holds one complete sum; gate/up partners differ in the lane bit of the
      // last halving step, duplicates in the bits below it
      constexpr int kPair = LPR / NV;
      const float other = shfl_xor_f(acc[0], kPair);
      const int idx = reduced_index<NV, LPR>(lane, 0);
      if ((idx & 1) == 0 && (sub & (kPair - 1)) == 0) {
        const int q = idx >> 1, i = q / TT, t = q % TT;
        const int n = nwave0 + pass * GR + grp + G * i;
        if (t < tile.count && n < I) {
          const float g = acc[0] * gsg, u = other * gsu;
          a.h[(size_t)(tile.row0 + t) * a.h_stride + n] = f32_to_bf16(silu(g) * u);
        }
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.f;
    }
  };

  if (!STAGED) {  // one step
    consume(0, s0);
    return;
  }
  // two register sets renamed by a 2-step unroll (a copy of a set in flight would wait)
#pragma unroll 1
  for (int it = 0; it < total; it += 2) {
    load_step<FMT, NI, 2, G, GR>(src, row_bytes, sstride, nbase, I - 1, sub, LPR, nci, nchunk,
                                 min(it + 1, total - 1), s1);
    consume(it, s0);
    if (it + 1 >= total) break;
    load_step<FMT, NI, 2, G, GR>(src, row_bytes, sstride, nbase, I - 1, sub, LPR, nci, nchunk,
                                 min(it + 2, total - 1), s0);
    consume(it + 1, s1);
  }
}

template <int FMT, int LPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_dec_gate_up(ExpertGemmArgs a, int rpw) {
  extern __shared__ __align__(16) uint16_t s_x[];
  Tile tile;
  if (!resolve_tile(a.src, blockIdx.y, tile)) return;
  if (blockIdx.x * kDecWaves * rpw >= a.I) return;
  // one step per wave (one pass, one chunk per lane and row): no staging, no pipeline
  const bool one = rpw == kGateRowsPerPass && a.H / DecFmt<FMT>::CPC <= LPR;
  if (tile.count == 1) {
    if (one) gate_up_body<FMT, 1, LPR, false>(a, tile, rpw, s_x);
    else gate_up_body<FMT, 1, LPR, true>(a, tile, rpw, s_x);
  } else if (tile.count == 2) {
    if (one) gate_up_body<FMT, 2, LPR, false>(a, tile, rpw, s_x);
    else gate_up_body<FMT, 2, LPR, true>(a, tile, rpw, s_x);
  } else {
    // four tokens halve the rows per pass: two steps, pipelined
    gate_up_body<FMT, 4, LPR, true>(a, tile, rpw, s_x);
  }
}

// ----------------------------------------------------------------------------- down
template <int FMT, int TT, int LPR, bool STAGED>
__device__ __forceinline__ void down_body(const ExpertGemmArgs& a, const Tile& tile, int rpw,
                                          uint16_t* s_x) {
  constexpr int G = kWave / LPR;
  constexpr int DR = RowSet<TT, LPR, kDownRowsPerPass>::R;  // rows per pass
  constexpr int NI = DR / G;
  constexpr int NV = NI * TT;
  static_assert(NV <= LPR, "one reduced value per lane expected");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  const int H = a.H, I = a.I;
  const int e = tile.group;
  constexpr int XW = DecFmt<FMT>::XW;
  const int nchunk = I / DecFmt<FMT>::CPC;
  const size_t row_bytes = dec_row_bytes<FMT>(I);
  const int sstride = dec_scale_stride<FMT>(I);
  const WSrc src{a.down.packed + (size_t)e * H * row_bytes, nullptr,
                 a.down.scales + e * dec_scale_expert_bytes<FMT>(H, I), nullptr};
  const float gsd = FMT == 0 ? a.down.global[e] : 1.0f;

  const int nwave0 = blockIdx.x * (kDecWaves * rpw) + wave * rpw;
  const int nci = (nchunk + LPR - 1) / LPR;
  const int total = (rpw / DR) * nci;
  WStep<NI, 1> s0, s1;
  const int nbase = nwave0 + grp;
  load_step<FMT, NI, 1, G, DR>(src, row_bytes, sstride, nbase, H - 1, sub, LPR, nci, nchunk, 0, s0);
  int rows[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) rows[t] = tile.row0 + (t < tile.count ? t : 0);
  if (STAGED) stage_activations<TT>(a.h, (size_t)a.h_stride, rows, I, s_x);
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.f;

  auto consume = [&](int it, const WStep<NI, 1>& st) {
    const int pass = it / nci, ci = it - pass * nci;
    const int c = sub + ci * LPR;
    if (c < nchunk) {
      uint32_t xv[TT][XW];
      if (STAGED) lds_act_chunk<TT, XW>(s_x, I, c, xv);
      else global_act_chunk<TT, XW>(a.h, (size_t)a.h_stride, rows, c, xv);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float r[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) r[t] = 0.f;
        chunk_dot<FMT, TT>(st.w[i][0], st.s[i][0], xv, r);
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[i * TT + t] += r[t];
      }
    }
    if (ci == nci - 1) {
      group_reduce_transpose<NV, LPR>(acc, lane);
      constexpr int kDup = LPR / NV;
      const int idx = reduced_index<NV, LPR>(lane, 0);
      if ((sub & (kDup - 1)) == 0) {
        const int i = idx / TT, t = idx % TT;
        const int n = nwave0 + pass * DR + grp + G * i;
        if (t < tile.count && n < H)
          reinterpret_cast<float*>(a.y)[(size_t)(tile.row0 + t) * H + n] = acc[0] * gsd;
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.f;
    }
  };

  if (!STAGED) {  // one step
    consume(0, s0);
    return;
  }
#pragma unroll 1
  for (int it = 0; it < total; it += 2) {
    load_step<FMT, NI, 1, G, DR>(src, row_bytes, sstride, nbase, H - 1, sub, LPR, nci, nchunk,
                                 min(it + 1, total - 1), s1);
    consume(it, s0);
    if (it + 1 >= total) break;
    load_step<FMT, NI, 1, G, DR>(src, row_bytes, sstride, nbase, H - 1, sub, LPR, nci, nchunk,
                                 min(it + 2, total - 1), s0);
    consume(it + 1, s1);
  }
}

template <int FMT, int LPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_dec_down(ExpertGemmArgs a, int rpw) {
  extern __shared__ __align__(16) uint16_t s_x[];
  Tile tile;
  if (!resolve_tile(a.src, blockIdx.y, tile)) return;
  if (blockIdx.x * kDecWaves * rpw >= a.H) return;
  const bool one = rpw == kDownRowsPerPass && a.I / DecFmt<FMT>::CPC <= LPR;
  if (tile.count == 1) {
    if (one) down_body<FMT, 1, LPR, false>(a, tile, rpw, s_x);
    else down_body<FMT, 1, LPR, true>(a, tile, rpw, s_x);
  } else if (tile.count == 2) {
    if (one) down_body<FMT, 2, LPR, false>(a, tile, rpw, s_x);
    else down_body<FMT, 2, LPR, true>(a, tile, rpw, s_x);
  } else {
    down_body<FMT, 4, LPR, true>(a, tile, rpw, s_x);
  }
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

// Rows per wave: one pass per wave unless the grid would run several short rounds of
// blocks (few tiles): then up to four passes, pipelined inside the wave (one per
// MOE_DEC_PASS_DIV one-pass blocks). DeepSeek-V3-like decode at 32 tokens, its shared expert
// beside it on the side stream: 2 passes 0.588-0.592 ms per step, 1 pass 0.590-0.594, 3 passes
// 0.601-0.604, 4 passes 0.604-0.605.
#ifndef MOE_DEC_PASS_DIV
#define MOE_DEC_PASS_DIV 8000
#endif
static int pick_rows_per_wave(int base, int n, int tile_bound) {
  const int blocks1 = ((n + kDecWaves * base - 1) / (kDecWaves * base)) * tile_bound;
  int m = blocks1 / MOE_DEC_PASS_DIV;
  m = m < 1 ? 1 : (m > 4 ? 4 : m);
  return base * m;
}

// LDS for the staged activations: kTileTok rows of K bf16. Launches beyond 64 KB need the
// kernel's dynamic-LDS limit raised; it is raised once per instantiation straight to the
// largest size the host lets through (kDecodeMaxLds), so a later call with a longer row
// never exceeds it. The function-local static makes the one call thread-safe.
static hipError_t raise_lds(const void* kern) {
  static_assert(kDecodeMaxLds <= 160 * 1024, "a CU has 160 KB of LDS");
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kDecodeMaxLds);
}

template <int FMT, int LPR>
static hipError_t launch_gu(const ExpertGemmArgs& a, int rpw, hipStream_t s) {
  const dim3 grid((a.I + kDecWaves * rpw - 1) / (kDecWaves * rpw), a.tile_bound);
  const size_t smem = (size_t)kTileTok * a.H * sizeof(uint16_t);
  if (smem > 65536) {
    static const hipError_t raised = raise_lds(reinterpret_cast<const void*>(k_dec_gate_up<FMT, LPR>));
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL((k_dec_gate_up<FMT, LPR>), grid, dim3(256), smem, s, a, rpw);
  return hipGetLastError();
}

template <int FMT, int LPR>
static hipError_t launch_dn(const ExpertGemmArgs& a, int rpw, hipStream_t s) {
  const dim3 grid((a.H + kDecWaves * rpw - 1) / (kDecWaves * rpw), a.tile_bound);
  const size_t smem = (size_t)kTileTok * a.I * sizeof(uint16_t);
  if (smem > 65536) {
    static const hipError_t raised = raise_lds(reinterpret_cast<const void*>(k_dec_down<FMT, LPR>));
    if (raised != hipSuccess) return raised;
  }
  hipLaunchKernelGGL((k_dec_down<FMT, LPR>), grid, dim3(256), smem, s, a, rpw);
  return hipGetLastError();
}

#define MOE_DISPATCH_LPR(LAUNCH, FMT, LPR, A, RPW, S)     \
  switch (LPR) {                                          \
    case 64: return LAUNCH<FMT, 64>(A, RPW, S);           \
    case 32: return LAUNCH<FMT, 32>(A, RPW, S);           \
    case 16: return LAUNCH<FMT, 16>(A, RPW, S);           \
    default: return LAUNCH<FMT, 8>(A, RPW, S);            \
  }

// ----------------------------------------------------------------------------- one step
// Rows of at most 64 chunks (K <= 2048 FP4 codes): a lane owns one 16-byte chunk of each
// of its rows (a group of LPR >= K / CPC lanes covers a row), so a wave loads all its
// weights at once and there is nothing to pipeline. The tile's tokens are then taken one
// after the other against the weights held in registers, their sums kept in registers
// and stored after the token loop; register use does not grow with the tile's tokens
// and stays within 64 VGPRs at ROWS = 4 (4/M rows per lane and matrix, 4 KB of weights
// per wave), so eight waves share each SIMD (five for MXFP4, whose scale decode needs more
// registers): they turn over finer than 8 KB waves in four.
// Grids of very many blocks (down projections onto a wide hidden size) take ROWS = 8:
// 8 KB per wave, four waves per SIMD, half the blocks.
template <int LPR, int M, int ROWS>
struct OneShape {
  static constexpr int G = kWave / LPR;                 // row groups per wave
  static constexpr int NI = (LPR < ROWS ? LPR : ROWS) / M;  // rows per lane and matrix
  static constexpr int GR = G * NI;                     // rows per wave
  static constexpr int NV = NI * M;                     // sums per lane before the reduction
  static_assert(NV <= LPR, "one reduced value per lane expected");
};

// The wave's GR output rows start at nbase; store(q, n, v) receives the result of the
// tile's q-th row for output row n (only rows n < N, one lane each).
template <int FMT, int LPR, int M, int ROWS, typename Store>
__device__ __forceinline__ void dec_one_body(const ExpertGemmArgs& a, const Tile& tile, int nbase,
                                             Store&& store) {
  using SH = OneShape<LPR, M, ROWS>;
  constexpr int G = SH::G, NI = SH::NI, GR = SH::GR, NV = SH::NV;
  constexpr int XW = DecFmt<FMT>::XW, CPC = DecFmt<FMT>::CPC;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  const int N = M == 2 ? a.I : a.H;  // output rows of each matrix
  const int K = M == 2 ? a.H : a.I;  // reduction length
  if (nbase >= N) return;  // whole wave
  const int nchunk = K / CPC;
  const bool live = sub < nchunk;
  const int c = live ? sub : nchunk - 1;
  const size_t row_bytes = dec_row_bytes<FMT>(K);
  const int sstride = dec_scale_stride<FMT>(K);
  const size_t sexp = dec_scale_expert_bytes<FMT>(N, K);
  const WeightDesc& w0 = M == 2 ? a.gate : a.down;
  const int e = tile.group;

  // every weight of the wave at once (rows clamped; results past N are not stored)
  uint4 w[NI][M];
  uint32_t sc[NI][M];
  const size_t eoff = (size_t)e * N * row_bytes;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = min(nbase + grp + G * i, N - 1);
    w[i][0] = load_weights16(w0.packed + eoff + (size_t)n * row_bytes + c * 16);
    sc[i][0] = load_chunk_scales<FMT>(w0.scales + e * sexp, n, sstride, c);
    if (M == 2) {
      w[i][M - 1] = load_weights16(a.up.packed + eoff + (size_t)n * row_bytes + c * 16);
      sc[i][M - 1] = load_chunk_scales<FMT>(a.up.scales + e * sexp, n, sstride, c);
    }
  }
  const float gs0 = FMT == 0 ? w0.global[e] : 1.0f;
  const float gs1 = M == 2 && FMT == 0 ? a.up.global[e] : 1.0f;
  const uint16_t* src = M == 2 ? a.x : a.h;
  const size_t stride = M == 2 ? (size_t)a.H : (size_t)a.h_stride;

  constexpr int kDiv = LPR / NV;  // lanes holding copies of one sum
  float res[kTileTok];
#pragma unroll
  for (int q = 0; q < kTileTok; ++q) res[q] = 0.f;
  int idx = 0;
  for (int t = 0; t < tile.count; ++t) {
    int tok = tile.tok[0];
#pragma unroll
    for (int q = 1; q < kTileTok; ++q) tok = t == q ? tile.tok[q] : tok;
    const int rows[1] = {M == 2 ? tok : tile.row0 + t};
    uint32_t xv[1][XW];
    global_act_chunk<1, XW>(src, stride, rows, c, xv);
    if (!live) {  // lanes past the row's chunks add nothing
#pragma unroll
      for (int q = 0; q < XW; ++q) xv[0][q] = 0u;
    }
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        // an opaque copy per token: decoding the weights once, outside the token loop,
        // would not fit the register budget
        uint4 wv = w[i][m];
        uint32_t sv = sc[i][m];
        asm volatile("" : "+v"(wv.x), "+v"(wv.y), "+v"(wv.z), "+v"(wv.w), "+v"(sv));
        float r[1] = {0.f};
        chunk_dot<FMT, 1>(wv, sv, xv, r);
        acc[i * M + m] = r[0];
      }
    group_reduce_transpose<NV, LPR>(acc, lane);
    idx = reduced_index<NV, LPR>(lane, 0);
    float v;
    if (M == 2) {  // gate / up partners differ in lane bit kDiv
      const float other = shfl_xor_f(acc[0], kDiv);
      v = silu(acc[0] * gs0) * (other * gs1);
    } else {
      v = acc[0] * gs0;
    }
#pragma unroll
    for (int q = 0; q < kTileTok; ++q) res[q] = t == q ? v : res[q];
  }
  // one store per owned row and token, after the loop (the compiler waits for every load in
  // flight before entering a loop that stores without loading anything itself)
  const bool owner = M == 2 ? ((idx & 1) == 0 && (sub & (kDiv - 1)) == 0) : (sub & (kDiv - 1)) == 0;
  const int n = nbase + grp + G * (M == 2 ? idx >> 1 : idx);
  if (owner && n < N) {
#pragma unroll
    for (int q = 0; q < kTileTok; ++q) {
      if (q < tile.count) store(q, n, res[q]);
    }
  }
}

// The tile's rows of h (gate+up) or y (down) in memory.
template <int M>
struct StoreRows {
  const ExpertGemmArgs& a;
  const Tile& tile;
  __device__ __forceinline__ void operator()(int q, int n, float v) const {
    if (M == 2) a.h[(size_t)(tile.row0 + q) * a.h_stride + n] = f32_to_bf16(v);
    else reinterpret_cast<float*>(a.y)[(size_t)(tile.row0 + q) * a.H + n] = v;
  }
};

template <int FMT, int LPR, int M, int ROWS>
__device__ __forceinline__ int one_nbase() {
  return (blockIdx.x * kDecWaves + (threadIdx.x >> 6)) * OneShape<LPR, M, ROWS>::GR;
}

template <int FMT, int LPR, int M, int ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ROWS == 4 ? (FMT == 0 ? 8 : 5) : 4))) void k_dec_one(ExpertGemmArgs a) {
  Tile tile;
  if (!resolve_tile(a.src, blockIdx.y, tile)) return;
  dec_one_body<FMT, LPR, M, ROWS>(a, tile, one_nbase<FMT, LPR, M, ROWS>(), StoreRows<M>{a, tile});
}

// A few tokens without a shared expert: the down projection of every slot and the blend in
// one kernel (MoE constructor page: the weighted-sum blend into the residual). A block has one
// wave per tile (at most kBlendMaxTiles; beyond that, several tiles a wave, one after the
// other), all on the same GR output rows; the waves leave their
// sums in LDS by row, then the block's first T x GR threads (token t, output row i) add that
// token's slots in order (w_j * y_j, a zero-computation expert's w_j * x_e, a dropped slot
// nothing) and the residual, exactly as the separate blend does, and store bf16 out. The fp32
// rows of y never reach memory and the blend needs no launch of its own.
constexpr int kBlendMaxTiles = 16;
constexpr int kBlendMaxSlots = kBlendMaxTiles * kTileTok;  // token rows of the block's tiles

template <int FMT, int LPR, int ROWS, bool MULTI>
__global__ __launch_bounds__(kBlendMaxTiles * 64) void k_dec_one_blend(ExpertGemmArgs a, CombineArgs cb) {
  constexpr int GR = OneShape<LPR, 1, ROWS>::GR;
  __shared__ float s_y[kBlendMaxSlots][GR];  // [row of a token][output row]
  // the blend's inputs that do not depend on the sums (each slot's row and weight, the
  // residual of the block's rows, in 4-byte slots) reach LDS by direct-to-LDS loads that
  // wave 0 issues before its part of the down projection: their latency is hidden, and no
  // register waits for them
  __shared__ int32_t s_inv[kBlendMaxSlots];
  __shared__ float s_w[kBlendMaxSlots];
  __shared__ uint32_t s_res[kBlendMaxSlots];
  const int nbase = blockIdx.x * GR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rbase = a.rows - cb.T * cb.K;  // first routed row (the tokens' rows follow)
  if (wave == 0) {
    if (lane < cb.T * cb.K) {
      dma4(cb.inv + lane, lds_addr(reinterpret_cast<const uint8_t*>(s_inv)));
      dma4(cb.w + lane, lds_addr(reinterpret_cast<const uint8_t*>(s_w)));
    }
    const int rt = lane / GR, rn = nbase + lane % GR;  // (token, output row) of a residual
    if (cb.residual && rt < cb.T && rn < cb.H)
      dma2(cb.residual + (size_t)rt * cb.H + rn, lds_addr(reinterpret_cast<const uint8_t*>(s_res)));
  }
  if constexpr (MULTI) {  // several tiles a wave, one after the other
    for (int tw = wave; tw < a.tile_bound; tw += (int)(blockDim.x >> 6)) {
      Tile tile;
      if (resolve_tile(a.src, tw, tile)) {
        auto store = [&](int q, int n, float v) { s_y[tile.row0 + q - rbase][n - nbase] = v; };
        dec_one_body<FMT, LPR, 1, ROWS>(a, tile, nbase, store);
      }
    }
  } else {  // one tile a wave (the loop would cost the 8 KB waves registers)
    Tile tile;
    if (resolve_tile(a.src, wave, tile)) {
      auto store = [&](int q, int n, float v) { s_y[tile.row0 + q - rbase][n - nbase] = v; };
      dec_one_body<FMT, LPR, 1, ROWS>(a, tile, nbase, store);
    }
  }
  if (wave == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // (the loads above landed)
  __syncthreads();
  const int t = threadIdx.x / GR, i = threadIdx.x % GR, n = nbase + i;
  if (t >= cb.T || n >= cb.H) return;
  float acc = 0.f;
  for (int j = 0; j < cb.K; ++j) {
    const int p = s_inv[t * cb.K + j];
    const float wj = s_w[t * cb.K + j];
    if (p >= 0) acc = fmaf(wj, s_y[p - rbase][i], acc);
    else if (p == -2) acc = fmaf(wj, bf16_to_f32(cb.xe[(size_t)t * cb.H + n]), acc);
  }
  if (cb.residual) acc += bf16_to_f32((uint16_t)(s_res[threadIdx.x] & 0xFFFFu));
  cb.out[(size_t)t * cb.H + n] = f32_to_bf16(acc);
}

// One token with top-K selection: the experts are chosen inside the gate+up kernel. The k
// selected experts are distinct, so the dispatch is their order: slot j's row is
// shared_rows + rank of its expert among the k, one 1-row tile per slot in expert order.
// Grid row 0 is the routing writer: its first block's first wave runs the full selection
// and writes the routing outputs and the dispatch (ids, weights, logits, row map, inverse
// map, tiles, tile count, error word) that the down projection and the blend read. Grid row
// 1 + r computes the expert of rank r: each block's first wave finds that expert with the
// lean selection (the same keys and rounds, no weights, no outputs) and hands it to the
// block's other waves through LDS (Qwen3-like layer at one token, graph-replayed: 15.8 us
// per step, against 16.4 us with the lean selection in every wave and no barrier).
template <int FMT, int LPR, int NPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FMT == 0 ? 8 : 5))) void k_dec_one_topk(ExpertGemmArgs a, TopkArgs ta, FusedRoute fr) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (blockIdx.y == 0) {
    if (blockIdx.x != 0 || wave != 0) return;
    const int id = topk_token<NPL>(ta, 0, nullptr, nullptr);
    int rank = 0;  // distinct experts: rank = how many selected experts have a lower index
    for (int j = 0; j < ta.K; ++j) rank += __shfl(id, j, kWave) < id ? 1 : 0;
    if (lane < ta.K) {
      const int row = fr.shared_rows + rank;
      fr.inv[lane] = row;
      fr.row_token[row] = 0;
      Tile tl;
      tl.group = id;
      tl.row0 = row;
      tl.count = 1;
      tl.pad = 0;
#pragma unroll
      for (int q = 0; q < kTileTok; ++q) tl.tok[q] = 0;
      fr.tiles[rank] = tl;
    }
    if (lane == 0) {
      publish_tile_count(fr.ntiles, ta.K);
      fr.err_word[0] = 0;
      if (fr.shared_rows) fr.row_token[0] = 0;
    }
    return;
  }
  const int r = (int)blockIdx.y - 1;
  Tile tile;
  __shared__ int s_grp;
  if (wave == 0) {
    const int g = topk_token<NPL, true>(ta, 0, nullptr, nullptr, r);
    if (lane == 0) s_grp = g;
  }
  __syncthreads();
  tile.group = s_grp;
  tile.row0 = fr.shared_rows + r;
  tile.count = 1;
  tile.pad = 0;
#pragma unroll
  for (int q = 0; q < kTileTok; ++q) tile.tok[q] = 0;
  dec_one_body<FMT, LPR, 2, 4>(a, tile, one_nbase<FMT, LPR, 2, 4>(), StoreRows<2>{a, tile});
}

// Host side: FP4 weights, rows of at most 64 chunks, tiles of at most kTileTok rows.
static int one_lanes(int nchunk) {
  int l = 8;
  while (l < nchunk) l <<= 1;
  return l;
}

static bool one_fits(int fmt, int K, int tile_h) {
  return fmt <= 1 && K / 32 <= 64 && tile_h <= kTileTok;
}

template <int FMT, int LPR, int M, int ROWS>
static hipError_t launch_one_t(const ExpertGemmArgs& a, hipStream_t s) {
  const int N = M == 2 ? a.I : a.H;
  const int rows = kDecWaves * OneShape<LPR, M, ROWS>::GR;
  hipLaunchKernelGGL((k_dec_one<FMT, LPR, M, ROWS>), dim3((N + rows - 1) / rows, a.tile_bound),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// Down projections onto at least this many outputs per expert run 8 KB waves (ROWS = 8):
// DeepSeek-V3-like H = 7168 at 32 tokens, about 204 vs 220 us with 4 KB waves; Qwen3-like
// H = 2048 at 8 tokens, 13.4 vs 13.9 us the other way.
constexpr int kOneWideMinN = 4096;

template <int M>
static hipError_t launch_one(const ExpertGemmArgs& a, int fmt, int K, hipStream_t s) {
  const int lpr = one_lanes(K / 32);
#define MOE_ONE_LPR(FMT, ROWS)                                    \
  switch (lpr) {                                                  \
    case 8: return launch_one_t<FMT, 8, M, ROWS>(a, s);           \
    case 16: return launch_one_t<FMT, 16, M, ROWS>(a, s);         \
    case 32: return launch_one_t<FMT, 32, M, ROWS>(a, s);         \
    default: return launch_one_t<FMT, 64, M, ROWS>(a, s);         \
  }
  if constexpr (M == 1) {
    if (a.H >= kOneWideMinN) {
      if (fmt == 0) { MOE_ONE_LPR(0, 8) }
      MOE_ONE_LPR(1, 8)
    }
  }
  if (fmt == 0) { MOE_ONE_LPR(0, 4) }
  MOE_ONE_LPR(1, 4)
#undef MOE_ONE_LPR
}

// codes per 16-byte chunk of a format (host side of DecFmt)
static int codes_per_chunk(int fmt) { return fmt <= 1 ? 32 : (fmt == 2 ? 16 : 8); }

hipError_t launch_decode_gate_up(const ExpertGemmArgs& a, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  if (one_fits(a.gate.fmt, a.H, a.src.tiles ? kDecodeTile : a.src.implicit_height))
    return launch_one<2>(a, a.gate.fmt, a.H, s);
  const int rpw = pick_rows_per_wave(kGateRowsPerPass, a.I, a.tile_bound);
  const int lpr = pick_lpr(a.H / codes_per_chunk(a.gate.fmt));
  switch (a.gate.fmt) {
    case 0: MOE_DISPATCH_LPR(launch_gu, 0, lpr, a, rpw, s)
    case 1: MOE_DISPATCH_LPR(launch_gu, 1, lpr, a, rpw, s)
    case 2: MOE_DISPATCH_LPR(launch_gu, 2, lpr, a, rpw, s)
    default: MOE_DISPATCH_LPR(launch_gu, 3, lpr, a, rpw, s)
  }
}

// (at most 128 experts: two keys per lane keep the selection within the kernel's 64 VGPRs)
bool decode_topk_fusable(int fmt, int H, int E) { return one_fits(fmt, H, kTileTok) && E <= 128; }

template <int FMT, int LPR>
static hipError_t launch_topk_t(const ExpertGemmArgs& a, const TopkArgs& ta, const FusedRoute& fr,
                                hipStream_t s) {
  const int rows = kDecWaves * OneShape<LPR, 2, 4>::GR;
  const dim3 grid((a.I + rows - 1) / rows, ta.K + 1);  // row 0: the routing writer
  const int npl = (ta.E + 63) / 64;
  if (npl <= 1) hipLaunchKernelGGL((k_dec_one_topk<FMT, LPR, 1>), grid, dim3(256), 0, s, a, ta, fr);
  else hipLaunchKernelGGL((k_dec_one_topk<FMT, LPR, 2>), grid, dim3(256), 0, s, a, ta, fr);
  return hipGetLastError();
}

hipError_t launch_decode_gate_up_topk(const ExpertGemmArgs& a, const TopkArgs& ta,
                                      const FusedRoute& fr, hipStream_t s) {
  if (!decode_topk_fusable(a.gate.fmt, a.H, ta.E) || ta.T != 1) return hipErrorInvalidValue;
  const int lpr = one_lanes(a.H / 32);
#define MOE_TOPK_LPR(FMT)                                  \
  switch (lpr) {                                           \
    case 8: return launch_topk_t<FMT, 8>(a, ta, fr, s);    \
    case 16: return launch_topk_t<FMT, 16>(a, ta, fr, s);  \
    case 32: return launch_topk_t<FMT, 32>(a, ta, fr, s);  \
    default: return launch_topk_t<FMT, 64>(a, ta, fr, s);  \
  }
  if (a.gate.fmt == 0) { MOE_TOPK_LPR(0) }
  MOE_TOPK_LPR(1)
#undef MOE_TOPK_LPR
}

// One token, no shared expert, FP4 down rows of at most 64 chunks, at most kBlendMaxTiles
// tiles: the down projection and the blend in one launch.
// Tiles a wave of the fused down+blend kernel may take, one after the other. Qwen3-like layer
// at eight tokens (up to 64 tiles, four a wave): step 47.2 -> 45.3 us eager, 45.9 -> 44.4 us
// replayed against the separate down projection and blend (their down stage 12.9 us, the
// fused one 16.0 us with the blend inside).
#ifndef MOE_BLEND_TILES_PER_WAVE
#define MOE_BLEND_TILES_PER_WAVE 4
#endif
bool decode_blend_fusable(const ExpertGemmArgs& a, const CombineArgs& cb) {
  if (cb.shared || !a.src.tiles || a.tile_bound > MOE_BLEND_TILES_PER_WAVE * kBlendMaxTiles ||
      !one_fits(a.down.fmt, a.I, kDecodeTile))
    return false;
  // several tiles a wave only with the 4 KB waves (the 8 KB waves' loop would spill)
  if (a.tile_bound > kBlendMaxTiles && a.H >= kOneWideMinN) return false;
  // output rows per block of the one-step down GEMV (OneShape<LPR, 1, ROWS>::GR)
  const int lpr = one_lanes(a.I / 32), rows = a.H >= kOneWideMinN ? 8 : 4;
  const int gr = (kWave / lpr) * (lpr < rows ? lpr : rows);
  // every slot's row and weight, and every (token, output row) residual, in one wave's lanes
  return cb.T * cb.K <= kWave && cb.T * gr <= kWave;
}

template <int FMT, int LPR, int ROWS>
static hipError_t launch_blend_t(const ExpertGemmArgs& a, const CombineArgs& cb, hipStream_t s) {
  constexpr int GR = OneShape<LPR, 1, ROWS>::GR;
  const int waves = a.tile_bound < kBlendMaxTiles ? a.tile_bound : kBlendMaxTiles;
  if (ROWS == 4 && a.tile_bound > kBlendMaxTiles)
    hipLaunchKernelGGL((k_dec_one_blend<FMT, LPR, ROWS, ROWS == 4>), dim3((a.H + GR - 1) / GR),
                       dim3(waves * 64), 0, s, a, cb);
  else
    hipLaunchKernelGGL((k_dec_one_blend<FMT, LPR, ROWS, false>), dim3((a.H + GR - 1) / GR),
                       dim3(waves * 64), 0, s, a, cb);
  return hipGetLastError();
}

hipError_t launch_decode_down_blend(const ExpertGemmArgs& a, const CombineArgs& cb,
                                    hipStream_t s) {
  if (!decode_blend_fusable(a, cb) || a.tile_bound <= 0) return hipErrorInvalidValue;
  const int lpr = one_lanes(a.I / 32);
  const bool wide = a.H >= kOneWideMinN;
#define MOE_BLEND_LPR(FMT, ROWS)                                  \
  switch (lpr) {                                                  \
    case 8: return launch_blend_t<FMT, 8, ROWS>(a, cb, s);        \
    case 16: return launch_blend_t<FMT, 16, ROWS>(a, cb, s);      \
    case 32: return launch_blend_t<FMT, 32, ROWS>(a, cb, s);      \
    default: return launch_blend_t<FMT, 64, ROWS>(a, cb, s);      \
  }
  if (a.down.fmt == 0) {
    if (wide) { MOE_BLEND_LPR(0, 8) }
    MOE_BLEND_LPR(0, 4)
  }
  if (wide) { MOE_BLEND_LPR(1, 8) }
  MOE_BLEND_LPR(1, 4)
#undef MOE_BLEND_LPR
}

hipError_t launch_decode_down(const ExpertGemmArgs& a, hipStream_t s) {
  if (a.tile_bound <= 0) return hipSuccess;
  if (one_fits(a.down.fmt, a.I, a.src.tiles ? kDecodeTile : a.src.implicit_height))
    return launch_one<1>(a, a.down.fmt, a.I, s);
  const int rpw = pick_rows_per_wave(kDownRowsPerPass, a.H, a.tile_bound);
  const int lpr = pick_lpr(a.I / codes_per_chunk(a.down.fmt));
  switch (a.down.fmt) {
    case 0: MOE_DISPATCH_LPR(launch_dn, 0, lpr, a, rpw, s)
    case 1: MOE_DISPATCH_LPR(launch_dn, 1, lpr, a, rpw, s)
    case 2: MOE_DISPATCH_LPR(launch_dn, 2, lpr, a, rpw, s)
    default: MOE_DISPATCH_LPR(launch_dn, 3, lpr, a, rpw, s)
  }
}

// ----------------------------------------------------------------------------- debug
// Decode one expert matrix to f32 [n, k] with the device routine of a path, 8 values per
// thread: path 1 (decode GEMV): codes -> bf16 (scale 1) -> f32, times the fp32 block scale;
// path 2 (MFMA operand): the bf16 operand the grouped GEMM feeds its MFMAs. FP4 then times
// the NVFP4 global scale (one fp32 rounding); BF16 weights are their own values.
__global__ void k_debug_dequant(WeightDesc w, int expert, int path, float* out) {
  const int groups_per_row = w.k / 8;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= w.n * groups_per_row) return;
  const int row = i / groups_per_row, d = i % groups_per_row;
  const size_t erow = (size_t)expert * w.n + row;
  uint32_t b[4];
  float scale_after = 1.0f, g = 1.0f;
  if (w.fmt <= 1) {
    const size_t rbytes = (size_t)w.k / 2;
    const uint32_t q = reinterpret_cast<const uint32_t*>(w.packed + erow * rbytes)[d];
    const int blk = w.fmt == 0 ? 16 : 32;
    const uint8_t sb = w.scales[erow * (w.k / blk) + (d * 8) / blk];
    g = w.fmt == 0 ? w.global[expert] : 1.0f;
    if (path == 1) {
      fp4x8_to_bf16(q, 1.0f, b);
      scale_after = w.fmt == 0 ? e4m3_to_f32(sb) : e8m0_to_f32(sb);
    } else {
      mfma_operand_fp4x8(w.fmt, q, sb, b);
    }
  } else if (w.fmt == 2) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(w.packed + erow * w.k) + 2 * d;
    const int kb = (w.k + 127) / 128, nb = (w.n + 127) / 128;
    const float sc = reinterpret_cast<const float*>(w.scales)[((size_t)expert * nb + row / 128) * kb +
                                                             (d * 8) / 128];
    if (path == 1) {
      fp8x4_to_bf16(q[0], b);
      fp8x4_to_bf16(q[1], b + 2);
      scale_after = sc;
    } else {
      mfma_operand_fp8x8(q[0], q[1], sc, b);
    }
  } else {
    const uint4 v = reinterpret_cast<const uint4*>(w.packed + erow * w.k * 2)[d];
    b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
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
