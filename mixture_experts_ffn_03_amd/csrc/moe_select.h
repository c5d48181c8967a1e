// Device routines shared by the top-K and dispatch kernels (moe_route.hip,
// moe_dispatch.hip): the per-token expert selection and the expert-grouping counting sort.
//
// MoE constructor page (spark_model/layers/moe/init.rs): softmax, sigmoid-with-bias and
// hash top-K kernels, and the sort-by-expert / tile work list of the grouped path; MoE
// module page (spark_model/layers/moe/mod.rs): docs of correction_bias_dev and
// tid2eid_dev, and indices and weights staying on the device.
#pragma once
#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// Selection keys: an order-preserving map of the fp32 key to uint32, so the largest
// value is the largest key, -0 == +0, and NaN (1) ranks below -inf (0x007FFFFF). 0 marks
// padding and experts already taken. Equal keys go to the lower expert index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_key(float f) {
  if (f != f) return 1u;         // NaN: below every number
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide reductions by DPP inside each row of 16 lanes (quad swaps, then the half-row
// and row mirrors), then the four rows' values read out and combined in row order. At
// every step both lanes of a pair combine the same two values, so all lanes end with the
// same result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Per-expert score of the sigmoid (1) and sqrt-softplus (2) modes, in fp64: rounded once
// to fp32 by the caller, it is the correctly rounded value in all but rare cases, so the
// selection is reproducible on any platform. softplus(l) = ln(1 + e^l) is evaluated as
// l + log1p(e^-l) for l > 0 and log1p(e^l) otherwise (no overflow).
__device__ __forceinline__ double score_f64(int score, float logit) {
  const double l = (double)logit;
  if (score == 1) return 1.0 / (1.0 + exp(-l));
  const double sp = l > 0.0 ? l + log1p(exp(-l)) : log1p(exp(l));
  return sqrt(sp);
}

// ---------------------------------------------------------------------------
// Scores + top-K of token t by one wavefront, its E keys spread over the 64 lanes (NPL
// per lane). Selection is k rounds of a wave-wide maximum of the ordered keys, ties to the
// lowest expert index by ballot. Writes ids / w (and logits_out, err_tok) to global
// memory; lds_ids / lds_err (if not null) also receive ids[t*K..] and the token's error.
// ---------------------------------------------------------------------------
// Returns, in lane j < K, the expert of slot j (-1 for a dropped slot; other lanes -1). The
// global outputs (ids, w, err_tok, logits_out) are written where their pointers are set.
// LEAN form (top-K selection only, no outputs, no routing weights): every lane returns the
// selected expert of rank `rank` in index order (the rank-th lowest index among the k
// selected), from the same keys and the same selection rounds as the full form; the
// softmax normaliser is only formed where a key needs it (softmax+bias).
template <int NPL, bool LEAN = false>
__device__ __forceinline__ int topk_token(const TopkArgs& a, int t, int32_t* lds_ids,
                                          int32_t* lds_err, int rank = 0) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K;

  // every load of the token up front (unconditional, clamped addresses), then the sums:
  // the split-K partials are added in slice order, then the logit bias
  float lg[NPL];
  float key[NPL];
  float cbias[NPL];
  if (a.logits_in) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + kWave * i;
      lg[i] = a.logits_in[(size_t)t * E + (e < E ? e : 0)];
    }
  } else {
    double pz[NPL][kRouterMaxSplit];
    double lb[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + kWave * i, ec = e < E ? e : 0;
#pragma unroll
      for (int z = 0; z < kRouterMaxSplit; ++z)
        pz[i][z] = a.partial[((size_t)(z < a.ks ? z : 0) * a.T + t) * E + ec];
      lb[i] = a.logit_bias ? (double)a.logit_bias[ec] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      double acc = 0.0;
#pragma unroll
      for (int z = 0; z < kRouterMaxSplit; ++z)
        if (z < a.ks) acc += pz[i][z];
      if (a.logit_bias) acc += lb[i];
      lg[i] = (float)acc;
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i, ec = e < E ? e : 0;
    cbias[i] = a.correction_bias ? a.correction_bias[ec] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      if (!LEAN && a.logits_out) a.logits_out[(size_t)t * E + e] = lg[i];
    } else {
      lg[i] = -__builtin_inff();  // padding: never selectable, no softmax mass
    }
    float k = lg[i];
    if (a.score == 1 || a.score == 2) {  // sigmoid / sqrt-softplus: fp32(score) + bias
      const float sg = (float)score_f64(a.score, lg[i]);
      k = a.correction_bias ? sg + cbias[i] : sg;
    }
    key[i] = k;
  }

  // softmax normaliser over all experts: m = max, S = sum exp(l - m) (fp32; fp64 for the
  // softmax+bias key, whose probability is rounded once)
  float m = -__builtin_inff(), S = 0.f;
  double S64 = 0.0;
  if ((!LEAN && a.score == 0) || a.score == 3) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) m = fmaxf(m, lg[i]);
    m = wave_max_dpp(m);
  }
  if (!LEAN && a.score == 0) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < E) S += expf(lg[i] - m);
    S = wave_sum_dpp(S);
  } else if (a.score == 3) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < E) S64 += exp((double)lg[i] - (double)m);
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) S64 += __shfl_xor(S64, msk, kWave);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float p = (float)(exp((double)lg[i] - (double)m) / S64);
      key[i] = a.correction_bias ? p + cbias[i] : p;
    }
  }

  int err = 0;
  int my_id = -1;  // lane j < K: the expert of slot j
  if (a.select == 0) {
    uint32_t kv[NPL];  // ordered keys; 0 = padding or taken
#pragma unroll
    for (int i = 0; i < NPL; ++i) kv[i] = lane + kWave * i < E ? ordered_key(key[i]) : 0u;
    for (int j = 0; j < K; ++j) {
      uint32_t best = kv[0];
#pragma unroll
      for (int i = 1; i < NPL; ++i) best = max(best, kv[i]);
      const uint32_t g = wave_max_u32(best);
      int idx = -1;  // lowest expert index holding the maximum (wave-uniform)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const uint64_t mk = __ballot(kv[i] == g);
        if (idx < 0 && mk) idx = kWave * i + __builtin_ctzll(mk);
      }
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == (idx >> 6) && lane == (idx & 63)) kv[i] = 0u;  // taken
      if (lane == j) my_id = idx;
    }
    if constexpr (LEAN) {
      // the selected experts are the valid lanes whose key was taken (a valid key is never
      // 0); walk their index-ordered masks to the rank-th one
      int r = rank, e = -1;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        uint64_t sel = __ballot(lane + kWave * i < E && kv[i] == 0u);
        const int c = __popcll(sel);
        if (e < 0 && r < c) {
          for (int q = 0; q < r; ++q) sel &= sel - 1;
          e = kWave * i + __builtin_ctzll(sel);
        }
        r -= c;
      }
      return e;
    }
  } else {  // hash routing: ids from the static table, no selection
    const int64_t tok = a.token_ids[t];
    const bool tok_ok = tok >= 0 && tok < a.vocab;
    if (!tok_ok) err |= 2;
    if (lane < K && tok_ok) {
      const int64_t e = a.tid2eid[tok * K + lane];
      if (e >= 0 && e < E) my_id = (int)e;
      else err |= 4;
    }
    err = __builtin_amdgcn_readfirstlane(err) | (int)(__ballot(err & 4) ? 4 : 0);
  }
  if constexpr (LEAN) return -1;  // (the lean form selects; it never takes hash routing)

  // the selected experts' logits, fetched from their lanes (every lane takes part)
  float l = 0.f;
  {
    const int src = my_id >= 0 ? my_id : 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float c = __shfl(lg[i], src & 63, kWave);
      if (i == (src >> 6)) l = c;
    }
  }

  // weights of the selected experts, one slot per lane, then the (optional) normalisation
  float wj = 0.f;
  if (lane < K && my_id >= 0) {
    wj = a.score == 0   ? expf(l - m) / S
         : a.score == 3 ? (float)(exp((double)l - (double)m) / S64)
                        : (float)score_f64(a.score, l);
  }
  if (a.renorm) {
    const float sum = wave_sum_dpp(wj);
    wj = sum > 0.f ? wj / sum : 0.f;
  }
  if (lane < K) {
    if (a.w) a.w[(size_t)t * K + lane] = wj * a.scaling;
    if (a.ids) a.ids[(size_t)t * K + lane] = my_id;
    if (lds_ids) lds_ids[t * K + lane] = my_id;
  }
  if (lane == 0) {
    if (a.err_tok) a.err_tok[t] = err;
    if (lds_err) lds_err[t] = err;
  }
  return lane < K ? my_id : -1;
}

// ---------------------------------------------------------------------------
// Dispatch (stable counting sort by expert) by one block of NW waves.
//
// Row space: when a shared expert is present its T rows come first (row t = token t),
// then the routed groups in expert order, each group's rows in (token, slot) order.
// Outputs: row_token[p] (token whose input feeds row p), inv[t*K + j] (row of slot
// (t, j); -2 for a zero-computation expert, id in [E, E + zero); -1 for any other id
// outside [0, E)), the tile list ((expert, first row, row
// count) runs of at most tile_h rows), ntiles and the call's error word. ids / err_tok
// may point to global or LDS memory; s_wbase holds NW x EMAX ints.
// ---------------------------------------------------------------------------
template <int NW>
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < NW ? s_tmp[lane] : 0;
    int inc = w;
#pragma unroll
    for (int d = 1; d < NW; d <<= 1) {
      const int y = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += y;
    }
    if (lane < NW) s_tmp[NW + lane] = inc - w;
    if (lane == NW - 1) s_tmp[2 * NW] = inc;
  }
  __syncthreads();
  const int r = x - v + s_tmp[NW + wave];
  *total = s_tmp[2 * NW];
  __syncthreads();
  return r;
}

// Dispatch of at most NW * 64 slots and EMAX experts by one block of NW waves (one thread
// per slot and per expert), for ids already in LDS: the same row space, tile list and error bits as
// dispatch_body, from a bitmap of the slots of each expert (s_mask[e * W + w], bit b =
// slot 64 w + b, W = ceil(S / 64) words). An expert's rows are its slots in slot order,
// so a slot's row inside the group is the number of the expert's bits below its own.
// Tiles of at most kTileTok rows get their tokens from the slots (no read-back).
// Two barriers after the ids are in place; s_mask must be zero on entry.
template <int NW, int EMAX>
__device__ void dispatch_bitmap(const DispatchArgs& a, const int32_t* ids, const int32_t* err_tok,
                                uint64_t* s_mask, int* s_off, int* s_toff, int* s_tot,
                                int* s_err) {
  constexpr int NT = NW * kWave;
  static_assert(EMAX <= NT && NT < (1 << 16), "one thread per expert; packed sums");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.K, S = a.T * a.K, W = (S + 63) / 64, h = a.tile_h;

  // slots into the experts' bitmaps; error bits
  const bool in = tid < S;
  const int e = in ? ids[tid] : -1;
  const bool valid = in && e >= 0 && e < E;
  int err = (in && !valid && !(err_tok && e == -1) && !(e >= E && e < E + a.zero)) ? 1 : 0;
  if (err_tok && tid < a.T) err |= err_tok[tid];
  if (valid) atomicOr((unsigned long long*)&s_mask[e * W + (tid >> 6)], 1ull << (tid & 63));
  if (err) atomicOr(s_err, err);
  for (int p = tid; p < a.shared_rows; p += NT) a.row_token[p] = p;
  __syncthreads();

  // per expert: row count and tile count, exclusive scans of both (packed in one int)
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < W; ++w) cnt += __popcll(s_mask[tid * W + w]);
  const int nt = (cnt + h - 1) / h;
  const int packed = cnt | (nt << 16);  // both sums <= S <= NW * 64 < 2^16
  int inc = packed;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += y;
  }
  constexpr int EW = (EMAX + 63) / 64;  // waves holding experts
  if (lane == 63 && wave < EW) s_tot[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < EW; ++w) {
    const int v = w * kWave < E ? s_tot[w] : 0;
    before += w < wave ? v : 0;
    all += v;
  }
  const int excl = inc - packed + before;
  const int row0 = a.shared_rows + (excl & 0xFFFF), toff = excl >> 16;
  if (tid < E) {
    s_off[tid] = row0;
    s_toff[tid] = toff;
    for (int i = 0; i < nt; ++i) {  // tile headers; short tiles' unused tokens are 0
      const int c = min(h, cnt - i * h);
      Tile* tl = a.tiles + toff + i;
      *(int4*)tl = make_int4(tid, row0 + i * h, c, 0);
#pragma unroll
      for (int q = 0; q < kTileTok; ++q)
        if (h > kTileTok || q >= c) tl->tok[q] = 0;
    }
  }
  if (tid == 0) {
    publish_tile_count(a.ntiles, all >> 16);
    a.err_word[0] = *s_err;
  }
  __syncthreads();

  // each slot: its row, the row's token, the token field of its tile
  if (valid) {
    const int wb = tid >> 6;
    int rank = __popcll(s_mask[e * W + wb] & ((1ull << (tid & 63)) - 1ull));
    for (int w = 0; w < wb; ++w) rank += __popcll(s_mask[e * W + w]);
    const int pos = s_off[e] + rank;
    const int tok = tid / K;
    a.row_token[pos] = tok;
    a.inv[tid] = pos;
    if (h <= kTileTok) a.tiles[s_toff[e] + rank / h].tok[rank % h] = tok;
  } else if (in) {
    a.inv[tid] = (e >= E && e < E + a.zero) ? -2 : -1;
  }
}

// chunks of 64 slots whose ids one wave loads at once
constexpr int kDispatchBatch = 8;

// Stable scatter of slots [sb, se) by one wave: row_token and inv of every slot; s_wbase_w
// (per expert) holds the wave's next row inside each expert group, s_off the groups' first
// rows. Lanes with equal ids are ranked by lane order within each chunk of 64 slots.
__device__ __forceinline__ void scatter_segment(const DispatchArgs& a, const int32_t* ids, int sb,
                                                int se, int* s_wbase_w, const int* s_off) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K;
  for (int c0 = sb; c0 < se; c0 += kDispatchBatch * kWave) {
    int ev[kDispatchBatch];
#pragma unroll
    for (int j = 0; j < kDispatchBatch; ++j) {
      const int s = c0 + j * kWave + lane;
      ev[j] = s < se ? ids[s] : -1;
    }
#pragma unroll
    for (int j = 0; j < kDispatchBatch; ++j) {
      if (c0 + j * kWave >= se) break;  // past the segment (wave-uniform)
      const int s = c0 + j * kWave + lane;
      const bool in = s < se;
      const int e = ev[j];
      const bool valid = in && e >= 0 && e < E;
      uint64_t m = __ballot(valid);
      for (int b = 0; (1 << b) < E; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      if (valid) {
        const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
        const int rank = __popcll(below);
        const int cntm = __popcll(m);
        const int base = s_wbase_w[e];
        const int pos = s_off[e] + base + rank;
        a.row_token[pos] = s / K;
        a.inv[s] = pos;
        if (rank == cntm - 1) s_wbase_w[e] = base + cntm;
      } else if (in) {
        a.inv[s] = (e >= E && e < E + a.zero) ? -2 : -1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Tile list of a block of NW waves: thread e < E holds its expert's row count `cnt`, s_off
// the group's first row; ceil(cnt / tile_h) runs per expert, experts in order. Tiles of at
// most kTileTok rows also carry their rows' tokens (row_token must be complete and visible).
template <int NW>
__device__ __forceinline__ void write_tiles(const DispatchArgs& a, int cnt, const int* s_off,
                                            int* s_tmp, int* ntot) {
  const int tid = threadIdx.x;
  const int h = a.tile_h;
  const int nt = (tid < a.E) ? (cnt + h - 1) / h : 0;
  const int toff = block_exclusive_scan<NW>(nt, s_tmp, ntot);
  __syncthreads();  // row_token of every routed row is written (read back below)
  if (tid < a.E) {
    for (int i = 0; i < nt; ++i) {
      Tile tl;
      tl.group = tid;
      tl.row0 = s_off[tid] + i * h;
      tl.count = min(h, cnt - i * h);
      tl.pad = 0;
#pragma unroll
      for (int q = 0; q < kTileTok; ++q)
        tl.tok[q] = (h <= kTileTok && q < tl.count) ? a.row_token[tl.row0 + q] : 0;
      a.tiles[toff + i] = tl;
    }
  }
}

template <int NW, int EMAX>
__device__ void dispatch_body(const DispatchArgs& a, const int32_t* ids, const int32_t* err_tok,
                              int (*s_wbase)[EMAX], int* s_off, int* s_tmp, int* s_err) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.K, S = a.T * a.K;

  for (int i = tid; i < NW * E; i += NT) s_wbase[i / E][i % E] = 0;
  if (tid == 0) *s_err = 0;
  for (int p = tid; p < a.shared_rows; p += NT) a.row_token[p] = p;
  __syncthreads();

  // each wave owns one contiguous segment of the slots (keeps the sort stable); the ids
  // of kDispatchBatch chunks of 64 slots are loaded together so that their latencies
  // overlap
  const int seg = (S + NW - 1) / NW;
  const int sb = wave * seg, se = min(S, sb + seg);
  int err = 0;
  for (int c0 = sb; c0 < se; c0 += kDispatchBatch * kWave) {
    int ev[kDispatchBatch];
#pragma unroll
    for (int j = 0; j < kDispatchBatch; ++j) {
      const int s = c0 + j * kWave + lane;
      ev[j] = s < se ? ids[s] : -1;
    }
#pragma unroll
    for (int j = 0; j < kDispatchBatch; ++j) {
      if (c0 + j * kWave >= se) break;  // past the segment (wave-uniform)
      const int s = c0 + j * kWave + lane;
      const int e = ev[j];
      if (s < se) {
        if (e >= 0 && e < E) atomicAdd(&s_wbase[wave][e], 1);
        else if (!(err_tok && e == -1) && !(e >= E && e < E + a.zero)) err |= 1;
      }
    }
  }
  if (err_tok)
    for (int t = tid; t < a.T; t += NT) err |= err_tok[t];
  if (err) atomicOr(s_err, err);
  __syncthreads();

  // per expert: base of each wave's segment inside the group, and the group size
  int cnt = 0;
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = s_wbase[w][tid];
      s_wbase[w][tid] = run;
      run += c;
    }
    cnt = run;
  }
  int total = 0;
  const int off = block_exclusive_scan<NW>(cnt, s_tmp, &total);
  if (tid < E) s_off[tid] = a.shared_rows + off;
  __syncthreads();

  // stable scatter: lanes with equal ids are ranked by lane order within each chunk
  scatter_segment(a, ids, sb, se, s_wbase[wave], s_off);

  // tile list: ceil(cnt / tile_h) runs per expert, experts in order
  int ntot = 0;
  write_tiles<NW>(a, cnt, s_off, s_tmp, &ntot);
  if (tid == 0) {
    publish_tile_count(a.ntiles, ntot);
    a.err_word[0] = *s_err;
  }
}

}  // namespace moe
