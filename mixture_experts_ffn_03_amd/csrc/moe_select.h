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
// Selection keys: a 64-bit composite (order-preserving key bits << 32 | ~index), so the
// largest composite is the largest key, equal keys go to the lower expert index, -0 ==
// +0, and NaN ranks below -inf. 0 is below every real composite (padding).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_key(float f) {
  if (f != f) return 0u;         // NaN: below everything
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(float key, int idx) {
  return ((uint64_t)ordered_key(key) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Wave-wide maximum (result in every lane): DPP swaps inside each row of 16 lanes (quad
// swaps, then the half-row and row mirrors), then the four row results are read out.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
  uint64_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * i);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * i);
    r[i] = ((uint64_t)hi << 32) | lo;
  }
  return max_u64(max_u64(r[0], r[1]), max_u64(r[2], r[3]));
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
// per lane). Selection is k rounds of a wave-wide arg-max on the composite. s_logit
// (>= E floats), s_id and s_w (>= K) are this wave's LDS scratch. Writes ids / w (and
// logits_out, err_tok) to global memory; lds_ids (if not null) also receives ids[t*K..].
// ---------------------------------------------------------------------------
template <int NPL>
__device__ __forceinline__ void topk_token(const TopkArgs& a, int t, float* s_logit, int* s_id,
                                           float* s_w, int32_t* lds_ids, int32_t* lds_err) {
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
      if (a.logits_out) a.logits_out[(size_t)t * E + e] = lg[i];
      s_logit[e] = lg[i];
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
  if (a.score == 0 || a.score == 3) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) m = fmaxf(m, lg[i]);
    m = wave_max(m);
  }
  if (a.score == 0) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < E) S += expf(lg[i] - m);
    S = wave_sum(S);
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
    uint64_t comp[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) comp[i] = lane + kWave * i < E ? composite(key[i], lane + kWave * i) : 0ull;
    for (int j = 0; j < K; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) best = max_u64(best, comp[i]);
      const uint64_t g = wave_max_u64(best);
      const int idx = (int)(0xFFFFFFFFu - (uint32_t)g);
      if ((idx & 63) == lane) {
#pragma unroll
        for (int i = 0; i < NPL; ++i)
          if (i == (idx >> 6)) comp[i] = 0;  // taken
      }
      if (lane == j) my_id = idx;
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
  (void)s_id;
  (void)s_w;
  __builtin_amdgcn_wave_barrier();  // s_logit written by every lane above
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // weights of the selected experts, one slot per lane, then the (optional) normalisation
  float wj = 0.f;
  if (lane < K && my_id >= 0) {
    const float l = s_logit[my_id];
    wj = a.score == 0   ? expf(l - m) / S
         : a.score == 3 ? (float)(exp((double)l - (double)m) / S64)
                        : (float)score_f64(a.score, l);
  }
  if (a.renorm) {
    const float sum = wave_sum(wj);
    wj = sum > 0.f ? wj / sum : 0.f;
  }
  if (lane < K) {
    a.w[(size_t)t * K + lane] = wj * a.scaling;
    a.ids[(size_t)t * K + lane] = my_id;
    if (lds_ids) lds_ids[t * K + lane] = my_id;
  }
  if (lane == 0) {
    if (a.err_tok) a.err_tok[t] = err;
    if (lds_err) lds_err[t] = err;
  }
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

// Dispatch of at most 64 slots (few tokens) by one wave, lane = slot: the same row space,
// tile list and error bits as dispatch_body, from ranks found by comparing every pair of
// slots (key = expert * 64 + slot: the stable order by expert, then token and slot).
// s_tok: 64 ints of LDS (tokens of the rows in rank order).
__device__ void dispatch_small(const DispatchArgs& a, const int32_t* ids, const int32_t* err_tok,
                               int* s_tok) {
  constexpr int kNone = 0x7fffffff;
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K, S = a.T * a.K;
  const bool in = lane < S;
  const int e = in ? ids[lane] : -1;
  const bool valid = in && e >= 0 && e < E;
  const bool zero = in && e >= E && e < E + a.zero;
  int err = (in && !valid && !zero && !(err_tok && e == -1)) ? 1 : 0;
  if (err_tok && lane < a.T) err |= err_tok[lane];
  if (lane < a.shared_rows) a.row_token[lane] = lane;  // shared_rows = T <= 64
  const int key = valid ? e * kWave + lane : kNone;
  int rank = 0, rexp = 0, cexp = 0;  // rows before mine; of my expert before mine; of my expert
  for (int j = 0; j < S; ++j) {  // lanes past S hold no slot
    const int kj = __builtin_amdgcn_readlane(key, j);
    const bool same = kj != kNone && (kj / kWave) == e;
    rank += kj < key;
    rexp += same && kj < key;
    cexp += same;
  }
  const int pos = a.shared_rows + rank;
  if (valid) {
    a.row_token[pos] = lane / K;
    a.inv[lane] = pos;
    s_tok[rank] = lane / K;
  } else if (in) {
    a.inv[lane] = zero ? -2 : -1;
  }
  const int h = a.tile_h;
  const bool start = valid && rexp % h == 0;
  const uint64_t smask = __ballot(start);
  int tidx = 0;  // tiles that start before mine
  for (int j = 0; j < S; ++j) {
    const int kj = __builtin_amdgcn_readlane(key, j);
    tidx += ((smask >> j) & 1) && kj < key;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (start) {
    Tile tl;
    tl.group = e;
    tl.row0 = pos;
    tl.count = min(h, cexp - rexp);
    tl.pad = 0;
#pragma unroll
    for (int q = 0; q < kTileTok; ++q)
      tl.tok[q] = (h <= kTileTok && q < tl.count) ? s_tok[rank + q] : 0;
    a.tiles[tidx] = tl;
  }
  int errbits = err;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) errbits |= __shfl_xor(errbits, m, kWave);
  if (lane == 0) {
    a.ntiles[0] = __popcll(smask);
    a.err_word[0] = errbits;
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
    a.ntiles[0] = ntot;
    a.err_word[0] = *s_err;
  }
}

}  // namespace moe
