// Dispatch build: groups the (token, slot) pairs of the routing by expert on the device,
// with no host synchronisation (MoE module page, module doc: indices and weights stay on
// the device; constructor page: the sort-by-expert and tile work-list kernels of the
// grouped prefill path).
//
// Row space: when a shared expert is present its T rows come first (row t = token t),
// then the routed groups in expert order, each group's rows in (token, slot) order
// (a stable counting sort). Outputs:
//   row_token[p]  token whose input feeds row p
//   inv[t*K + j]  row of slot (t, j), or -1 if its id is outside [0, E)
//   tiles         (expert, first row, row count) runs of at most tile_h rows
//   ntiles        number of tiles
//   err_word      MOE_DEVERR_* bits of this call
#include "moe_select.h"

namespace moe {

constexpr int kDispatchThreads = 1024;
constexpr int kDispatchWaves = kDispatchThreads / kWave;

__global__ __launch_bounds__(kDispatchThreads) void k_dispatch(DispatchArgs a) {
  __shared__ int s_wbase[kDispatchWaves][kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_tmp[2 * kDispatchWaves + 1];
  __shared__ int s_err;
  dispatch_body<kDispatchWaves, kMaxExperts>(a, a.ids, a.err_tok, s_wbase, s_off, s_tmp, &s_err);
}

// At most one slot per thread whose experts' bitmaps (E x ceil(S / 64) words, the dynamic
// LDS of the launch) fit kBitmapMaxLds: the bitmap dispatch on ids in memory.
constexpr size_t kBitmapMaxLds = 48 * 1024;

__global__ __launch_bounds__(kDispatchThreads) void k_dispatch_bitmap(DispatchArgs a) {
  extern __shared__ uint64_t s_mask[];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_toff[kMaxExperts];
  __shared__ int s_tot[kDispatchWaves];
  __shared__ int s_err;
  const int n = a.E * ((a.T * a.K + 63) / 64);
  for (int i = threadIdx.x; i < n; i += kDispatchThreads) s_mask[i] = 0ull;
  if (threadIdx.x == 0) s_err = 0;
  __syncthreads();
  dispatch_bitmap<kDispatchWaves, kMaxExperts>(a, a.ids, a.err_tok, s_mask, s_off, s_toff, s_tot,
                                               &s_err);
}

// ---------------------------------------------------------------------------
// Many slots: the same counting sort over blocks of kDispChunk slots (16 waves, one chunk
// of 64 slots each). Launch 1 counts each block's slots per expert (and ORs the error bits
// of its slots and of its share of the tokens) into cntb [E, blocks] (expert-major, blocks
// rounded up to a multiple of 4; the extra blocks count nothing). Launch 2: each block
// sums the counts of the blocks before it and of all blocks per expert, recounts its own
// waves' slots for their places inside the block, and scatters; its block 0 writes the
// tile list, the tile count and the error word.
// ---------------------------------------------------------------------------
constexpr int kDispSeg = kDispChunk / kDispatchWaves;  // slots per wave (one chunk)
static_assert(kDispSeg == kWave, "one chunk of 64 slots per wave");

// per-wave expert counts of this block's slots into s_wc (zeroed here); returns error bits
__device__ __forceinline__ int count_block_slots(const DispatchArgs& a, int (*s_wc)[kMaxExperts]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, S = a.T * a.K;
  for (int i = tid; i < kDispatchWaves * E; i += kDispatchThreads) s_wc[i / E][i % E] = 0;
  __syncthreads();
  const int s = blockIdx.x * kDispChunk + wave * kDispSeg + lane;
  const int e = s < S ? a.ids[s] : -1;
  int err = 0;
  if (s < S) {
    if (e >= 0 && e < E) atomicAdd(&s_wc[wave][e], 1);
    else if (!(a.err_tok && e == -1) && !(e >= E && e < E + a.zero)) err |= 1;
  }
  __syncthreads();
  return err;
}

__global__ __launch_bounds__(kDispatchThreads) void k_dispatch_count(DispatchArgs a) {
  __shared__ int s_wc[kDispatchWaves][kMaxExperts];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0;
  int err = count_block_slots(a, s_wc);
  if (a.err_tok) {  // this block's share of the tokens
    const int tpb = (a.T + gridDim.x - 1) / gridDim.x;
    const int t1 = min(a.T, (int)(blockIdx.x + 1) * tpb);
    for (int t = blockIdx.x * tpb + tid; t < t1; t += kDispatchThreads) err |= a.err_tok[t];
  }
  if (err) atomicOr(&s_err, err);
  if (tid < a.E) {
    int c = 0;
    for (int w = 0; w < kDispatchWaves; ++w) c += s_wc[w][tid];
    a.wcnt[(size_t)tid * gridDim.x + blockIdx.x] = c;
  }
  __syncthreads();
  if (tid == 0) a.err_part[blockIdx.x] = s_err;
}

__global__ __launch_bounds__(kDispatchThreads) void k_dispatch_scatter(DispatchArgs a) {
  __shared__ int s_wc[kDispatchWaves][kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_tmp[2 * kDispatchWaves + 1];
  __shared__ int s_err;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int E = a.E, S = a.T * a.K;
  const int nb = gridDim.x;  // a multiple of 4
  // block 0: the error bits of every block of the count launch, requested up front and
  // OR-ed over the block (one load per thread, not a loop of dependent loads)
  int perr = 0;
  if (blockIdx.x == 0) {
    if (tid == 0) s_err = 0;
    for (int b = tid; b < nb; b += kDispatchThreads) perr |= a.err_part[b];
  }
  // per expert: rows of the blocks before this one, and the group size
  int cnt = 0, before = 0;
  if (tid < E) {
    const uint4* row = reinterpret_cast<const uint4*>(a.wcnt + (size_t)tid * nb);
    for (int b = 0; b < nb; b += 32) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = b + 4 * j < nb ? row[b / 4 + j] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c4[4] = {(int)v[j].x, (int)v[j].y, (int)v[j].z, (int)v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (b + 4 * j + q == (int)blockIdx.x) before = cnt;
          cnt += c4[q];
        }
      }
    }
  }
  int total = 0;
  const int off = block_exclusive_scan<kDispatchWaves>(cnt, s_tmp, &total);
  count_block_slots(a, s_wc);  // (synchronises the block)
  if (tid < E) {
    s_off[tid] = a.shared_rows + off;
    int run = before;  // this block's waves, in order
    for (int w = 0; w < kDispatchWaves; ++w) {
      const int c = s_wc[w][tid];
      s_wc[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  const int sb = blockIdx.x * kDispChunk + wave * kDispSeg, se = min(S, sb + kDispSeg);
  scatter_segment(a, a.ids, sb, se, s_wc[wave], s_off);
  if (blockIdx.x != 0) return;
  for (int p = tid; p < a.shared_rows; p += kDispatchThreads) a.row_token[p] = p;
  if (perr) atomicOr(&s_err, perr);  // (s_err was zeroed before the block's first barrier)
  int ntot = 0;
  write_tiles<kDispatchWaves>(a, cnt, s_off, s_tmp, &ntot);  // prefill tiles: no tokens read
  __syncthreads();
  if (tid == 0) {
    publish_tile_count(a.ntiles, ntot);
    a.err_word[0] = s_err;
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int S = a.T * a.K;
  if (dispatch_multi_block(S, a.tile_h)) {
    const int blocks = dispatch_blocks(S);
    hipLaunchKernelGGL(k_dispatch_count, dim3(blocks), dim3(kDispatchThreads), 0, s, a);
    hipLaunchKernelGGL(k_dispatch_scatter, dim3(blocks), dim3(kDispatchThreads), 0, s, a);
    return hipGetLastError();
  }
  const size_t mask_bytes = (size_t)a.E * ((S + 63) / 64) * sizeof(uint64_t);
  if (S <= kDispatchThreads && mask_bytes <= kBitmapMaxLds) {
    hipLaunchKernelGGL(k_dispatch_bitmap, dim3(1), dim3(kDispatchThreads), mask_bytes, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kDispatchThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-K and dispatch in one block, for few tokens and experts: the block's waves select
// the experts of the tokens (topk_token, ids kept in LDS), then sort the slots by expert
// (dispatch_bitmap).
// Saves a launch and a round trip of the ids through memory.
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 16;
static_assert(kFusedMaxSlots <= kFusedWaves * 64, "one thread per slot");

template <int NPL>
__global__ __launch_bounds__(kFusedWaves * 64) void k_topk_dispatch(TopkArgs ta, DispatchArgs da) {
  constexpr int kWords = kFusedMaxSlots / 64;
  __shared__ uint64_t s_mask[kFusedMaxExperts * kWords];
  __shared__ int32_t s_ids[kFusedMaxSlots];
  __shared__ int32_t s_errt[kFusedMaxTokens];
  __shared__ int s_off[kFusedMaxExperts];
  __shared__ int s_toff[kFusedMaxExperts];
  __shared__ int s_tot[kFusedWaves];
  __shared__ int s_err;
  const int wave = threadIdx.x >> 6;
  const int S = da.T * da.K;
  {  // clear the bitmaps while the waves select
    const int nw = da.E * ((S + 63) / 64);
    for (int i = threadIdx.x; i < nw; i += kFusedWaves * 64) s_mask[i] = 0ull;
    if (threadIdx.x == 0) s_err = 0;
  }
  for (int t = wave; t < ta.T; t += kFusedWaves) topk_token<NPL>(ta, t, s_ids, s_errt);
  __syncthreads();
  dispatch_bitmap<kFusedWaves, kFusedMaxExperts>(da, s_ids, s_errt, s_mask, s_off, s_toff, s_tot,
                                                &s_err);
}

bool fused_topk_dispatch_fits(int T, int E, int K) {
  return T <= kFusedMaxTokens && E <= kFusedMaxExperts && T * K <= kFusedMaxSlots;
}

hipError_t launch_topk_dispatch(const TopkArgs& ta, const DispatchArgs& da, hipStream_t s) {
  const int npl = (ta.E + 63) / 64;
  const dim3 grid(1), block(kFusedWaves * 64);
  if (npl <= 1) hipLaunchKernelGGL(k_topk_dispatch<1>, grid, block, 0, s, ta, da);
  else if (npl <= 2) hipLaunchKernelGGL(k_topk_dispatch<2>, grid, block, 0, s, ta, da);
  else hipLaunchKernelGGL(k_topk_dispatch<4>, grid, block, 0, s, ta, da);
  return hipGetLastError();
}

}  // namespace moe
