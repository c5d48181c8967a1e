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
#include "moe_device.h"

namespace moe {

constexpr int kDispatchThreads = 1024;
constexpr int kDispatchWaves = kDispatchThreads / kWave;

// Exclusive prefix sum of one int per thread over the block; *total gets the sum.
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
    const int w = lane < kDispatchWaves ? s_tmp[lane] : 0;
    int inc = w;
#pragma unroll
    for (int d = 1; d < kDispatchWaves; d <<= 1) {
      const int y = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += y;
    }
    if (lane < kDispatchWaves) s_tmp[kDispatchWaves + lane] = inc - w;
    if (lane == kDispatchWaves - 1) s_tmp[2 * kDispatchWaves] = inc;
  }
  __syncthreads();
  const int r = x - v + s_tmp[kDispatchWaves + wave];
  *total = s_tmp[2 * kDispatchWaves];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kDispatchThreads) void k_dispatch(DispatchArgs a) {
  __shared__ int s_wbase[kDispatchWaves][kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_tmp[2 * kDispatchWaves + 1];
  __shared__ int s_err;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.K, S = a.T * a.K;

  for (int i = tid; i < kDispatchWaves * E; i += kDispatchThreads) s_wbase[i / E][i % E] = 0;
  if (tid == 0) s_err = 0;
  for (int p = tid; p < a.shared_rows; p += kDispatchThreads) a.row_token[p] = p;
  __syncthreads();

  // each wave owns one contiguous segment of the slots (keeps the sort stable)
  const int seg = (S + kDispatchWaves - 1) / kDispatchWaves;
  const int sb = wave * seg, se = min(S, sb + seg);
  int err = 0;
  for (int c0 = sb; c0 < se; c0 += kWave) {
    const int s = c0 + lane;
    if (s < se) {
      const int e = a.ids[s];
      if (e >= 0 && e < E) atomicAdd(&s_wbase[wave][e], 1);
      else if (!(a.err_tok && e == -1)) err |= 1;
    }
  }
  if (a.err_tok)
    for (int t = tid; t < a.T; t += kDispatchThreads) err |= a.err_tok[t];
  if (err) atomicOr(&s_err, err);
  __syncthreads();

  // per expert: base of each wave's segment inside the group, and the group size
  int cnt = 0;
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kDispatchWaves; ++w) {
      const int c = s_wbase[w][tid];
      s_wbase[w][tid] = run;
      run += c;
    }
    cnt = run;
  }
  int total = 0;
  const int off = block_exclusive_scan(cnt, s_tmp, &total);
  if (tid < E) s_off[tid] = a.shared_rows + off;
  __syncthreads();

  // stable scatter: lanes with equal ids are ranked by lane order within each chunk
  for (int c0 = sb; c0 < se; c0 += kWave) {
    const int s = c0 + lane;
    const bool in = s < se;
    const int e = in ? a.ids[s] : -1;
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
      const int base = s_wbase[wave][e];
      const int pos = s_off[e] + base + rank;
      a.row_token[pos] = s / K;
      a.inv[s] = pos;
      if (rank == cntm - 1) s_wbase[wave][e] = base + cntm;
    } else if (in) {
      a.inv[s] = -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // tile list: ceil(cnt / tile_h) runs per expert, experts in order
  const int h = a.tile_h;
  const int nt = (tid < E) ? (cnt + h - 1) / h : 0;
  int ntot = 0;
  const int toff = block_exclusive_scan(nt, s_tmp, &ntot);
  __syncthreads();  // row_token of every routed row is written (read back below)
  if (tid < E) {
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
  if (tid == 0) {
    a.ntiles[0] = ntot;
    a.err_word[0] = s_err;
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kDispatchThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
