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
  if (a.T * a.K <= kSmallDispatchSlots) {  // few slots: one wave
    if (threadIdx.x < kWave) dispatch_small(a, a.ids, a.err_tok, s_wbase[0]);
    return;
  }
  dispatch_body<kDispatchWaves, kMaxExperts>(a, a.ids, a.err_tok, s_wbase, s_off, s_tmp, &s_err);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kDispatchThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-K and dispatch in one block, for few tokens and experts: the block's waves select
// the experts of the tokens (topk_token, ids kept in LDS), then sort the slots by expert
// (dispatch_body). Saves a launch and a round trip of the ids through memory.
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 16;

template <int NPL>
__global__ __launch_bounds__(kFusedWaves * 64) void k_topk_dispatch(TopkArgs ta, DispatchArgs da) {
  __shared__ float s_logit[kFusedWaves][kFusedMaxExperts];
  __shared__ int s_id[kFusedWaves][kMaxTopK];
  __shared__ float s_w[kFusedWaves][kMaxTopK];
  __shared__ int32_t s_ids[kFusedMaxSlots];
  __shared__ int32_t s_errt[kFusedMaxTokens];
  __shared__ int s_wbase[kFusedWaves][kFusedMaxExperts];
  __shared__ int s_off[kFusedMaxExperts];
  __shared__ int s_tmp[2 * kFusedWaves + 1];
  __shared__ int s_err;
  const int wave = threadIdx.x >> 6;
  for (int t = wave; t < ta.T; t += kFusedWaves)
    topk_token<NPL>(ta, t, s_logit[wave], s_id[wave], s_w[wave], s_ids, s_errt);
  __syncthreads();
  if (da.T * da.K <= kSmallDispatchSlots) {  // few slots: one wave
    if (wave == 0) dispatch_small(da, s_ids, s_errt, s_wbase[0]);
    return;
  }
  dispatch_body<kFusedWaves, kFusedMaxExperts>(da, s_ids, s_errt, s_wbase, s_off, s_tmp, &s_err);
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
