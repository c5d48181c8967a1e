// Routing kernels: pre-expert RMSNorm, router GEMM, scores + top-K selection.
//
// Router (MoE constructor page, spark_model/layers/moe/init.rs: the fp32-output router
// GEMM and the softmax / sigmoid-with-bias / hash top-K kernels; MoE module page,
// spark_model/layers/moe/mod.rs: docs of dense_gemm_f32out, correction_bias_dev and
// tid2eid_dev).
//
// Logits are fp32(x . W_r^T + bias). The products of two bf16 values are exact, and the
// kernel sums them in fp64, so the fp32 logit is the correctly rounded dot product in all
// but vanishingly rare cases, whatever the summation order. That makes the expert choice
// reproducible against any exact evaluation, which a plain fp32 accumulation (order-
// dependent in the last bit) cannot promise at near-ties.
#include "moe_select.h"

namespace moe {

// ---------------------------------------------------------------------------
// RMSNorm: out = bf16(x * rsqrt(mean(x^2) + eps) * gamma), one block per token
// (MoE module page, doc of MoeLayer.pre_expert_norm: the experts see the normalised
// input, the router the raw one).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ gamma,
                                                 uint16_t* __restrict__ out, int H, float eps) {
  // 16-byte pieces (8 values; H is a multiple of 32), the second pass re-reading the row
  // from the cache
  const int t = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  const uint4* gr = reinterpret_cast<const uint4*>(gamma);
  uint4* orow = reinterpret_cast<uint4*>(out + (size_t)t * H);
  const int np = H / 8;
  float ss = 0.f;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const uint4 q = xr[i];
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_to_f32(d[j] & 0xFFFFu), hi = bf16_to_f32(d[j] >> 16);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const uint4 q = xr[i], g = gr[i];
    const uint32_t d[4] = {q.x, q.y, q.z, q.w}, e[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = (bf16_to_f32(d[j] & 0xFFFFu) * r) * bf16_to_f32(e[j] & 0xFFFFu);
      const float hi = (bf16_to_f32(d[j] >> 16) * r) * bf16_to_f32(e[j] >> 16);
      o[j] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
    }
    orow[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, uint16_t* out, int T, int H,
                          float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, s, x, gamma, out, H, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router GEMM, fp64 sums: partial[z][t][e] = sum_{h in slice z} x[t,h] * W_r[e,h], on
// the fp64 matrix cores. A block computes 16 experts x MF 16-token fragments (a tile of
// up to 64 tokens; blockIdx.y walks the token tiles) over one H slice with
// v_mfma_f64_16x16x4_f64 on exactly widened bf16 operands; its four waves take
// interleaved 32-wide K chunks and are summed in a fixed order at the end. H is split
// over blocks so that the grid fills the chip (z = slice).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bf16x8_to_f64(const uint4& v, double (&o)[8]) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (double)bf16_to_f32(d[i] & 0xFFFFu);
    o[2 * i + 1] = (double)bf16_to_f32(d[i] >> 16);
  }
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// MF 16-token fragments x NE 16-expert groups. MFMA operand layout (16x16x4 f64): lane l
// holds A[l % 16][l / 16] and B[l / 16][l % 16]; the result D[l / 16 + 4 v][l % 16] sits in
// element v. The K index of (lane quad q, step s) inside a 32-wide chunk is 8q + s for both
// operands. Each widened token operand feeds NE MFMAs, each widened expert operand MF.
template <int MF, int NE>
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w,
                                                     double* __restrict__ partial, int T, int E,
                                                     int H, int hsplit) {
  __shared__ f64x4_t s_red[3][NE][MF][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int idx = lane & 15, q = lane >> 4;
  const int e0 = blockIdx.x * 16 * NE;
  const int tb = blockIdx.y * 16 * MF;  // first token of the tile
  const int kb = blockIdx.z * hsplit;
  const int ke = min(H, kb + hsplit);
  const uint16_t* wrow[NE];
#pragma unroll
  for (int g = 0; g < NE; ++g) {
    const int e = e0 + 16 * g + idx;
    wrow[g] = w + (size_t)(e < E ? e : 0) * H + 8 * q;  // rows past E: results not stored
  }
  const uint16_t* xrow[MF];
  bool tv[MF];
#pragma unroll
  for (int m = 0; m < MF; ++m) {
    const int t = tb + m * 16 + idx;
    tv[m] = t < T;
    xrow[m] = x + (size_t)(tv[m] ? t : 0) * H + 8 * q;
  }
  // with at most two accumulators per wave (few tokens), odd chunks add into a second set,
  // halving the dependent MFMA chain; the two are added once at the end
  constexpr int NALT = MF * NE <= 2 ? 2 : 1;
  f64x4_t acc[NE][MF], accb[NE][MF];
#pragma unroll
  for (int g = 0; g < NE; ++g)
#pragma unroll
    for (int m = 0; m < MF; ++m) acc[g][m] = accb[g][m] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  // the operands of the wave's next two 32-wide chunks are in flight while the current
  // chunk's MFMAs run (one chunk ahead is shorter than a loaded HBM round trip)
  const int kstart = kb + 32 * wave;
  uint4 wv[NE], w1[NE], xv[MF], x1[MF];
#pragma unroll
  for (int g = 0; g < NE; ++g) wv[g] = w1[g] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int m = 0; m < MF; ++m) xv[m] = x1[m] = make_uint4(0, 0, 0, 0);
  // (unconditional loads: rows past T read row 0 and are zeroed after the load; the
  // prefetches past the slice re-read the current chunk)
  auto load = [&](int k0, uint4 (&w_)[NE], uint4 (&x_)[MF]) {
#pragma unroll
    for (int g = 0; g < NE; ++g) w_[g] = *reinterpret_cast<const uint4*>(wrow[g] + k0);
#pragma unroll
    for (int m = 0; m < MF; ++m) x_[m] = *reinterpret_cast<const uint4*>(xrow[m] + k0);
  };
  if (kstart < ke) {
    load(kstart, wv, xv);
    load(kstart + 128 < ke ? kstart + 128 : kstart, w1, x1);
  }
  for (int k0 = kstart, odd = 0; k0 < ke; k0 += 128, odd ^= 1) {
    uint4 wn[NE], xn[MF];
    load(k0 + 256 < ke ? k0 + 256 : k0, wn, xn);
    double xd[MF][8];
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const uint4 v = tv[m] ? xv[m] : make_uint4(0, 0, 0, 0);
      bf16x8_to_f64(v, xd[m]);
    }
#pragma unroll
    for (int g = 0; g < NE; ++g) {
      double wd[8];
      bf16x8_to_f64(wv[g], wd);
      if (NALT == 2 && odd) {
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
          for (int m = 0; m < MF; ++m)
            accb[g][m] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[m][st], wd[st], accb[g][m], 0, 0, 0);
      } else {
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
          for (int m = 0; m < MF; ++m)
            acc[g][m] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[m][st], wd[st], acc[g][m], 0, 0, 0);
      }
    }
#pragma unroll
    for (int g = 0; g < NE; ++g) {
      wv[g] = w1[g];
      w1[g] = wn[g];
    }
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      xv[m] = x1[m];
      x1[m] = xn[m];
    }
  }
  if (NALT == 2) {
#pragma unroll
    for (int g = 0; g < NE; ++g)
#pragma unroll
      for (int m = 0; m < MF; ++m) acc[g][m] += accb[g][m];
  }
  if (wave > 0) {
#pragma unroll
    for (int g = 0; g < NE; ++g)
#pragma unroll
      for (int m = 0; m < MF; ++m) s_red[wave - 1][g][m][lane] = acc[g][m];
  }
  __syncthreads();
  if (wave != 0) return;
  double* p = partial + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int g = 0; g < NE; ++g) {
    const int e = e0 + 16 * g + idx;
    if (e >= E) continue;
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const f64x4_t sum =
          ((acc[g][m] + s_red[0][g][m][lane]) + s_red[1][g][m][lane]) + s_red[2][g][m][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = tb + m * 16 + q + 4 * v;
        if (t < T) p[(size_t)t * E + e] = sum[v];
      }
    }
  }
}

// 16-expert groups per block: two once a block has four 16-token fragments and the experts
// fill them (the prefill router), else one.
#ifndef MOE_ROUTER_NE
#define MOE_ROUTER_NE 2
#endif
static int router_ne(int T, int E) { return (T >= 64 && E >= 32) ? MOE_ROUTER_NE : 1; }

RouterPlan plan_router(int T, int E, int H) {
  RouterPlan r;
  // enough H slices that the grid has about 512 blocks (two per CU)
  const int ge = 16 * router_ne(T, E);
  const int blocks = max(1, ((E + ge - 1) / ge) * ((T + 63) / 64));  // T = 0: no launch
  int ks = min((512 + blocks - 1) / blocks, min(kRouterMaxSplit, H / 32));
  ks = max(ks, 1);
  r.hsplit = ((H + ks - 1) / ks + 31) / 32 * 32;  // whole 32-wide chunks
  r.ks = (H + r.hsplit - 1) / r.hsplit;
  return r;
}

hipError_t launch_router_partial(const uint16_t* x, const uint16_t* w, double* partial, int T,
                                 int E, int H, int ks, int hsplit, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int mf = T >= 64 ? 4 : (T + 15) / 16;  // 16-token fragments per block
  const int ne = router_ne(T, E);
  const dim3 grid((E + 16 * ne - 1) / (16 * ne), (T + 16 * mf - 1) / (16 * mf), ks);
  if (mf == 1) hipLaunchKernelGGL((k_router_mfma<1, 1>), grid, dim3(256), 0, s, x, w, partial, T, E, H, hsplit);
  else if (mf == 2) hipLaunchKernelGGL((k_router_mfma<2, 1>), grid, dim3(256), 0, s, x, w, partial, T, E, H, hsplit);
  else if (mf == 3) hipLaunchKernelGGL((k_router_mfma<3, 1>), grid, dim3(256), 0, s, x, w, partial, T, E, H, hsplit);
  else if (ne == 2) hipLaunchKernelGGL((k_router_mfma<4, 2>), grid, dim3(256), 0, s, x, w, partial, T, E, H, hsplit);
  else hipLaunchKernelGGL((k_router_mfma<4, 1>), grid, dim3(256), 0, s, x, w, partial, T, E, H, hsplit);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scores + top-K: one wavefront per token (topk_token), kTopkWaves tokens per block.
// ---------------------------------------------------------------------------
constexpr int kTopkWaves = 4;

template <int NPL>
__global__ __launch_bounds__(256) void k_topk(TopkArgs a) {
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= a.T) return;  // whole wavefronts exit together
  topk_token<NPL>(a, t, nullptr, nullptr);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + kTopkWaves - 1) / kTopkWaves), block(64 * kTopkWaves);
  const int npl = (a.E + 63) / 64;
  if (npl <= 1) hipLaunchKernelGGL(k_topk<1>, grid, block, 0, s, a);
  else if (npl <= 2) hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, a);
  else if (npl <= 4) hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, a);
  else if (npl <= 8) hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_topk<16>, grid, block, 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Hash routing whose weights need only the selected experts' logits (sigmoid or
// sqrt-softplus scores, or a renormalised softmax, where the normaliser over all experts
// cancels), when no logits are asked for: one block per token reads its k experts from the
// table and forms just those k router dot products, one wave per slot (fp64 over H, each
// lane 8 columns per step, then a wave reduction; rounded to fp32 once with the logit bias, as the full
// router's logits are), instead of the router GEMM over every expert (hidden a multiple of
// 512, at most 4096). The weights follow the
// hash branch of topk_token, the softmax taken over the selected experts (the renormalised
// weights are the same). Error bits as topk_token's.
// ---------------------------------------------------------------------------
constexpr int kGatherSteps = 8;  // steps of 512 columns: hidden sizes up to 4096
constexpr int kGatherWaves = 8;  // one block per token; wave w takes slots w, w + 8, ...

__global__ __launch_bounds__(kGatherWaves * 64) void k_hash_gather(TopkArgs a,
                                                                  const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  int H) {
  __shared__ int s_id[kMaxTopK];
  __shared__ float s_l[kMaxTopK];
  __shared__ int s_err;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int E = a.E, K = a.K;
  // the token's row in registers (8 columns per lane and step of 512), requested first
  const int ns = H / (kWave * 8);
  const uint16_t* xr = x + (size_t)t * H + lane * 8;
  uint4 xv[kGatherSteps];
#pragma unroll
  for (int q = 0; q < kGatherSteps; ++q)
    if (q < ns) xv[q] = *reinterpret_cast<const uint4*>(xr + q * kWave * 8);
  if (wave == 0) {  // the slots' experts from the table
    const int64_t tok = a.token_ids[t];
    const bool tok_ok = tok >= 0 && tok < a.vocab;
    int err = tok_ok ? 0 : 2;
    int my_id = -1;
    if (lane < K && tok_ok) {
      const int64_t e = a.tid2eid[tok * K + lane];
      if (e >= 0 && e < E) my_id = (int)e;
      else err |= 4;
    }
    if (lane < K) s_id[lane] = my_id;
    // (the ballot over the whole wave: a table error sits in the lane of its slot)
    const int werr = __builtin_amdgcn_readfirstlane(err) | (int)(__ballot(err & 4) ? 4 : 0);
    if (lane == 0) s_err = werr;
  }
  __syncthreads();
  // slot j's dot product: every step's weight piece requested at once, fp64 sums, a wave
  // reduction, one rounding to fp32 with the logit bias
  for (int j = wave; j < K; j += kGatherWaves) {
    const int e = s_id[j];
    if (e < 0) continue;  // (wave-uniform) a dropped slot has no logit
    const uint16_t* er = wr + (size_t)e * H + lane * 8;
    uint4 wv[kGatherSteps];
#pragma unroll
    for (int q = 0; q < kGatherSteps; ++q)
      if (q < ns) wv[q] = *reinterpret_cast<const uint4*>(er + q * kWave * 8);
    double acc = 0.0;
#pragma unroll
    for (int q = 0; q < kGatherSteps; ++q) {
      if (q >= ns) break;
      double xd[8], wd[8];
      bf16x8_to_f64(xv[q], xd);
      bf16x8_to_f64(wv[q], wd);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fma(xd[i], wd[i], acc);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
    if (a.logit_bias) acc += (double)a.logit_bias[e];
    if (lane == 0) s_l[j] = (float)acc;
  }
  __syncthreads();
  if (wave != 0) return;
  const int my_id = lane < K ? s_id[lane] : -1;
  const bool sel = my_id >= 0;
  const float l = sel ? s_l[lane] : 0.f;
  float wj = 0.f;
  if (a.score == 0) {  // softmax over the selected experts (renormalised: as over all)
    float m = sel ? l : -__builtin_inff();
    m = wave_max_dpp(m);
    const float p = sel ? expf(l - m) : 0.f;
    const float S = wave_sum_dpp(p);
    wj = sel ? p / S : 0.f;
  } else if (sel) {
    wj = (float)score_f64(a.score, l);
  }
  if (a.renorm) {
    const float sum = wave_sum_dpp(wj);
    wj = sum > 0.f ? wj / sum : 0.f;
  }
  if (lane < K) {
    a.w[(size_t)t * K + lane] = wj * a.scaling;
    a.ids[(size_t)t * K + lane] = my_id;
  }
  if (lane == 0 && a.err_tok) a.err_tok[t] = s_err;
}

bool hash_gather_fits(const TopkArgs& a, int H) {
  return a.select == 1 && !a.logits_out && !a.logits_in && H % (kWave * 8) == 0 &&
         H <= kGatherSteps * kWave * 8 &&
         (a.score == 1 || a.score == 2 || (a.score == 0 && a.renorm));
}

hipError_t launch_hash_gather(const TopkArgs& a, const uint16_t* x, const uint16_t* w, int H,
                              hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_hash_gather, dim3(a.T), dim3(kGatherWaves * 64), 0, s, a, x, w, H);
  return hipGetLastError();
}

}  // namespace moe
