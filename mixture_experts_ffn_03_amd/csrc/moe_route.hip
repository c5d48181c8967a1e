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
#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// RMSNorm: out = bf16(x * rsqrt(mean(x^2) + eps) * gamma), one block per token
// (MoE module page, doc of MoeLayer.pre_expert_norm: the experts see the normalised
// input, the router the raw one).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ gamma,
                                                 uint16_t* __restrict__ out, int H, float eps) {
  const int t = blockIdx.x;
  const uint16_t* xr = x + (size_t)t * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float v = bf16_to_f32(xr[i]);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* orow = out + (size_t)t * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    orow[i] = f32_to_bf16((bf16_to_f32(xr[i]) * r) * bf16_to_f32(gamma[i]));
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, uint16_t* out, int T, int H,
                          float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, s, x, gamma, out, H, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router GEMM, fp64 sums: partial[z][t][e] = sum_{h in slice z} x[t,h] * W_r[e,h].
//
// Few tokens (decode): one block per expert row. The block streams the row once with
// 16-byte loads, and every thread dots its chunks with each token's activations; the
// per-token sums are reduced across the block in a fixed order (one slice, z = 0).
//
// Many tokens (prefill): 64 tokens x 64 experts per block with a 4x4 fp64 register
// block per thread over LDS tiles, H split in z so that the grid fills the chip.
// ---------------------------------------------------------------------------
constexpr int kRowTok = 8;  // tokens per pass of the row kernel

__device__ __forceinline__ void bf16x8_to_f64(const uint4& v, double (&o)[8]) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (double)bf16_to_f32(d[i] & 0xFFFFu);
    o[2 * i + 1] = (double)bf16_to_f32(d[i] >> 16);
  }
}

__global__ __launch_bounds__(256) void k_router_rows(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w,
                                                     double* __restrict__ partial, int T, int E,
                                                     int H) {
  __shared__ double s_red[4][kRowTok];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nchunk = H / 8;
  const uint16_t* wrow = w + (size_t)e * H;
  for (int t0 = 0; t0 < T; t0 += kRowTok) {
    double acc[kRowTok];
#pragma unroll
    for (int t = 0; t < kRowTok; ++t) acc[t] = 0.0;
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      double wv[8];
      bf16x8_to_f64(*reinterpret_cast<const uint4*>(wrow + c * 8), wv);
#pragma unroll
      for (int t = 0; t < kRowTok; ++t) {
        if (t0 + t < T) {
          double xv[8];
          bf16x8_to_f64(*reinterpret_cast<const uint4*>(x + (size_t)(t0 + t) * H + c * 8), xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[t] = fma(xv[i], wv[i], acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kRowTok; ++t) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) acc[t] += __shfl_xor(acc[t], m, kWave);
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < kRowTok; ++t) s_red[wave][t] = acc[t];
    }
    __syncthreads();
    if (threadIdx.x < kRowTok && t0 + threadIdx.x < T) {
      const int t = threadIdx.x;
      partial[(size_t)(t0 + t) * E + e] = (s_red[0][t] + s_red[1][t]) + (s_red[2][t] + s_red[3][t]);
    }
    __syncthreads();
  }
}

constexpr int kRt = 64;   // tokens per block tile
constexpr int kRe = 64;   // experts per block tile
constexpr int kRk = 16;   // K per LDS stage

__global__ __launch_bounds__(256) void k_router_tiled(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w,
                                                      double* __restrict__ partial, int T, int E,
                                                      int H, int hsplit) {
  __shared__ __align__(16) double xs[kRk][kRt + 2];
  __shared__ __align__(16) double ws[kRk][kRe + 2];
  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * kRe, t0 = blockIdx.y * kRt;
  const int kb = blockIdx.z * hsplit;
  const int ke = min(H, kb + hsplit);
  const int tx = tid & 15, ty = tid >> 4;  // experts 4*tx.., tokens 4*ty..
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  // loader: threads 0..127 load x rows, 128..255 W rows; 16 k = two 16-byte pieces per row
  const int lrow = (tid & 127) >> 1, lpiece = tid & 1;
  const bool lx = tid < 128;
  for (int k0 = kb; k0 < ke; k0 += kRk) {
    double v[8];
    const int k = k0 + lpiece * 8;
    const int r = (lx ? t0 : e0) + lrow;
    const int lim = lx ? T : E;
    if (r < lim && k < ke) {
      const uint16_t* src = (lx ? x : w) + (size_t)r * H + k;
      bf16x8_to_f64(*reinterpret_cast<const uint4*>(src), v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0;
    }
    double(*dst)[kRt + 2] = lx ? xs : ws;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[lpiece * 8 + i][lrow] = v[i];
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRk; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = xs[kk][ty * 4 + i];
        b[i] = ws[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  double* p = partial + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) p[(size_t)t * E + e] = acc[i][j];
    }
  }
}

RouterPlan plan_router(int T, int E, int H) {
  RouterPlan r;
  if (T <= kRouterRowsMaxT) {
    r.ks = 1;
    r.hsplit = H;
    return r;
  }
  const int blocks = ((E + kRe - 1) / kRe) * ((T + kRt - 1) / kRt);
  int ks = (256 + blocks - 1) / blocks;
  if (ks > kRouterMaxSplit) ks = kRouterMaxSplit;
  if (ks > H / 64) ks = H / 64;
  if (ks < 1) ks = 1;
  r.hsplit = ((H + ks - 1) / ks + kRk - 1) / kRk * kRk;
  r.ks = (H + r.hsplit - 1) / r.hsplit;
  return r;
}

hipError_t launch_router_partial(const uint16_t* x, const uint16_t* w, double* partial, int T,
                                 int E, int H, int ks, int hsplit, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kRouterRowsMaxT) {
    hipLaunchKernelGGL(k_router_rows, dim3(E), dim3(256), 0, s, x, w, partial, T, E, H);
  } else {
    dim3 grid((E + kRe - 1) / kRe, (T + kRt - 1) / kRt, ks);
    hipLaunchKernelGGL(k_router_tiled, grid, dim3(256), 0, s, x, w, partial, T, E, H, hsplit);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scores + top-K: one wavefront per token, the token's keys spread over the 64 lanes
// (NPL per lane). Selection is k rounds of a wave-wide arg-max on a 64-bit composite
// (order-preserving key bits << 32 | ~index): the largest key wins, equal keys go to
// the lower expert index, -0 == +0, and NaN ranks below -inf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_key(float f) {
  if (f != f) return 0u;                         // NaN: below everything
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(float key, int idx) {
  return ((uint64_t)ordered_key(key) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int kTopkWaves = 4;

template <int NPL>
__global__ __launch_bounds__(256) void k_topk(TopkArgs a) {
  __shared__ float s_logit[kTopkWaves][kMaxExperts];
  __shared__ int s_id[kTopkWaves][kMaxTopK];
  __shared__ float s_w[kTopkWaves][kMaxTopK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= a.T) return;  // whole wavefronts exit together
  const int E = a.E, K = a.K;

  float lg[NPL];
  float key[NPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i;
    float l = -__builtin_inff();
    if (e < E) {
      if (a.logits_in) {
        l = a.logits_in[(size_t)t * E + e];
      } else {
        // the split-K partials: independent loads first, then a fixed-order sum
        double pz[kRouterMaxSplit];
#pragma unroll
        for (int z = 0; z < kRouterMaxSplit; ++z)
          pz[z] = z < a.ks ? a.partial[((size_t)z * a.T + t) * E + e] : 0.0;
        double acc = 0.0;
#pragma unroll
        for (int z = 0; z < kRouterMaxSplit; ++z)
          if (z < a.ks) acc += pz[z];
        if (a.logit_bias) acc += (double)a.logit_bias[e];
        l = (float)acc;
      }
      if (a.logits_out) a.logits_out[(size_t)t * E + e] = l;
      s_logit[wave][e] = l;
    } else {
      taken |= 1u << i;  // padding is never selectable
    }
    lg[i] = l;
    float k = l;
    if (a.score == 1) {  // sigmoid: key = fp32(sigmoid) + correction bias (fp32 add)
      const float sg = (float)(1.0 / (1.0 + exp(-(double)l)));
      k = a.correction_bias && e < E ? sg + a.correction_bias[e] : sg;
    }
    key[i] = k;
  }

  // softmax normaliser over all experts (fp32): m = max, S = sum exp(l - m)
  float m = -__builtin_inff(), S = 0.f;
  if (a.score == 0) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) m = fmaxf(m, lg[i]);
    m = wave_max(m);
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < E) S += expf(lg[i] - m);
    S = wave_sum(S);
  }
  __builtin_amdgcn_wave_barrier();

  int err = 0;
  if (a.select == 0) {
    for (int j = 0; j < K; ++j) {
      uint64_t best = 0;
      bool have = false;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        if (!(taken & (1u << i))) {
          const uint64_t c = composite(key[i], lane + kWave * i);
          if (!have || c > best) { best = c; have = true; }
        }
      }
      uint64_t g = best;
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const uint64_t o = shfl_xor_u64(g, msk);
        g = o > g ? o : g;
      }
      const int idx = (int)(0xFFFFFFFFu - (uint32_t)g);
      if ((idx & 63) == lane) taken |= 1u << (idx >> 6);
      if (lane == 0) s_id[wave][j] = idx;
    }
  } else {  // hash routing: ids from the static table, no selection
    const int64_t tok = a.token_ids[t];
    const bool tok_ok = tok >= 0 && tok < a.vocab;
    if (!tok_ok) err |= 2;
    if (lane == 0) {
      for (int j = 0; j < K; ++j) {
        int id = -1;
        if (tok_ok) {
          const int64_t e = a.tid2eid[tok * K + j];
          if (e >= 0 && e < E) id = (int)e;
          else err |= 4;
        }
        s_id[wave][j] = id;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  if (lane == 0) {
    float sum = 0.f;
    for (int j = 0; j < K; ++j) {
      const int id = s_id[wave][j];
      float wj = 0.f;
      if (id >= 0) {
        const float l = s_logit[wave][id];
        wj = a.score == 0 ? expf(l - m) / S : (float)(1.0 / (1.0 + exp(-(double)l)));
      }
      s_w[wave][j] = wj;
      sum += wj;
    }
    for (int j = 0; j < K; ++j) {
      float wj = s_w[wave][j];
      if (a.renorm) wj = sum > 0.f ? wj / sum : 0.f;
      a.w[(size_t)t * K + j] = wj * a.scaling;
      a.ids[(size_t)t * K + j] = s_id[wave][j];
    }
    if (a.err_tok) a.err_tok[t] = err;
  }
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

}  // namespace moe
