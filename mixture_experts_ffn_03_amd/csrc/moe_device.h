// Device helpers of the gfx950 MoE kernels: bf16 packing, FP4 block decoding and
// wavefront (64-lane) reductions. Every kernel of the library includes this file;
// nothing here is used on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Weight streams of the decode GEMVs: each 16-byte piece of an expert's weights is read once
// per layer call, so these loads carry the non-temporal hint (streaming cache policy). Measured
// on the Qwen3-like 8-token decode: gate+up 20.6 -> 19.6 us, step 50.0 -> 46.8 us; neutral on
// the DeepSeek-V3-like and one-token decodes. The block-scale bytes stay plain loads: neighbouring
// lanes and passes share their lines (non-temporal scales slowed the DeepSeek-V3-like gate+up by
// 3 %). Build flag MOE_NT_WEIGHTS=0 gives plain weight loads.
#ifndef MOE_NT_WEIGHTS
#define MOE_NT_WEIGHTS 1
#endif
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_weights16(const void* p) {
#if MOE_NT_WEIGHTS
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

// Tile count of a dispatch, written with the persistent GEMMs' work counters zeroed
// (one thread; the GEMMs run after the dispatch on the same stream).
__device__ __forceinline__ void publish_tile_count(int32_t* ntiles, int n) {
  ntiles[0] = n;
#pragma unroll
  for (int i = 0; i < kWorkCtrSets * kXcds; ++i) ntiles[kWorkCtrOffset + i * kWorkCtrStride] = 0;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-to-nearest-even fp32 -> bf16 (gfx950 converts natively; denormals kept).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// SiLU(g) = g * sigmoid(g) = g / (1 + e^-g) from the hardware base-2 exponential and
// reciprocal (about 1 ulp each; the product is rounded to bf16 next). Large -g gives
// e^-g = inf and a zero result; large g gives g.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Two fp32 -> fp16 pair, round to nearest even, saturating at +-65504 (fmaxf / fminf order:
// a NaN becomes -65504).
__device__ __forceinline__ uint32_t pack_f16x2_sat(float lo, float hi) {
  lo = fminf(fmaxf(lo, -65504.f), 65504.f);
  hi = fminf(fmaxf(hi, -65504.f), 65504.f);
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Two floats -> fp16 pair, round to nearest even, no saturation (beyond the range: +-inf).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Nonzero in bit 15 or 31 where an fp16 of the pair is infinite or NaN (exponent field all
// ones: adding one to it carries out of the field).
__device__ __forceinline__ uint32_t f16x2_nonfinite_bits(uint32_t p) {
  return ((p & 0x7C007C00u) + 0x04000400u) & 0x80008000u;
}

__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Scale decoding. E4M3 here is the OCP "FN" variant (bias 7, max 448, NaN at
// S.1111.111), which NVFP4 uses for its per-16 block scales; E8M0 is the MX
// per-32 shared exponent 2^(s-127) with 0xFF = NaN.
// ---------------------------------------------------------------------------
// gfx950's FP8 convert reads the OCP E4M3FN encoding (NaN only at S.1111.111, no inf);
// the exhaustive dequant parity test checks every code against the format definition.
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return e4m3_byte_to_f32<0>(b); }

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  if (b == 0xFFu) return __uint_as_float(0x7FC00000u);
  if (b == 0u) return __uint_as_float(0x00400000u);  // 2^-127 (fp32 denormal)
  return __uint_as_float(b << 23);
}

// ---------------------------------------------------------------------------
// E2M1 decoding with the gfx950 scaled converts. The instruction applies only the
// exponent of its f32 scale operand (checked exhaustively against the format
// definition by the dequant parity test), so it is exact for power-of-two scales
// (E8M0 and 1.0) and an E4M3 block scale is applied as a separate fp32 factor.
// ---------------------------------------------------------------------------

// Byte `sel` of q (codes 2*sel, 2*sel+1; low nibble first) -> bf16 pair times 2^exp(scale).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t q, float pow2_scale) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, pow2_scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t q, float pow2_scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, pow2_scale, SEL);
}

// 8 codes (one dword) -> 4 bf16 pairs, exact values e2m1 * 2^exp(pow2_scale).
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t q, float pow2_scale, uint32_t out[4]) {
  out[0] = fp4x2_to_bf16x2<0>(q, pow2_scale);
  out[1] = fp4x2_to_bf16x2<1>(q, pow2_scale);
  out[2] = fp4x2_to_bf16x2<2>(q, pow2_scale);
  out[3] = fp4x2_to_bf16x2<3>(q, pow2_scale);
}

// 8 codes -> 4 bf16 pairs of e2m1 * s for an arbitrary fp32 factor s whose product with
// every E2M1 value is representable in bf16 (true for every E4M3 value): decode to f32,
// multiply (exact), convert (exact).
__device__ __forceinline__ void fp4x8_to_bf16_scaled(uint32_t q, float s, uint32_t out[4]) {
  f32x2_t a = fp4x2_to_f32x2<0>(q, 1.0f);
  f32x2_t b = fp4x2_to_f32x2<1>(q, 1.0f);
  f32x2_t c = fp4x2_to_f32x2<2>(q, 1.0f);
  f32x2_t d = fp4x2_to_f32x2<3>(q, 1.0f);
  out[0] = pack_bf16x2(a[0] * s, a[1] * s);
  out[1] = pack_bf16x2(b[0] * s, b[1] * s);
  out[2] = pack_bf16x2(c[0] * s, c[1] * s);
  out[3] = pack_bf16x2(d[0] * s, d[1] * s);
}

// Scale operand of the scaled convert for an E8M0 code: 2^(b-127) as f32 bits
// (b = 0 is the denormal 2^-127; b = 255 gives the f32 exponent field 255).
__device__ __forceinline__ float e8m0_cvt_scale(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// The bf16 B operand of the grouped GEMM for 8 codes of one scale block: exact
// e2m1 * scale for both formats (MXFP4 through the scaled convert, NVFP4 through fp32).
template <int FMT>
__device__ __forceinline__ void mfma_operand_fp4x8(uint32_t q, uint32_t sb, uint32_t out[4]) {
  if (FMT == 1) fp4x8_to_bf16(q, e8m0_cvt_scale(sb), out);
  else fp4x8_to_bf16_scaled(q, e4m3_to_f32(sb), out);
}

__device__ __forceinline__ void mfma_operand_fp4x8(int fmt, uint32_t q, uint32_t sb,
                                                   uint32_t out[4]) {
  if (fmt == 1) mfma_operand_fp4x8<1>(q, sb, out);
  else mfma_operand_fp4x8<0>(q, sb, out);
}

// Four E4M3 codes (byte j = code j) -> two bf16 pairs, exact (E4M3's range and 3-bit
// mantissa fit bf16; scale operand 1.0).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t q, uint32_t out[2]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true));
}

// The bf16 B operand of the grouped GEMM for 8 E4M3 codes (two dwords) of one 128 x 128
// block with fp32 scale s: bf16(e4m3 * s), one rounding per element.
__device__ __forceinline__ void mfma_operand_fp8x8(uint32_t q0, uint32_t q1, float s,
                                                   uint32_t out[4]) {
  const uint32_t q[2] = {q0, q1};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[i], 1.0f, false);
    const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[i], 1.0f, true);
    out[2 * i] = pack_bf16x2(a[0] * s, a[1] * s);
    out[2 * i + 1] = pack_bf16x2(b[0] * s, b[1] * s);
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}

// Sum NV per-lane values over each aligned group of L lanes (L a power of two <= 64),
// halving the value count at each of the first log2(NV) butterfly distances so that
// no lane reduces every value. On return a lane holds NF = max(1, NV / L) complete
// sums in v[0..NF); the value index of v[i] is reduced_index(lane, i). The steps are
// unrolled at compile time (a runtime index would push the array into scratch memory).
template <int NV, int D, int N>
struct GroupReduceStep {
  static __device__ __forceinline__ void run(float (&v)[NV], int lane) {
    if constexpr (D >= 1) {
      if constexpr (N > 1) {
        constexpr int H = N / 2;
        const bool upper = (lane & D) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          const float send = upper ? v[i] : v[i + H];
          const float keep = upper ? v[i + H] : v[i];
          v[i] = keep + shfl_xor_f(send, D);
        }
        GroupReduceStep<NV, D / 2, H>::run(v, lane);
      } else {
        v[0] += shfl_xor_f(v[0], D);
        GroupReduceStep<NV, D / 2, 1>::run(v, lane);
      }
    }
  }
};

template <int NV, int L>
__device__ __forceinline__ void group_reduce_transpose(float (&v)[NV], int lane) {
  GroupReduceStep<NV, L / 2, NV>::run(v, lane);
}

// Value index held in v[i] after group_reduce_transpose<NV, L>.
template <int NV, int L>
__device__ __forceinline__ int reduced_index(int lane, int i) {
  int idx = i, n = NV;
#pragma unroll
  for (int d = L / 2; d >= 1; d >>= 1) {
    if (n > 1) {
      n >>= 1;
      if (lane & d) idx += n;
    }
  }
  return idx;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// Direct-to-LDS loads: every active lane reads SIZE bytes at its own global address; the
// wave writes them to LDS at m0 + lane * SIZE (m0 = the wave-uniform base; the 2-byte form
// fills 4-byte slots, the value in the low half). The compiler cannot see them: their wait
// (vmcnt) is issued by hand.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
// the same with the non-temporal hint: weight rows that one block streams once (256-code
// stages of 32-row tiles, whose experts rarely have a second row tile). Hash layer gate+up
// 498 -> 476 us; on 128-row tiles, whose weights the expert's other row tiles re-read from the
// caches, the hint made gate+up 25 % slower.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}

}  // namespace moe
