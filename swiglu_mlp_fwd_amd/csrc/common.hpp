// Shared device-side definitions for libswiglu (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swg {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Reinterpret one 32-bit word as two bf16 (element 0 = low half).  Takes the
// word by value: bit-casting a vector element lvalue directly reads element 0.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float f) { return (bf16)f; }
__device__ __forceinline__ float from_bf16(bf16 b) { return (float)b; }

// e^-a for a >= 0 as p * 2^n with p in [1, 2) (up to one ulp of slack at
// the ends) and integer n:  e^-a = 2^t, t = -a log2(e).  n = floor of the
// rounded product; f = t - n is formed by one fused multiply-add from the
// exact product -a * L2E_hi (L2E_hi = log2(e) rounded to fp32), and the tail
// -a * (log2(e) - L2E_hi) is applied to first order:
//   2^t = 2^f * 2^tail ~ 2^f * (1 + tail ln 2),  |tail| < 2^-17.
// With the hardware exp2 (v_exp_f32) on f in [0, 1) the result is good to
// about two ulps for every a.  Contraction is off so the compiler cannot
// fold the rounding of the product used for floor() into f.
__device__ __forceinline__ void exp_neg_split(float a, float& p, int& n) {
#pragma clang fp contract(off)
  constexpr float kL2eHi = 1.44269502162933349609375f;      // fp32(log2 e)
  constexpr float kL2eLo = 1.925963033500011079e-08f;       // log2 e - kL2eHi
  constexpr float kLn2 = 0.693147180559945309f;
  const float nf = floorf(-a * kL2eHi);
  const float f = __builtin_fmaf(-a, kL2eHi, -nf);
  const float tail = -a * kL2eLo;
  const float e2 = __builtin_amdgcn_exp2f(f);
  p = __builtin_fmaf(e2 * tail, kLn2, e2);
  n = (int)nf;
}

// sigma(z) and SiLU(z) = z * sigma(z) in fp32, from e = exp(-|z|) in (0, 1]
// so no step overflows:  sigma(|z|) = 1 / (1 + e),  sigma(-|z|) = e / (1 + e).
// The reciprocal is the hardware v_rcp_f32 refined by one Newton step.
// IEEE rules carry the special values: SiLU(+inf) = +inf,
// SiLU(-inf) = -inf * 0 = NaN, SiLU(NaN) = NaN.  For z below about -87 the
// fp32 value of e flushes to zero and SiLU(z) returns -0 (|true value| is
// below 1e-36); the elementwise kernel, whose output is fp32, handles that
// range exactly on its own.
__device__ __forceinline__ void sigmoid_silu_f32(float z, float& s, float& silu) {
#pragma clang fp contract(off)
  float p;
  int n;
  exp_neg_split(fminf(fabsf(z), 128.0f), p, n);   // fminf drops NaN: z = NaN handled below
  const float e = ldexpf(p, n);
  const float d = 1.0f + e;
  float r = __builtin_amdgcn_rcpf(d);
  r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
  s = (z >= 0.0f) ? r : e * r;
  if (z != z) s = z;
  silu = z * s;
}

// sigma(z) and 1 - sigma(z), both to a few ulps (the complement is not
// formed by subtracting, which would lose it for large z):
//   z >= 0: sigma = 1 / (1 + e),  1 - sigma = e / (1 + e),  e = exp(-|z|),
//   z < 0 : the two swap.  NaN gives NaN for both.
__device__ __forceinline__ void sigmoid_pair_f32(float z, float& s, float& c) {
#pragma clang fp contract(off)
  float p;
  int n;
  exp_neg_split(fminf(fabsf(z), 128.0f), p, n);
  const float e = ldexpf(p, n);
  const float d = 1.0f + e;
  float r = __builtin_amdgcn_rcpf(d);
  r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
  const float er = e * r;
  s = (z >= 0.0f) ? r : er;
  c = (z >= 0.0f) ? er : r;
  if (z != z) s = c = z;
}

// fp64 -> bf16 with one rounding (to nearest even): round to fp32 by
// round-to-odd, then to bf16 by RNE.  Round-to-odd keeps the information
// the second rounding needs (fp32 has 16 more bits than bf16), so the pair
// equals a direct RNE of d.
__device__ __forceinline__ uint32_t bf16_bits_rne(double d) {
  const float f = (float)d;
  uint32_t b = f32_bits(f);
  if ((double)f != d && (b & 1u) == 0u && f == f) {
    // Inexact with an even last bit: the odd neighbour lies toward d.
    b += (fabs((double)f) > fabs(d)) ? -1 : 1;
  }
  return __builtin_bit_cast(uint16_t, to_bf16(bits_f32(b)));
}

// sigma(z) and SiLU(z) for results that are rounded to bf16 right after:
// sigma = 1 / (1 + 2^(-z log2 e)) with the hardware exp2 and reciprocal
// (about 13 VALU slots instead of about 25).  The product z log2 e is
// rounded once, so sigma carries a relative error of at most
// |z| * 2^-24 * ln 2 plus a few ulps: below 1e-5 for -87 < z < 100, far
// under the 2^-8 of the bf16 rounding that follows.  Below z = -87 sigma
// leaves the normal fp32 range and from z = -88.7 (2^(-z log2 e) overflows)
// it is 0, so there SiLU(z) keeps only the absolute accuracy of a result
// below 2^-126 |z|.  Limits follow IEEE:
// z -> -inf gives sigma = 0 (2^+inf = inf, 1 / inf = 0), so SiLU(-inf) =
// -inf * 0 = NaN as in the accurate form; z = +inf gives sigma = 1; NaN
// propagates.
__device__ __forceinline__ void sigmoid_silu_bf16out(float z, float& s, float& silu) {
  constexpr float kL2e = 1.44269504088896340736f;
  const float e = __builtin_amdgcn_exp2f(-z * kL2e);
  s = __builtin_amdgcn_rcpf(1.0f + e);
  silu = z * s;
}

// GELU with the tanh approximation, as z * sigma(2 y) with
// y = sqrt(2/pi) (z + 0.044715 z^3), i.e. 2 y = z (c1 + c3 z^2): the identity
// (1 + tanh y) / 2 = sigma(2 y) is exact and avoids the cancellation of
// 1 + tanh(y) for negative z.  Infinities and NaN follow IEEE as for SiLU.
constexpr float kGeluC1 = 1.5957691216057308f;      // 2 sqrt(2 / pi)
constexpr float kGeluC3 = 0.07135481627260025f;     // 2 sqrt(2 / pi) * 0.044715

// Accurate form (fp32 outputs).
__device__ __forceinline__ float gelu_tanh_f32(float z) {
  const float t = z * __builtin_fmaf(kGeluC3, z * z, kGeluC1);
  float s, c;
  sigmoid_pair_f32(t, s, c);
  return z * s;
}

// Short form for results rounded to bf16 right after (hardware exp2 and
// reciprocal, as sigmoid_silu_bf16out).
__device__ __forceinline__ float gelu_tanh_bf16out(float z) {
  const float t = z * __builtin_fmaf(kGeluC3, z * z, kGeluC1);
  constexpr float kL2e = 1.44269504088896340736f;
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t * kL2e));
}

__device__ __forceinline__ float silu_f32(float z) {
  float s, silu;
  sigmoid_silu_f32(z, s, silu);
  return silu;
}

// Bijection from the hardware workgroup index to a logical tile index such
// that each XCD (workgroups are dealt to the 8 XCDs round-robin) receives a
// contiguous range of logical tiles, so tiles that share operands share an
// L2.
__device__ __forceinline__ int xcd_remap(int bid, int ntiles) {
  constexpr int kXcds = 8;
  int q = ntiles / kXcds, r = ntiles % kXcds;
  int x = bid % kXcds, j = bid / kXcds;
  int start = x * q + (x < r ? x : r);
  return start + j;
}

}  // namespace swg
