// FP8 block quantisation helpers shared by the elementwise kernel and the
// FP8-output epilogue of the dual GEMM ("quant: add SwiGLU forward/backward
// VMI kernels", TileKernels-PTO PR 20, implementation notes: 1x32 blocks,
// packed UE8M0 scales, E4M3 cast without saturation keeping NaN).
#pragma once

#include "common.hpp"

namespace swg {

// UE8M0 exponent of a block: smallest E with amax <= 448 * 2^E, clamped to
// [-127, 127]; E = 128 when amax is +inf.  amax is finite-or-inf, >= 0.
// With amax = 1.f * 2^ea: 448 * 2^E = 1.75 * 2^(E + 8), so E = ea - 8 when
// 1.f <= 1.75 and ea - 7 otherwise.
__device__ __forceinline__ int block_exponent(float amax) {
  const uint32_t a = f32_bits(amax);
  if (a >= 0x7F800000u) return 128;
  if (a == 0) return -127;
  int ea;
  uint32_t frac;
  if (a >= 0x00800000u) {
    ea = (int)(a >> 23) - 127;
    frac = a & 0x7FFFFFu;
  } else {                                  // subnormal: normalise the mantissa
    const int lz = __clz(a);                // a < 2^23, so lz >= 9
    ea = (31 - lz) - 149;
    frac = (a << (lz - 8)) & 0x7FFFFFu;
  }
  int E = ea - 8 + (frac > 0x600000u ? 1 : 0);
  return E < -127 ? -127 : E;
}

// E4M3FN codes of RNE(h * 2^-E) for two values, no saturation, NaN/inf ->
// NaN, using the gfx950 conversion v_cvt_pk_fp8_f32 (OCP E4M3FN, current
// rounding mode = nearest even, no clamp).  The scale 2^-E is exact in fp32
// for E in [-127, 128] (2^-128 is a subnormal) and the product h * 2^-E is
// exact whenever it is a normal number; when it is below 2^-126 it is far
// below half the smallest E4M3 step (2^-10), so any rounding of the product
// cannot change the code.
__device__ __forceinline__ uint32_t e4m3_pair(float h0, float h1, float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(h0 * s, h1 * s, 0, false) & 0xFFFFu;
}

// h = SiLU(g) * u in fp64 (swiglu_value: rounded once to fp32).
//
// e^-|g| = p 2^n (exp_neg_split); sigma(|g|) = 1 / (1 + e) and
// sigma(-|g|) = p r 2^n with r = 1 / (1 + e).  The product g u sigma is
// formed in fp64, where g * u is exact and the scale 2^n is applied by
// ldexp, and is rounded to fp32 once.  So no intermediate is ever an fp32
// subnormal: a subnormal gate times a large up, or a very negative gate
// (sigma below 2^-126), keeps its precision.  fp64 multiplies run at the fp32
// rate on this chip.  Special values follow IEEE: g = -inf gives 2^n -> 0 and
// -inf * 0 = NaN; g = +inf gives inf * u; NaN propagates.
__device__ __forceinline__ double swiglu_value_d(float g, float u) {
#pragma clang fp contract(off)
  float p;
  int n;
  exp_neg_split(fminf(fabsf(g), 1024.0f), p, n);  // e^-1024 is 0 even in fp64
  const float d = 1.0f + ldexpf(p, n);
  float r = __builtin_amdgcn_rcpf(d);
  r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
  const bool pos = g >= 0.0f;
  const double sig = ldexp((double)(pos ? r : p * r), pos ? 0 : n);
  return ((double)g * (double)u) * sig;
}

__device__ __forceinline__ float swiglu_value(float g, float u) { return (float)swiglu_value_d(g, u); }

// h = GELU_tanh(g) * u in fp64 (gelu_value: rounded once to fp32),
// GELU_tanh(z) = z sigma(t) with
// t = 2 sqrt(2/pi) (z + 0.044715 z^3) ("VisualGen MLP: cublasLt GELU-tanh
// epilogue for the unquantized bf16 path", TensorRT-LLM PR 17693, the GELU
// tanh activation; (1 + tanh y) / 2 = sigma(2 y)).
//
// The argument t is formed in fp64: in fp32 its rounding error would be
// multiplied by |t| in sigma's tail (sigma(-a) ~ e^-a), hundreds of ulps at
// |t| ~ 100.  |t| (capped at 1024, where e^-|t| is 0 even in fp64) is split
// as ah + al with ah = fp32(|t|), |al| <= 2^-14; e^-|t| = p 2^n (1 - al)
// to well under an ulp, and the rest is as in swiglu_value.
__device__ __forceinline__ double gelu_value_d(float g, float u) {
#pragma clang fp contract(off)
  constexpr double kC1 = 1.5957691216057308;      // 2 sqrt(2 / pi)
  constexpr double kC3 = 0.071354816272600254;    // 2 sqrt(2 / pi) * 0.044715
  const double z = g;
  const double t = z * (kC1 + kC3 * (z * z));
  const double a = fmin(fabs(t), 1024.0);         // fmin drops NaN: g = NaN propagates below
  const float ah = (float)a;
  const float al = (float)(a - (double)ah);
  float p;
  int n;
  exp_neg_split(ah, p, n);
  p = p - p * al;
  const float d = 1.0f + ldexpf(p, n);
  float r = __builtin_amdgcn_rcpf(d);
  r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
  const bool pos = t >= 0.0;
  const double sig = ldexp((double)(pos ? r : p * r), pos ? 0 : n);
  return (z * (double)u) * sig;
}

__device__ __forceinline__ float gelu_value(float g, float u) { return (float)gelu_value_d(g, u); }

}  // namespace swg
