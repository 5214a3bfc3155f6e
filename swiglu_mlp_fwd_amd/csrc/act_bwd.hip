// Elementwise SwiGLU backward on materialised gate/up, with an optional clamp
// and optional per-row (routing) weights.
//
// "quant: add SwiGLU forward/backward VMI kernels" (TileKernels-PTO PR 20):
// the performance section's backward table (gate/up given, clamp, routing
// weights with recompute) and the implementation notes (weight_grad is a
// reassociated reduction).  With the forward
//   y[r, c] = w[r] * SiLU(g'[r, c]) * u'[r, c],  g' = clamp(g), u' = clamp(u)
// (w = 1 without weights), the kernel computes from dy
//   dg = w dy u' s (1 + g' (1 - s))   where |g| <= L or g is NaN, else 0
//   du = w dy SiLU(g')                where |u| <= L or u is NaN, else 0
//   weight_grad[r] = sum_c dy SiLU(g') u'
// with s = sigma(g').  sigma and 1 - sigma come from the accurate fp32 form
// (each to a few ulps, the complement without cancellation); the products
// and the row sum are formed in fp64 and the outputs rounded to fp32 once.
//
// Mapping: one wave per row (grid-stride over rows); lane l handles the
// 16-byte chunks l, l + 64, ... of the row, kUnroll chunks' loads issued
// before any is used; the row sum is reduced across the wave with xor
// shuffles and written by lane 0.
#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;         // 4 waves, one row each
constexpr int kMaxBlocks = 4096;
constexpr int kUnroll = 4;

template <bool kClamp>
__device__ __forceinline__ void bwd_elem(float g, float u, float dy, double w, float L, float& dg,
                                         float& du, double& acc) {
  bool pg = true, pu = true;
  if (kClamp) {
    pg = !(fabsf(g) > L);
    pu = !(fabsf(u) > L);
    g = pg ? g : copysignf(L, g);
    u = pu ? u : copysignf(L, u);
  }
  float s, c;
  sigmoid_pair_f32(g, s, c);
  const double silu = (double)g * (double)s;
  const double dh = w * (double)dy;
  const double t = (double)s * (1.0 + (double)g * (double)c);
  dg = pg ? (float)(dh * (double)u * t) : 0.0f;
  du = pu ? (float)(dh * silu) : 0.0f;
  acc += (double)dy * (silu * (double)u);
}

template <bool kClamp, bool kWeights, bool kGrad>
__global__ __launch_bounds__(kThreads) void act_bwd_kernel(const float* __restrict__ gate,
                                                           const float* __restrict__ up,
                                                           const float* __restrict__ dy,
                                                           const float* __restrict__ weights, float L,
                                                           float* __restrict__ dgate,
                                                           float* __restrict__ dup,
                                                           float* __restrict__ wgrad, int64_t rows,
                                                           int64_t cols) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = cols / 4;
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < rows;
       r += (int64_t)gridDim.x * (kThreads / 64)) {
    const double w = kWeights ? (double)weights[r] : 1.0;
    const f32x4* g4 = reinterpret_cast<const f32x4*>(gate + r * cols);
    const f32x4* u4 = reinterpret_cast<const f32x4*>(up + r * cols);
    const f32x4* d4 = reinterpret_cast<const f32x4*>(dy + r * cols);
    f32x4* og = reinterpret_cast<f32x4*>(dgate + r * cols);
    f32x4* ou = reinterpret_cast<f32x4*>(dup + r * cols);
    double acc = 0.0;
    for (int64_t c0 = lane; c0 < nch; c0 += 64 * kUnroll) {
      f32x4 G[kUnroll], U[kUnroll], D[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t c = c0 + 64 * j;
        if (c < nch) {
          G[j] = __builtin_nontemporal_load(g4 + c);
          U[j] = __builtin_nontemporal_load(u4 + c);
          D[j] = __builtin_nontemporal_load(d4 + c);
        }
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t c = c0 + 64 * j;
        if (c >= nch) break;
        float a[4], b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bwd_elem<kClamp>(G[j][e], U[j][e], D[j][e], w, L, a[e], b[e], acc);
        __builtin_nontemporal_store(f32x4{a[0], a[1], a[2], a[3]}, og + c);
        __builtin_nontemporal_store(f32x4{b[0], b[1], b[2], b[3]}, ou + c);
      }
    }
    if (kGrad) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) wgrad[r] = (float)acc;
    }
  }
}

template <bool kClamp, bool kWeights, bool kGrad>
void launch_ab(unsigned grid, const float* gate, const float* up, const float* dy, const float* w,
               float L, float* dg, float* du, float* wgrad, int64_t rows, int64_t cols, hipStream_t s) {
  hipLaunchKernelGGL((act_bwd_kernel<kClamp, kWeights, kGrad>), dim3(grid), dim3(kThreads), 0, s,
                     gate, up, dy, w, L, dg, du, wgrad, rows, cols);
}

}  // namespace

hipError_t launch_act_bwd(int64_t rows, int64_t cols, const float* gate, const float* up,
                          const float* dy, const float* weights, float limit, bool clamp,
                          float* dgate, float* dup, float* wgrad, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t want = (rows + kThreads / 64 - 1) / (kThreads / 64);
  const unsigned grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  const bool w = weights != nullptr, g = wgrad != nullptr;
#define SWG_AB(C, W, G) launch_ab<C, W, G>(grid, gate, up, dy, weights, limit, dgate, dup, wgrad, rows, cols, s)
  if (clamp) {
    if (w) { if (g) SWG_AB(true, true, true); else SWG_AB(true, true, false); }
    else { if (g) SWG_AB(true, false, true); else SWG_AB(true, false, false); }
  } else {
    if (w) { if (g) SWG_AB(false, true, true); else SWG_AB(false, true, false); }
    else { if (g) SWG_AB(false, false, true); else SWG_AB(false, false, false); }
  }
#undef SWG_AB
  return hipGetLastError();
}

}  // namespace swg
