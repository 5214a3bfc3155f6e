// Decode forward, 1 <= M <= 8 tokens, bf16: h = SiLU(x Wg^T) * (x Wu^T).
//
// The work is bound by reading Wg and Wu from HBM once ("Fused SwiGLU
// benchmark", AstrAI docs/developer/swiglu_benchmark.md, sections L20
// findings and HBM re-measurement: the wide shapes are weight-bandwidth
// dominated and the fused kernel sits at the dual-stream cold-read floor).
// No matrix cores: the dot products run on the vector ALU with the bf16 dot2
// instruction (two bf16 products accumulated into fp32 per lane-op).
//
// Mapping: each half-wave (32 lanes) owns one output column n and streams
// the rows Wg[n, :] and Wu[n, :] with 16-byte loads (lane j reads chunks
// j, j+32, ...); x [M, K] is staged once per workgroup in LDS and each 16-byte
// chunk of it is reused for both weights.  Per lane the 2M partial sums are
// reduced across the half-wave with butterfly shuffles; lane 0 of the half
// applies SiLU(g) * u and stores the M outputs of its column.
#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

// 8 waves: x is staged once per 16 columns, and at M = 8 (64 KiB of x at
// K = 4096) two workgroups per CU still give 16 waves of loads in flight.
constexpr int kThreads = 512;
constexpr int kColsPerBlock = 16;  // 8 waves x 2 half-waves

// x exchanged across the half-waves (measured faster from M = 6 up; below,
// the extra exchange costs more than the LDS reads it saves).
template <int M> constexpr bool kSplitX = M >= 6 && M % 2 == 0;

template <int M, Act A>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const bf16* __restrict__ x,
                                                        const bf16* __restrict__ wg,
                                                        const bf16* __restrict__ wu,
                                                        bf16* __restrict__ h, int N, int K,
                                                        float gmul, float umul) {
  extern __shared__ u32x4 xs[];  // [M][K / 8]
  const int nch = K >> 3;
  const int tid = threadIdx.x;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);
  for (int i = tid; i < M * nch; i += kThreads) xs[i] = xg[i];
  __syncthreads();

  const int lane = tid & 63;
  const int hl = lane & 31;
  const int col0 = (blockIdx.x * (kThreads / 64) + (tid >> 6)) * 2;
  if (col0 >= N) return;                           // the whole wave is past the end
  const int col = col0 + (lane >> 5);
  const bool live = col < N;
  // A half-wave past the end streams the last column again and stores
  // nothing, so both halves stay active for the cross-half exchange below.
  const int ccol = live ? col : N - 1;

  const u32x4* rg = reinterpret_cast<const u32x4*>(wg + (int64_t)ccol * K);
  const u32x4* ru = reinterpret_cast<const u32x4*>(wu + (int64_t)ccol * K);
  float ag[M], au[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ag[m] = au[m] = 0.0f;

  if constexpr (kSplitX<M>) {
    // The two half-waves read the same x chunks.  Each reads half of the
    // M rows (the lower half rows 0..M/2-1, the upper half the rest) and
    // v_permlane32_swap hands every lane both halves' values: half the LDS
    // reads of x per weight chunk.
    constexpr int H = M / 2;
    const int mb = (lane >> 5) * H;
#pragma unroll 2
    for (int c = hl; c < nch; c += 32) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
#pragma unroll
      for (int q = 0; q < H; ++q) {
        const u32x4 xv = xs[(mb + q) * nch + c];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // r[0]: the lower half's value (row q), r[1]: the upper half's (row H + q).
          const auto r = __builtin_amdgcn_permlane32_swap(xv[t], xv[t], false, false);
          const bf16x2 lo = as_bf16x2(r[0]), hi = as_bf16x2(r[1]);
          ag[q] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vg[t]), lo, ag[q], false);
          au[q] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vu[t]), lo, au[q], false);
          ag[H + q] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vg[t]), hi, ag[H + q], false);
          au[H + q] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vu[t]), hi, au[H + q], false);
        }
      }
    }
  } else {
#pragma unroll 4
    for (int c = hl; c < nch; c += 32) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4 xv = xs[m * nch + c];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 xx = as_bf16x2(xv[t]);
          ag[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vg[t]), xx, ag[m], false);
          au[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vu[t]), xx, au[m], false);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      ag[m] += __shfl_xor(ag[m], off, 32);
      au[m] += __shfl_xor(au[m], off, 32);
    }
  }
  if (live && hl == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float g = gmul * ag[m], u = umul * au[m];
      const float a = (A == Act::kGeluTanh) ? gelu_tanh_f32(g) : silu_f32(g);
      h[(int64_t)m * N + col] = to_bf16(a * u);
    }
  }
}

template <int M, Act A>
hipError_t launch_m(int N, int K, const void* x, const void* wg, const void* wu, void* h,
                    float gm, float um, hipStream_t s) {
  const unsigned blocks = (unsigned)((N + kColsPerBlock - 1) / kColsPerBlock);
  const size_t lds = (size_t)M * K * 2;
  hipLaunchKernelGGL((gemv_kernel<M, A>), dim3(blocks), dim3(kThreads), lds, s,
                     static_cast<const bf16*>(x), static_cast<const bf16*>(wg),
                     static_cast<const bf16*>(wu), static_cast<bf16*>(h), N, K, gm, um);
  return hipGetLastError();
}

template <Act A>
hipError_t launch_act(int M, int N, int K, const void* x, const void* wg, const void* wu, void* h,
                      float gm, float um, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1, A>(N, K, x, wg, wu, h, gm, um, s);
    case 2: return launch_m<2, A>(N, K, x, wg, wu, h, gm, um, s);
    case 3: return launch_m<3, A>(N, K, x, wg, wu, h, gm, um, s);
    case 4: return launch_m<4, A>(N, K, x, wg, wu, h, gm, um, s);
    case 5: return launch_m<5, A>(N, K, x, wg, wu, h, gm, um, s);
    case 6: return launch_m<6, A>(N, K, x, wg, wu, h, gm, um, s);
    case 7: return launch_m<7, A>(N, K, x, wg, wu, h, gm, um, s);
    case 8: return launch_m<8, A>(N, K, x, wg, wu, h, gm, um, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(Act act, int M, int N, int K, const void* x, const void* wg, const void* wu,
                       void* h, float gmul, float umul, hipStream_t s) {
  return act == Act::kGeluTanh ? launch_act<Act::kGeluTanh>(M, N, K, x, wg, wu, h, gmul, umul, s)
                               : launch_act<Act::kSilu>(M, N, K, x, wg, wu, h, gmul, umul, s);
}

}  // namespace swg
