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
// j, j+32, ...); x [M, K] is staged in LDS and each 16-byte chunk of it is
// reused for both weights.  Per lane the 2M partial sums are reduced across
// the half-wave with butterfly shuffles; lane 0 of the half applies
// act(g) * u and stores the M outputs of its column.
//
// x up to 64 KiB (M K <= 32768) is staged whole; larger x in K-phases of at
// most about 36 KiB: the workgroup stages x[:, phase], streams the weights
// of that phase, and moves on.  Then four workgroups (32 waves, the most a
// CU holds) share a CU's 160 KiB of LDS whatever K is, where x staged whole
// at M = 8, K = 6144 (96 KiB) left one.  There is no limit on K.
//
// The read-only twin (kTwin) is the same kernel with the same grid, LDS
// footprint, x staging and weight loads, and no arithmetic: each lane folds
// the loaded words into one value.  Its time is the floor of this access
// pattern, the counterpart on the same buffers of the benchmark page's
// pure-read loop.
#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

// 8 waves: x is staged once per 16 columns.
constexpr int kThreads = 512;
constexpr int kColsPerBlock = 16;  // 8 waves x 2 half-waves
// x up to this size is staged whole (at 64 KiB two workgroups still share
// a CU); beyond it, in phases of at most kPhaseBytes (four per CU).
constexpr int kWholeBytes = 64 * 1024;
constexpr int kPhaseBytes = 36 * 1024;

// x exchanged across the half-waves (measured faster from M = 6 up; below,
// the extra exchange costs more than the LDS reads it saves).
template <int M> constexpr bool kSplitX = M >= 6 && M % 2 == 0;

// One half-wave's pass over chunks [0, nc) of its column's weight rows
// rg, ru, against x chunks xs[m * stride + c]: dot products into ag, au,
// or, for the twin, a fold of the loaded words.
template <int M, bool kTwin>
__device__ __forceinline__ void stream_chunks(const u32x4* __restrict__ rg, const u32x4* __restrict__ ru,
                                              const u32x4* xs, int stride, int nc, int lane,
                                              float (&ag)[M], float (&au)[M], uint32_t& fold) {
  const int hl = lane & 31;
  if constexpr (kTwin) {
    // The weight stream of the branch below that this M takes (same loads,
    // same unrolling), folded into one word.
    auto eat = [&](int c) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
      fold ^= vg[0] ^ vg[1] ^ vg[2] ^ vg[3] ^ vu[0] ^ vu[1] ^ vu[2] ^ vu[3];
    };
    if constexpr (kSplitX<M>) {
#pragma unroll 2
      for (int c = hl; c < nc; c += 32) eat(c);
    } else {
#pragma unroll 4
      for (int c = hl; c < nc; c += 32) eat(c);
    }
  } else if constexpr (kSplitX<M>) {
    // The two half-waves read the same x chunks.  Each reads half of the
    // M rows (the lower half rows 0..M/2-1, the upper half the rest) and
    // v_permlane32_swap hands every lane both halves' values: half the LDS
    // reads of x per weight chunk.
    constexpr int H = M / 2;
    const int mb = (lane >> 5) * H;
#pragma unroll 2
    for (int c = hl; c < nc; c += 32) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
#pragma unroll
      for (int q = 0; q < H; ++q) {
        const u32x4 xv = xs[(mb + q) * stride + c];
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
    for (int c = hl; c < nc; c += 32) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4 xv = xs[m * stride + c];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 xx = as_bf16x2(xv[t]);
          ag[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vg[t]), xx, ag[m], false);
          au[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vu[t]), xx, au[m], false);
        }
      }
    }
  }
}

// The end of a half-wave's column: reduce the partial sums (or folds) over
// the 32 lanes, and lane 0 stores act(g) * u for the M rows (or the fold).
template <int M, Act A, bool kTwin>
__device__ __forceinline__ void finish_column(float (&ag)[M], float (&au)[M], uint32_t fold, bool live, int hl,
                                              int col, int N, float gmul, float umul, bf16* __restrict__ h,
                                              uint32_t* __restrict__ sink) {
  if constexpr (kTwin) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) fold ^= __shfl_xor(fold, off, 32);
    if (live && hl == 0) sink[col] = fold;
    return;
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

// x staged whole (M K * 2 <= kWholeBytes).
template <int M, Act A, bool kTwin>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const bf16* __restrict__ x,
                                                        const bf16* __restrict__ wg,
                                                        const bf16* __restrict__ wu,
                                                        bf16* __restrict__ h, int N, int K,
                                                        float gmul, float umul, uint32_t* __restrict__ sink) {
  extern __shared__ u32x4 xs[];  // [M][K / 8]
  const int nch = K >> 3;
  const int tid = threadIdx.x;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);
  for (int i = tid; i < M * nch; i += kThreads) xs[i] = xg[i];
  __syncthreads();

  const int lane = tid & 63;
  const int col0 = (blockIdx.x * (kThreads / 64) + (tid >> 6)) * 2;
  if (col0 >= N) return;                           // the whole wave is past the end
  const int col = col0 + (lane >> 5);
  const bool live = col < N;
  // A half-wave past the end streams the last column again and stores
  // nothing, so both halves stay active for the cross-half exchange.
  const int ccol = live ? col : N - 1;

  const u32x4* rg = reinterpret_cast<const u32x4*>(wg + (int64_t)ccol * K);
  const u32x4* ru = reinterpret_cast<const u32x4*>(wu + (int64_t)ccol * K);
  float ag[M], au[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ag[m] = au[m] = 0.0f;
  uint32_t fold = 0;
  stream_chunks<M, kTwin>(rg, ru, xs, nch, nch, lane, ag, au, fold);
  finish_column<M, A, kTwin>(ag, au, fold, live, lane & 31, col, N, gmul, umul, h, sink);
}

// x staged in phases of pch chunks per row (a multiple of 32): stage
// x[:, phase], stream the weights of that phase, move on.
template <int M, Act A, bool kTwin>
__global__ __launch_bounds__(kThreads) void gemv_phased_kernel(const bf16* __restrict__ x,
                                                               const bf16* __restrict__ wg,
                                                               const bf16* __restrict__ wu,
                                                               bf16* __restrict__ h, int N, int K, int pch,
                                                               float gmul, float umul,
                                                               uint32_t* __restrict__ sink) {
  extern __shared__ u32x4 xs[];  // [M][pch]
  const int nch = K >> 3;
  const int tid = threadIdx.x;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);

  const int lane = tid & 63;
  const int col0 = (blockIdx.x * (kThreads / 64) + (tid >> 6)) * 2;
  // A wave past the end still takes part in the staging and the barriers.
  const bool wave_live = col0 < N;
  const int col = col0 + (lane >> 5);
  const bool live = col < N;
  const int ccol = live ? col : N - 1;

  const u32x4* rg = reinterpret_cast<const u32x4*>(wg + (int64_t)ccol * K);
  const u32x4* ru = reinterpret_cast<const u32x4*>(wu + (int64_t)ccol * K);
  float ag[M], au[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ag[m] = au[m] = 0.0f;
  uint32_t fold = 0;
  for (int k0 = 0; k0 < nch; k0 += pch) {
    const int nc = min(pch, nch - k0);          // chunks of each row in this phase
    if (k0 > 0) __syncthreads();                // every wave is done with the last phase's x
    for (int i = tid; i < M * nc; i += kThreads) {
      const int m = i / nc, c = i - m * nc;
      xs[i] = xg[(int64_t)m * nch + k0 + c];
    }
    __syncthreads();
    if (wave_live) stream_chunks<M, kTwin>(rg + k0, ru + k0, xs, nc, nc, lane, ag, au, fold);
  }
  if (!wave_live) return;
  finish_column<M, A, kTwin>(ag, au, fold, live, lane & 31, col, N, gmul, umul, h, sink);
}

// Chunks of each x row per phase: the fewest equal phases of at most
// kPhaseBytes, each a multiple of 32 chunks (one pass of a half-wave), which
// may add up to 31 chunks per row to a phase.
inline int phase_chunks(int M, int K) {
  const int64_t nch = K / 8;
  const int64_t nph = ((int64_t)M * nch * 16 + kPhaseBytes - 1) / kPhaseBytes;
  const int64_t per = (nch + nph - 1) / nph;
  return (int)((per + 31) / 32 * 32);
}

template <int M, Act A, bool kTwin>
hipError_t launch_m(int N, int K, const void* x, const void* wg, const void* wu, void* h,
                    float gm, float um, uint32_t* sink, hipStream_t s) {
  const unsigned blocks = (unsigned)((N + kColsPerBlock - 1) / kColsPerBlock);
  const size_t whole = (size_t)M * K * 2;
  if (whole <= (size_t)kWholeBytes) {
    hipLaunchKernelGGL((gemv_kernel<M, A, kTwin>), dim3(blocks), dim3(kThreads), whole, s,
                       static_cast<const bf16*>(x), static_cast<const bf16*>(wg),
                       static_cast<const bf16*>(wu), static_cast<bf16*>(h), N, K, gm, um, sink);
  } else {
    const int pch = phase_chunks(M, K);
    const size_t lds = (size_t)M * pch * 16;     // at most 36 KiB + 31 chunks per row
    hipLaunchKernelGGL((gemv_phased_kernel<M, A, kTwin>), dim3(blocks), dim3(kThreads), lds, s,
                       static_cast<const bf16*>(x), static_cast<const bf16*>(wg),
                       static_cast<const bf16*>(wu), static_cast<bf16*>(h), N, K, pch, gm, um, sink);
  }
  return hipGetLastError();
}

template <Act A, bool kTwin>
hipError_t launch_act(int M, int N, int K, const void* x, const void* wg, const void* wu, void* h,
                      float gm, float um, uint32_t* sink, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 2: return launch_m<2, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 3: return launch_m<3, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 4: return launch_m<4, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 5: return launch_m<5, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 6: return launch_m<6, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 7: return launch_m<7, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 8: return launch_m<8, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(Act act, int M, int N, int K, const void* x, const void* wg, const void* wu,
                       void* h, float gmul, float umul, hipStream_t s) {
  return act == Act::kGeluTanh ? launch_act<Act::kGeluTanh, false>(M, N, K, x, wg, wu, h, gmul, umul, nullptr, s)
                               : launch_act<Act::kSilu, false>(M, N, K, x, wg, wu, h, gmul, umul, nullptr, s);
}

hipError_t launch_gemv_read_twin(int M, int N, int K, const void* x, const void* wg, const void* wu,
                                 uint32_t* sink, hipStream_t s) {
  return launch_act<Act::kSilu, true>(M, N, K, x, wg, wu, nullptr, 1.0f, 1.0f, sink, s);
}

}  // namespace swg
