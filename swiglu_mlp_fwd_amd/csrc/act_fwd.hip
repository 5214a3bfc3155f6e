// Elementwise gated activation without quantisation: h = act(g') * u' with
// g' = clamp(gate), u' = clamp(up), written as fp32 or bf16, plus the clamp
// count.
//
// "quant: add SwiGLU forward/backward VMI kernels" (TileKernels-PTO PR 20),
// performance section: the forward table runs the same SwiGLU with fp32 and
// bf16 outputs beside the e4m3 one, and the implementation notes keep a
// non-quantised output mode.  h is formed in fp64 from the fp32 inputs (the
// once-rounded values of the quantiser, fp8.hpp) and rounded once to the
// output type.
//
// Mapping as in the quantiser: the array is flat (the activation is
// elementwise), each lane takes 8 consecutive elements (two 16-byte loads
// per input) with kUnroll chunks' loads issued before any is used; the clamp
// count is reduced per workgroup into the workgroup's slot and the slots are
// summed by a second launch (count.hip).
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 8192;
static_assert(kMaxBlocks <= kCountSlots, "one count slot per workgroup");
constexpr int kUnroll = 4;

template <typename TO> __device__ __forceinline__ void store8(TO* h, int64_t c, const double (&v)[8]);
template <> __device__ __forceinline__ void store8<float>(float* h, int64_t c, const double (&v)[8]) {
  f32x4* p = reinterpret_cast<f32x4*>(h) + 2 * c;
  __builtin_nontemporal_store(f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}, p);
  __builtin_nontemporal_store(f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]}, p + 1);
}
template <> __device__ __forceinline__ void store8<bf16>(bf16* h, int64_t c, const double (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_bits_rne(v[2 * i]) | (bf16_bits_rne(v[2 * i + 1]) << 16);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(h) + c);
}

template <Act A, typename TO, bool kClamp, bool kCount>
__global__ __launch_bounds__(kThreads) void act_fwd_kernel(const float* __restrict__ gate,
                                                           const float* __restrict__ up, float L,
                                                           TO* __restrict__ h,
                                                           unsigned long long* __restrict__ count,
                                                           uint32_t* __restrict__ slots, int64_t nchunks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t cnt = 0;
  if (!kCount && count != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *count = 0ull;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < nchunks; c0 += kUnroll * stride) {
    f32x4 G0[kUnroll], G1[kUnroll], U0[kUnroll], U1[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = c0 + j * stride;
      if (c < nchunks) {
        const f32x4* gp = reinterpret_cast<const f32x4*>(gate) + 2 * c;
        const f32x4* up4 = reinterpret_cast<const f32x4*>(up) + 2 * c;
        G0[j] = __builtin_nontemporal_load(gp);
        G1[j] = __builtin_nontemporal_load(gp + 1);
        U0[j] = __builtin_nontemporal_load(up4);
        U1[j] = __builtin_nontemporal_load(up4 + 1);
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = c0 + j * stride;
      if (c >= nchunks) break;
      double v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g = e < 4 ? G0[j][e] : G1[j][e - 4];
        float u = e < 4 ? U0[j][e] : U1[j][e - 4];
        if (kClamp) {
          const bool cg = fabsf(g) > L, cu = fabsf(u) > L;   // false for NaN: passes uncounted
          if (kCount) cnt += (uint32_t)cg + (uint32_t)cu;
          g = cg ? copysignf(L, g) : g;
          u = cu ? copysignf(L, u) : u;
        }
        v[e] = A == Act::kGeluTanh ? gelu_value_d(g, u) : swiglu_value_d(g, u);
      }
      store8<TO>(h, c, v);
    }
  }
  if (kCount) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    __shared__ uint32_t wsum[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
      slots[blockIdx.x] = t;
    }
  }
}

template <Act A, typename TO>
void launch_typed(bool counting, bool clamp, unsigned grid, const float* gate, const float* up, float L,
                  void* h, uint64_t* count, uint32_t* slots, int64_t nchunks, hipStream_t s) {
  auto* cnt = reinterpret_cast<unsigned long long*>(count);
  TO* out = static_cast<TO*>(h);
  if (counting)
    hipLaunchKernelGGL((act_fwd_kernel<A, TO, true, true>), dim3(grid), dim3(kThreads), 0, s, gate, up, L, out, cnt,
                       slots, nchunks);
  else if (clamp)
    hipLaunchKernelGGL((act_fwd_kernel<A, TO, true, false>), dim3(grid), dim3(kThreads), 0, s, gate, up, L, out, cnt,
                       slots, nchunks);
  else
    hipLaunchKernelGGL((act_fwd_kernel<A, TO, false, false>), dim3(grid), dim3(kThreads), 0, s, gate, up, L, out, cnt,
                       slots, nchunks);
}

}  // namespace

hipError_t launch_act_fwd(Act act, Dt out, int64_t rows, int64_t cols, const float* gate, const float* up,
                          float limit, bool clamp, void* h, uint64_t* count, hipStream_t s) {
  const bool counting = clamp && count != nullptr;
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) {
    // Nothing to walk: a given counter receives 0.
    return count != nullptr ? launch_count_sum(nullptr, 0, count, s) : hipSuccess;
  }
  uint32_t* slots = nullptr;
  if (counting) {
    const hipError_t e = count_slots(s, &slots);
    if (e != hipSuccess) return e;
  }
  const int64_t want = (nchunks + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  if (act == Act::kGeluTanh) {
    if (out == Dt::kBF16) launch_typed<Act::kGeluTanh, bf16>(counting, clamp, grid, gate, up, limit, h, count, slots, nchunks, s);
    else launch_typed<Act::kGeluTanh, float>(counting, clamp, grid, gate, up, limit, h, count, slots, nchunks, s);
  } else {
    if (out == Dt::kBF16) launch_typed<Act::kSilu, bf16>(counting, clamp, grid, gate, up, limit, h, count, slots, nchunks, s);
    else launch_typed<Act::kSilu, float>(counting, clamp, grid, gate, up, limit, h, count, slots, nchunks, s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !counting) return e;
  return launch_count_sum(slots, (int)grid, count, s);
}

}  // namespace swg
