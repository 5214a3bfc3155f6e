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
// elementwise) and walked in spans of 512 elements, one per wave, lane l
// taking 16-byte vectors 128 s + l and 128 s + 64 + l of span s, so each
// load and store instruction of a wave covers one contiguous range; kUnroll
// units' loads are issued before any is used.  The clamp count is reduced
// per workgroup into the workgroup's slot and the slots are summed by a
// second launch (count.hip).
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 8192;
static_assert(kMaxBlocks <= kCountSlots, "one count slot per workgroup");
constexpr int kUnroll = 4;

template <typename TO> __device__ __forceinline__ void store4(TO* h, int64_t v, const double (&r)[4]);
template <> __device__ __forceinline__ void store4<float>(float* h, int64_t v, const double (&r)[4]) {
  __builtin_nontemporal_store(f32x4{(float)r[0], (float)r[1], (float)r[2], (float)r[3]}, reinterpret_cast<f32x4*>(h) + v);
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* h, int64_t v, const double (&r)[4]) {
  const u32x2 w = {bf16_bits_rne(r[0]) | (bf16_bits_rne(r[1]) << 16), bf16_bits_rne(r[2]) | (bf16_bits_rne(r[3]) << 16)};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(h) + v);
}

template <Act A, typename TO, bool kClamp, bool kCount>
__global__ __launch_bounds__(kThreads) void act_fwd_kernel(const float* __restrict__ gate,
                                                           const float* __restrict__ up, float L,
                                                           TO* __restrict__ h,
                                                           unsigned long long* __restrict__ count,
                                                           uint32_t* __restrict__ slots, int64_t nvec, int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const f32x4* g4 = reinterpret_cast<const f32x4*>(gate);
  const f32x4* u4 = reinterpret_cast<const f32x4*>(up);
  uint32_t cnt = 0;
  if (!kCount && count != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *count = 0ull;
  // Unit c is lane c % 64 of span c / 64 (the quantiser's walk).
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < units; c0 += kUnroll * stride) {
    f32x4 G[kUnroll][2], U[kUnroll][2];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = c0 + j * stride;
      const int64_t v0 = (c >> 6) * 128 + (c & 63);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int64_t v = v0 + 64 * hf;
        const bool in = c < units && v < nvec;
        G[j][hf] = in ? __builtin_nontemporal_load(g4 + v) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        U[j][hf] = in ? __builtin_nontemporal_load(u4 + v) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = c0 + j * stride;
      if (c >= units) break;
      const int64_t v0 = (c >> 6) * 128 + (c & 63);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int64_t v = v0 + 64 * hf;
        if (v >= nvec) continue;
        double r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float g = G[j][hf][e], u = U[j][hf][e];
          if (kClamp) {
            const bool cg = fabsf(g) > L, cu = fabsf(u) > L;   // false for NaN: passes uncounted
            if (kCount) cnt += (uint32_t)cg + (uint32_t)cu;
            g = cg ? copysignf(L, g) : g;
            u = cu ? copysignf(L, u) : u;
          }
          r[e] = A == Act::kGeluTanh ? gelu_value_d(g, u) : swiglu_value_d(g, u);
        }
        store4<TO>(h, v, r);
      }
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
                  void* h, uint64_t* count, uint32_t* slots, int64_t nvec, int64_t units, hipStream_t s) {
  auto* cnt = reinterpret_cast<unsigned long long*>(count);
  TO* out = static_cast<TO*>(h);
  if (counting)
    hipLaunchKernelGGL((act_fwd_kernel<A, TO, true, true>), dim3(grid), dim3(kThreads), 0, s, gate, up, L, out, cnt,
                       slots, nvec, units);
  else if (clamp)
    hipLaunchKernelGGL((act_fwd_kernel<A, TO, true, false>), dim3(grid), dim3(kThreads), 0, s, gate, up, L, out, cnt,
                       slots, nvec, units);
  else
    hipLaunchKernelGGL((act_fwd_kernel<A, TO, false, false>), dim3(grid), dim3(kThreads), 0, s, gate, up, L, out, cnt,
                       slots, nvec, units);
}

}  // namespace

hipError_t launch_act_fwd(Act act, Dt out, int64_t rows, int64_t cols, const float* gate, const float* up,
                          float limit, bool clamp, void* h, uint64_t* count, hipStream_t s) {
  const bool counting = clamp && count != nullptr;
  const int64_t nvec = rows * cols / 4;
  const int64_t units = (nvec + 127) / 128 * 64;
  if (nvec == 0) {
    // Nothing to walk: a given counter receives 0.
    return count != nullptr ? launch_count_sum(nullptr, 0, count, s) : hipSuccess;
  }
  uint32_t* slots = nullptr;
  if (counting) {
    const hipError_t e = count_slots(s, &slots);
    if (e != hipSuccess) return e;
  }
  const int64_t want = (units + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  if (act == Act::kGeluTanh) {
    if (out == Dt::kBF16) launch_typed<Act::kGeluTanh, bf16>(counting, clamp, grid, gate, up, limit, h, count, slots, nvec, units, s);
    else launch_typed<Act::kGeluTanh, float>(counting, clamp, grid, gate, up, limit, h, count, slots, nvec, units, s);
  } else {
    if (out == Dt::kBF16) launch_typed<Act::kSilu, bf16>(counting, clamp, grid, gate, up, limit, h, count, slots, nvec, units, s);
    else launch_typed<Act::kSilu, float>(counting, clamp, grid, gate, up, limit, h, count, slots, nvec, units, s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !counting) return e;
  return launch_count_sum(slots, (int)grid, count, s);
}

}  // namespace swg
