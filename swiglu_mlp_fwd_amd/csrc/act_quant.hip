// Elementwise SwiGLU (or GeGLU) with FP8 (E4M3FN) 1x32 block quantisation,
// one pass.
//
// "quant: add SwiGLU forward/backward VMI kernels" (TileKernels-PTO PR 20),
// overview and implementation notes: an optional clamp with a count of the
// clamped values, h = SiLU(gate) * up, one scale per 32 consecutive elements
// of a row stored packed as a UE8M0 byte, and an E4M3 cast without
// saturation that keeps NaN; validation covers subnormal inputs, non-finite
// inputs and the packed scale of a block whose amax is infinite.
//
// Mapping: with cols % 32 == 0 the 1x32 blocks tile the flattened
// [rows, cols] array, so block b covers elements [32 b, 32 b + 32) and its
// scale byte sits at scale[b].  Each lane handles 8 consecutive elements
// (two 16-byte loads per input), a quad of 4 lanes covers one block, and the
// block amax is reduced across the quad with two xor-shuffles.  The block
// exponent comes from the bits of amax (integer logic); the codes from the
// hardware FP8 conversion of h * 2^-E.
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 8192;
static_assert(kMaxBlocks <= kCountSlots, "one count slot per workgroup");
// Chunks per lane per loop iteration.  At 4001 x 3584, 8192 workgroups with
// 2 chunks in flight and non-temporal code stores measured 24.9 us against
// 25.8 us for 4096 with 4 (the read-only twin moved the same way).
constexpr int kUnroll = 2;

// kTwin: the same kernel with the same grid, loads and stores and no
// arithmetic (the stored bytes are folds of the loaded words): the floor of
// this kernel's byte pattern, 8 bytes read and 1 + 1/32 written per element.
template <Act A, bool kClamp, bool kCount, bool kHout, bool kTwin = false>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(const float* __restrict__ gate,
                                                             const float* __restrict__ up, float L,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scale,
                                                             unsigned long long* __restrict__ count,
                                                             uint32_t* __restrict__ slots,
                                                             float* __restrict__ hout,
                                                             int64_t nchunks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t cnt = 0;
  // Without counting, a given counter just receives 0 (one store, no
  // separate zeroing launch).
  if (!kCount && count != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *count = 0ull;
  // kUnroll chunks per lane per iteration (grid-stride apart): all their
  // loads are issued before any is used, for more bytes in flight.
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
    const f32x4 g0 = G0[j], g1 = G1[j], u0 = U0[j], u1 = U1[j];
    if constexpr (kTwin) {
      const uint32_t lo = f32_bits(g0[0]) ^ f32_bits(g0[1]) ^ f32_bits(g0[2]) ^ f32_bits(g0[3]) ^ f32_bits(u0[0]) ^
                          f32_bits(u0[1]) ^ f32_bits(u0[2]) ^ f32_bits(u0[3]);
      const uint32_t hi = f32_bits(g1[0]) ^ f32_bits(g1[1]) ^ f32_bits(g1[2]) ^ f32_bits(g1[3]) ^ f32_bits(u1[0]) ^
                          f32_bits(u1[1]) ^ f32_bits(u1[2]) ^ f32_bits(u1[3]);
      __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(q + 8 * c));
      if ((threadIdx.x & 3) == 0) scale[c >> 2] = (uint8_t)(lo ^ hi);
      continue;
    }
    float h[8];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float g = e < 4 ? g0[e] : g1[e - 4];
      float u = e < 4 ? u0[e] : u1[e - 4];
      if (kClamp) {
        // |v| > L is false for NaN, so NaN passes through uncounted.
        const bool cg = fabsf(g) > L, cu = fabsf(u) > L;
        if (kCount) cnt += (uint32_t)cg + (uint32_t)cu;
        g = cg ? copysignf(L, g) : g;
        u = cu ? copysignf(L, u) : u;
      }
      h[e] = A == Act::kGeluTanh ? gelu_value(g, u) : swiglu_value(g, u);
      amax = fmaxf(amax, fabsf(h[e]));  // maxNum: NaN operands are ignored
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int E = block_exponent(amax);
    const float sc = ldexpf(1.0f, -E);
    const uint32_t lo = e4m3_pair(h[0], h[1], sc) | (e4m3_pair(h[2], h[3], sc) << 16);
    const uint32_t hi = e4m3_pair(h[4], h[5], sc) | (e4m3_pair(h[6], h[7], sc) << 16);
    __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(q + 8 * c));
    if ((threadIdx.x & 3) == 0) scale[c >> 2] = (uint8_t)(E + 127);
    if (kHout) {
      f32x4* hp = reinterpret_cast<f32x4*>(hout) + 2 * c;
      hp[0] = f32x4{h[0], h[1], h[2], h[3]};
      hp[1] = f32x4{h[4], h[5], h[6], h[7]};
    }
    }
  }
  if (kCount) {
    // Wave sums, then the workgroup's count into its own slot (summed into
    // the caller's count by the next launch).
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

template <Act A, bool kClamp, bool kCount, bool kHout>
void launch_aq(unsigned grid, const float* gate, const float* up, float L, uint8_t* q,
               uint8_t* scale, uint64_t* count, uint32_t* slots, float* hout, int64_t nchunks, hipStream_t s) {
  hipLaunchKernelGGL((act_quant_kernel<A, kClamp, kCount, kHout>), dim3(grid), dim3(kThreads), 0, s,
                     gate, up, L, q, scale, reinterpret_cast<unsigned long long*>(count), slots, hout,
                     nchunks);
}

template <Act A>
void launch_aq_variant(bool counting, bool clamp, unsigned grid, const float* gate, const float* up,
                       float limit, uint8_t* q, uint8_t* scale, uint64_t* count, uint32_t* slots, float* hout,
                       int64_t nchunks, hipStream_t s) {
  // The count is only accumulated when a counter is given and the clamp is
  // on; with the clamp off no value can exceed the limit.
  if (counting) {
    if (hout) launch_aq<A, true, true, true>(grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
    else launch_aq<A, true, true, false>(grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
  } else if (clamp) {
    if (hout) launch_aq<A, true, false, true>(grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
    else launch_aq<A, true, false, false>(grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
  } else {
    if (hout) launch_aq<A, false, false, true>(grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
    else launch_aq<A, false, false, false>(grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
  }
}

}  // namespace

hipError_t launch_act_quant_twin(int64_t rows, int64_t cols, const float* gate, const float* up, uint8_t* q,
                                 uint8_t* scale, hipStream_t s) {
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) return hipSuccess;
  const int64_t want = (nchunks + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  hipLaunchKernelGGL((act_quant_kernel<Act::kSilu, false, false, false, true>), dim3(grid), dim3(kThreads), 0, s,
                     gate, up, 0.0f, q, scale, nullptr, nullptr, nullptr, nchunks);
  return hipGetLastError();
}

hipError_t launch_act_quant(Act act, int64_t rows, int64_t cols, const float* gate, const float* up,
                            float limit, bool clamp, uint8_t* q, uint8_t* scale, uint64_t* count,
                            float* hout, hipStream_t s) {
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
  if (act == Act::kGeluTanh)
    launch_aq_variant<Act::kGeluTanh>(counting, clamp, grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
  else
    launch_aq_variant<Act::kSilu>(counting, clamp, grid, gate, up, limit, q, scale, count, slots, hout, nchunks, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !counting) return e;
  return launch_count_sum(slots, (int)grid, count, s);
}

}  // namespace swg
