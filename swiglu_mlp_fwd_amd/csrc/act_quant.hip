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
// scale byte sits at scale[b].  The array is walked in spans of 512
// elements (128 16-byte vectors per input), one span per wave: lane l takes
// vectors 128 s + l and 128 s + 64 + l of span s, so every load and store
// instruction of a wave covers one contiguous range (1 KiB of each input).
// Eight lanes cover one block in each half of the span, and the block amax
// is reduced across them with three xor-shuffles.  The block exponent comes
// from the bits of amax (integer logic); the codes from the hardware FP8
// conversion of h * 2^-E.  (Each lane taking 8 consecutive elements instead,
// two adjacent 16-byte vectors, covers every 32-byte slot of a wave's range
// half per instruction: that layout streamed 1.7-1.8 times slower in a
// probe of the same bytes.)
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 8192;
static_assert(kMaxBlocks <= kCountSlots, "one count slot per workgroup");
// Units per lane per loop iteration.  At 4001 x 3584 (one unit per lane),
// with the earlier lane mapping, 8192 workgroups with 2 chunks in flight
// and non-temporal code stores measured 24.9 us against 25.8 us for 4096
// with 4 (the read-only twin moved the same way).
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
                                                             int64_t nvec, int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const f32x4* g4 = reinterpret_cast<const f32x4*>(gate);
  const f32x4* u4 = reinterpret_cast<const f32x4*>(up);
  const int lane = threadIdx.x & 63;
  uint32_t cnt = 0;
  // Without counting, a given counter just receives 0 (one store, no
  // separate zeroing launch).
  if (!kCount && count != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *count = 0ull;
  // Unit c (64 per span, consecutive in a wave) is lane c % 64 of span
  // c / 64.  kUnroll units per lane per iteration (grid-stride apart): all
  // their loads are issued before any is used, for more bytes in flight.
  // units and the strides are multiples of 64, so a wave is either wholly
  // inside the walk or wholly past it; within the last span a half is live
  // when its vector lies inside the array (whole blocks, since 32 | n).
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
      if constexpr (kTwin) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int64_t v = v0 + 64 * hf;      // vector index; elements 4 v .. 4 v + 3, block v / 8
          const f32x4 g4v = G[j][hf], u4v = U[j][hf];
          const uint32_t f = f32_bits(g4v[0]) ^ f32_bits(g4v[1]) ^ f32_bits(g4v[2]) ^ f32_bits(g4v[3]) ^
                             f32_bits(u4v[0]) ^ f32_bits(u4v[1]) ^ f32_bits(u4v[2]) ^ f32_bits(u4v[3]);
          if (v < nvec) {
            __builtin_nontemporal_store(f, reinterpret_cast<uint32_t*>(q + 4 * v));
            if ((lane & 7) == 0) scale[v >> 3] = (uint8_t)f;
          }
        }
        continue;
      }
      // Both halves' values first, then their two amax reductions side by
      // side, then the codes: the halves' work interleaves.
      float h[2][4];
      float amax[2] = {0.0f, 0.0f};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float g = G[j][hf][e], u = U[j][hf][e];
          if (kClamp) {
            // |v| > L is false for NaN, so NaN passes through uncounted.
            const bool cg = fabsf(g) > L, cu = fabsf(u) > L;
            if (kCount) cnt += (uint32_t)cg + (uint32_t)cu;
            g = cg ? copysignf(L, g) : g;
            u = cu ? copysignf(L, u) : u;
          }
          h[hf][e] = A == Act::kGeluTanh ? gelu_value(g, u) : swiglu_value(g, u);
          amax[hf] = fmaxf(amax[hf], fabsf(h[hf][e]));   // maxNum: NaN operands are ignored
        }
#pragma unroll
      for (int m = 1; m <= 4; m <<= 1) {
        amax[0] = fmaxf(amax[0], __shfl_xor(amax[0], m));
        amax[1] = fmaxf(amax[1], __shfl_xor(amax[1], m));
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int64_t v = v0 + 64 * hf;        // vector index; elements 4 v .. 4 v + 3, block v / 8
        const int E = block_exponent(amax[hf]);
        const float sc = ldexpf(1.0f, -E);
        const uint32_t codes = e4m3_pair(h[hf][0], h[hf][1], sc) | (e4m3_pair(h[hf][2], h[hf][3], sc) << 16);
        if (v < nvec) {
          __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t*>(q + 4 * v));
          if ((lane & 7) == 0) scale[v >> 3] = (uint8_t)(E + 127);
          if (kHout) reinterpret_cast<f32x4*>(hout)[v] = f32x4{h[hf][0], h[hf][1], h[hf][2], h[hf][3]};
        }
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

// The walk: nvec 16-byte vectors per input, in spans of 128; 64 units per
// span; a grid of at most kMaxBlocks workgroups.
struct Walk {
  int64_t nvec, units;
  unsigned grid;
};
inline Walk walk_of(int64_t rows, int64_t cols) {
  Walk w;
  w.nvec = rows * cols / 4;
  w.units = (w.nvec + 127) / 128 * 64;
  const int64_t want = (w.units + kThreads - 1) / kThreads;
  w.grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  return w;
}

template <Act A, bool kClamp, bool kCount, bool kHout>
void launch_aq(const Walk& w, const float* gate, const float* up, float L, uint8_t* q,
               uint8_t* scale, uint64_t* count, uint32_t* slots, float* hout, hipStream_t s) {
  hipLaunchKernelGGL((act_quant_kernel<A, kClamp, kCount, kHout>), dim3(w.grid), dim3(kThreads), 0, s,
                     gate, up, L, q, scale, reinterpret_cast<unsigned long long*>(count), slots, hout,
                     w.nvec, w.units);
}

template <Act A>
void launch_aq_variant(bool counting, bool clamp, const Walk& w, const float* gate, const float* up,
                       float limit, uint8_t* q, uint8_t* scale, uint64_t* count, uint32_t* slots, float* hout,
                       hipStream_t s) {
  // The count is only accumulated when a counter is given and the clamp is
  // on; with the clamp off no value can exceed the limit.
  if (counting) {
    if (hout) launch_aq<A, true, true, true>(w, gate, up, limit, q, scale, count, slots, hout, s);
    else launch_aq<A, true, true, false>(w, gate, up, limit, q, scale, count, slots, hout, s);
  } else if (clamp) {
    if (hout) launch_aq<A, true, false, true>(w, gate, up, limit, q, scale, count, slots, hout, s);
    else launch_aq<A, true, false, false>(w, gate, up, limit, q, scale, count, slots, hout, s);
  } else {
    if (hout) launch_aq<A, false, false, true>(w, gate, up, limit, q, scale, count, slots, hout, s);
    else launch_aq<A, false, false, false>(w, gate, up, limit, q, scale, count, slots, hout, s);
  }
}

}  // namespace

hipError_t launch_act_quant_twin(int64_t rows, int64_t cols, const float* gate, const float* up, uint8_t* q,
                                 uint8_t* scale, hipStream_t s) {
  const Walk w = walk_of(rows, cols);
  if (w.nvec == 0) return hipSuccess;
  hipLaunchKernelGGL((act_quant_kernel<Act::kSilu, false, false, false, true>), dim3(w.grid), dim3(kThreads), 0, s,
                     gate, up, 0.0f, q, scale, nullptr, nullptr, nullptr, w.nvec, w.units);
  return hipGetLastError();
}

hipError_t launch_act_quant(Act act, int64_t rows, int64_t cols, const float* gate, const float* up,
                            float limit, bool clamp, uint8_t* q, uint8_t* scale, uint64_t* count,
                            float* hout, hipStream_t s) {
  const bool counting = clamp && count != nullptr;
  const Walk w = walk_of(rows, cols);
  if (w.nvec == 0) {
    // Nothing to walk: a given counter receives 0.
    return count != nullptr ? launch_count_sum(nullptr, 0, count, s) : hipSuccess;
  }
  uint32_t* slots = nullptr;
  if (counting) {
    const hipError_t e = count_slots(s, &slots);
    if (e != hipSuccess) return e;
  }
  if (act == Act::kGeluTanh)
    launch_aq_variant<Act::kGeluTanh>(counting, clamp, w, gate, up, limit, q, scale, count, slots, hout, s);
  else
    launch_aq_variant<Act::kSilu>(counting, clamp, w, gate, up, limit, q, scale, count, slots, hout, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !counting) return e;
  return launch_count_sum(slots, (int)w.grid, count, s);
}

}  // namespace swg
