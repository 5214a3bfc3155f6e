// Cold-read floor probe: stream two buffers once with 16-byte loads and do
// nothing with the data but fold it into one word per workgroup.  This is the
// "pure-read loop" of "Fused SwiGLU benchmark" (AstrAI
// docs/developer/swiglu_benchmark.md, section HBM re-measurement), against
// which the decode kernel's weight stream is compared on the same rotated
// buffers.
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 4096;

__global__ __launch_bounds__(kThreads) void probe_read2_kernel(const u32x4* __restrict__ a,
                                                               const u32x4* __restrict__ b,
                                                               int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __builtin_nontemporal_load(a + i + j * stride);
      v[2 * j + 1] = __builtin_nontemporal_load(b + i + j * stride);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 va = __builtin_nontemporal_load(a + i);
    const u32x4 vb = __builtin_nontemporal_load(b + i);
    acc ^= va[0] ^ va[1] ^ va[2] ^ va[3] ^ vb[0] ^ vb[1] ^ vb[2] ^ vb[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// The same pure read with a chosen shape: kT threads per workgroup, kU
// 16-byte chunks of each buffer in flight per lane, a grid of up to
// max_blocks workgroups (grid-stride beyond).  The fastest of a few shapes
// is the floor: at 21 MB per buffer 256 or 512 threads with 2-8 chunks in
// flight read 8-10 % faster than the fixed shape above, at 90 MB 512 threads
// with 1 chunk and a grid covering the buffers in one pass 9-16 % faster
// (several runs).  A lane stores its fold only
// in the practically impossible case that it equals kNever, which keeps the
// loads from being elided without a reduction at the end of every
// workgroup (that reduction alone cost 0.5 us of an 8 us read).
constexpr uint32_t kNever = 0x9E3779B9u;

template <int kT, int kU>
__global__ __launch_bounds__(kT) void probe_read2_cfg_kernel(const u32x4* __restrict__ a,
                                                             const u32x4* __restrict__ b, int64_t n16,
                                                             uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kT;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  for (; i + (kU - 1) * stride < n16; i += kU * stride) {
    u32x4 v[2 * kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      v[2 * j] = __builtin_nontemporal_load(a + i + j * stride);
      v[2 * j + 1] = __builtin_nontemporal_load(b + i + j * stride);
    }
#pragma unroll
    for (int j = 0; j < 2 * kU; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 va = __builtin_nontemporal_load(a + i);
    const u32x4 vb = __builtin_nontemporal_load(b + i);
    acc ^= va[0] ^ va[1] ^ va[2] ^ va[3] ^ vb[0] ^ vb[1] ^ vb[2] ^ vb[3];
  }
  if (acc == kNever) sink[blockIdx.x & 4095] = acc;
}

template <int kT, int kU>
void launch_read2_cfg(const void* a, const void* b, int64_t n16, int max_blocks, uint32_t* sink, hipStream_t s) {
  const int64_t want = (n16 + (int64_t)kT * kU - 1) / ((int64_t)kT * kU);
  const unsigned grid = (unsigned)(want < max_blocks ? want : max_blocks);
  hipLaunchKernelGGL((probe_read2_cfg_kernel<kT, kU>), dim3(grid), dim3(kT), 0, s, static_cast<const u32x4*>(a),
                     static_cast<const u32x4*>(b), n16, sink);
}

// Matrix-core ceiling probe: back-to-back v_mfma_f32_16x16x32_bf16 (the
// form the forward and the dX/dW products use) on register operands, eight
// independent accumulator chains per wave, eight waves per workgroup, no
// memory traffic in the loop.  The operands are
// lane-dependent bf16 values of magnitude 2^-7..2^-6 with random signs, so
// the datapath toggles as it does on real data.  What it measures is the
// dense bf16 rate the chip sustains under its power and clock limits, the
// ceiling a GEMM kernel can approach.
constexpr int kMfmaThreads = 512;

__global__ __launch_bounds__(kMfmaThreads) void probe_mfma_kernel(int iters, float* sink) {
  const uint32_t tid = blockIdx.x * kMfmaThreads + threadIdx.x;
  u32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t ha = (tid * 2654435761u) ^ (0x9E3779B9u * (uint32_t)(j + 1));
    uint32_t hb = (tid * 2246822519u) ^ (0x85EBCA6Bu * (uint32_t)(j + 7));
    ha ^= ha >> 15;
    hb ^= hb >> 13;
    // Two bf16 per word: exponent 120 (2^-7), random mantissa and sign.
    a[j] = (0x3C003C00u | (ha & 0x007F007Fu)) | (ha & 0x80008000u);
    b[j] = (0x3C003C00u | (hb & 0x007F007Fu)) | (hb & 0x80008000u);
  }
  const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[c][e] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[c][e];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

// Exhaustive check aid for the FP8 encoders: over the fp32 bit patterns
// [first, last], each thread walks a contiguous run and reports `first` and
// every pattern p whose result differs from that of p - 1, as the pair
// (p, result) (atomic append; the order of the list is arbitrary).  kind 0: the E4M3 code of the value at
// scale 1 (e4m3_pair, the path of every quantiser); kind 1: the UE8M0 byte of
// the value taken as a block amax (block_exponent).  On a run of patterns
// of one sign the value is monotone in the pattern, and both functions are
// monotone step functions of the value, so the list determines every result.
__device__ __forceinline__ uint32_t encode_probe(uint32_t p, int kind) {
  const float v = bits_f32(p);
  if (kind == 0) return e4m3_pair(v, 0.0f, 1.0f) & 0xFFu;
  return (uint32_t)(block_exponent(v) + 127);
}

constexpr int kRun = 4096;     // patterns per thread

__global__ __launch_bounds__(256) void probe_transitions_kernel(uint32_t first, uint32_t last, int kind,
                                                                uint32_t* __restrict__ out, uint32_t capacity,
                                                                uint32_t* __restrict__ count) {
  const uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t lo = (uint64_t)first + t * kRun;
  if (lo > last) return;
  const uint64_t hi = min((uint64_t)last, lo + kRun - 1);
  // The first pattern of the range always starts a run.
  uint32_t prev = lo > first ? encode_probe((uint32_t)(lo - 1), kind) : ~0u;
  for (uint64_t p = lo; p <= hi; ++p) {
    const uint32_t c = encode_probe((uint32_t)p, kind);
    if (c != prev) {
      const uint32_t i = atomicAdd(count, 1u);
      if (i < capacity) {
        out[2 * i] = (uint32_t)p;
        out[2 * i + 1] = c;
      }
    }
    prev = c;
  }
}

}  // namespace

hipError_t launch_probe_transitions(uint32_t first, uint32_t last, int kind, uint32_t* out, uint32_t capacity,
                                    uint32_t* count, hipStream_t s) {
  const uint64_t n = (uint64_t)last - first + 1;
  const uint64_t threads = (n + kRun - 1) / kRun;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(probe_transitions_kernel, dim3(grid), dim3(256), 0, s, first, last, kind, out, capacity, count);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int blocks, float* sink, hipStream_t s) {
  if (iters <= 0 || blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_read2_cfg(const void* a, const void* b, size_t bytes, int threads, int chunks,
                                  int max_blocks, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int key = threads * 16 + chunks;
  switch (key) {
    case 256 * 16 + 1: launch_read2_cfg<256, 1>(a, b, n16, max_blocks, sink, s); break;
    case 256 * 16 + 2: launch_read2_cfg<256, 2>(a, b, n16, max_blocks, sink, s); break;
    case 256 * 16 + 4: launch_read2_cfg<256, 4>(a, b, n16, max_blocks, sink, s); break;
    case 256 * 16 + 8: launch_read2_cfg<256, 8>(a, b, n16, max_blocks, sink, s); break;
    case 512 * 16 + 1: launch_read2_cfg<512, 1>(a, b, n16, max_blocks, sink, s); break;
    case 512 * 16 + 2: launch_read2_cfg<512, 2>(a, b, n16, max_blocks, sink, s); break;
    case 512 * 16 + 4: launch_read2_cfg<512, 4>(a, b, n16, max_blocks, sink, s); break;
    case 512 * 16 + 8: launch_read2_cfg<512, 8>(a, b, n16, max_blocks, sink, s); break;
    default: return hipErrorInvalidValue;             // the caller checks the shape first
  }
  return hipGetLastError();
}

hipError_t launch_probe_read2(const void* a, const void* b, size_t bytes, uint32_t* sink,
                              hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t want = (n16 + kThreads * 4 - 1) / (kThreads * 4);
  const unsigned grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
  hipLaunchKernelGGL(probe_read2_kernel, dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(a), static_cast<const u32x4*>(b), n16, sink);
  return hipGetLastError();
}

}  // namespace swg
