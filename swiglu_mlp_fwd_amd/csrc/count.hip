// Clamp counts of the elementwise kernels without same-address atomics.
//
// "quant: add SwiGLU forward/backward VMI kernels" (TileKernels-PTO PR 20),
// overview: the clamp comes with a count of the clamped values.  Adding
// every workgroup's count to the caller's uint64 with one atomic each
// serialises at one L2 channel (8192 workgroups: about 66 us at 4001 x 3584,
// against 25 us for the whole pass without a count) and would need the
// uint64 cleared by a launch of its own first.  Instead each workgroup of a
// counting launch writes its count to its own slot, and one small kernel
// then sums the slots into the caller's uint64 (so nothing needs clearing).
//
// The slots are a file-scope device array of 16 regions of 8192 slots; each
// counting call takes the next region in turn, so up to 16 counting calls
// may be in flight on one GPU at once (a captured graph keeps the region it
// was captured with).
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kRegions = 16;
static __device__ __align__(256) uint32_t count_slot_array[kRegions][kCountSlots];

// The sum: 1024 threads, each with its 8 slots in two 16-byte loads issued
// together, so the launch waits for one memory round trip, then a tree in LDS.
constexpr int kSumThreads = 1024;
constexpr int kPerThread = kCountSlots / kSumThreads;
static_assert(kPerThread == 8, "two 16-byte loads per thread");

__global__ __launch_bounds__(kSumThreads) void sum_slots_kernel(const uint32_t* __restrict__ slots, int n,
                                                                unsigned long long* __restrict__ out) {
  __shared__ unsigned long long part[kSumThreads];
  const int i0 = threadIdx.x * kPerThread;
  unsigned long long t = 0;
  if (i0 + kPerThread <= n) {
    // slots is 32-byte aligned (regions of 8192 slots from a 256-byte aligned base)
    const u32x4 a = reinterpret_cast<const u32x4*>(slots + i0)[0];
    const u32x4 b = reinterpret_cast<const u32x4*>(slots + i0)[1];
    t = (unsigned long long)a[0] + a[1] + a[2] + a[3] + b[0] + b[1] + b[2] + b[3];
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (i0 + e < n) t += slots[i0 + e];
  }
  part[threadIdx.x] = t;
  __syncthreads();
#pragma unroll
  for (int w = kSumThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = part[0];
}

// Device address of the slot array on device dev (each GPU holds its own
// copy), looked up on the first call on that device.
hipError_t slot_array_address(int dev, uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t result[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    result[dev] = symbol_address_on(dev, HIP_SYMBOL(count_slot_array), &p);
    addr[dev] = p;
  });
  *out = static_cast<uint32_t*>(addr[dev]);
  return result[dev];
}

std::atomic<uint32_t> next_region{0};

}  // namespace

hipError_t count_slots(hipStream_t s, uint32_t** slots) {
  int dev = 0;
  hipError_t e = stream_device(s, &dev);
  if (e != hipSuccess) return e;
  uint32_t* base = nullptr;
  e = slot_array_address(dev, &base);
  if (e != hipSuccess) return e;
  const uint32_t r = next_region.fetch_add(1, std::memory_order_relaxed) % kRegions;
  *slots = base + (size_t)r * kCountSlots;
  return hipSuccess;
}

hipError_t launch_count_sum(const uint32_t* slots, int nblocks, uint64_t* count, hipStream_t s) {
  if (nblocks < 0 || nblocks > kCountSlots) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sum_slots_kernel, dim3(1), dim3(kSumThreads), 0, s, slots, nblocks,
                     reinterpret_cast<unsigned long long*>(count));
  return hipGetLastError();
}

}  // namespace swg
