// Internal launch interface of the GEMM-shaped kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace swg {

// C[m, n] = sum_r A[m, r] * B[n, r]: both operands have the reduction index
// contiguous (the nn.Linear layout), so one kernel family serves the forward
// dual GEMM and, after transposes, every backward contraction.
struct GemmArgs {
  const void* a;       // A [arows, r], row stride lda (elements)
  const void* b0;      // B0 [brows, r], row stride ldb
  const void* b1;      // B1 [brows, r] (dual only)
  int64_t lda, ldb;
  int arows, brows;    // rows of A / B that exist; rows beyond read as zero
  int m, n, r;         // output tile space m x n; reduction length r
  // epilogue
  void* out0;
  void* out1;
  int64_t ldo;         // row stride of outputs (elements)
  int split;           // store: rows < split go to out0, others to out1 (row - split)
  int lim0, lim1;      // store: rows of out0 / out1 that exist
  int ncols;           // columns of the output that exist (store / swiglu)
  const void* dh;      // dswiglu: upstream gradient [arows, ncols], row stride lddh
  int64_t lddh;
  int du_off;          // dswiglu: du is written at column du_off + n of out0
  int64_t ldt;         // dswiglu with out1 != null: out1 receives out0 transposed,
                       // [2 du_off, ldt] with rows m in [arows, ldt) zero (bf16 only)
  // FP8-output forward: E4M3 codes in out0 (row stride ldo bytes), UE8M0
  // scale bytes in q_scale (row stride n / 32), optional fp32 h in q_h (ldo).
  void* q_scale;
  float* q_h;
  // Gated epilogues (forward, FP8 forward, dswiglu): the projections are
  // scaled before use, g <- gmul * g and u <- umul * u (1 leaves them exact).
  float gmul = 1.0f, umul = 1.0f;
};

enum class Dt { kF32 = 0, kBF16 = 1 };
enum class Act { kSilu = 0, kGeluTanh = 1 };   // the gate activation of the gated forward

// Allows `Kernel` up to `lds` bytes of dynamic LDS (the default limit is
// 64 KiB; gfx950 has 160 KiB per workgroup).  The attribute belongs to the
// kernel on the current device, so it is set once per (kernel, device) with
// the largest size that kernel is ever launched with; concurrent first calls
// are serialised by call_once.
template <auto Kernel>
hipError_t allow_lds(size_t lds) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static hipError_t result[kMaxDevices];
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto set = [&] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds);
  };
  if (dev < 0 || dev >= kMaxDevices) return set();
  std::call_once(once[dev], [&] { result[dev] = set(); });
  return result[dev];
}

// The device a stream belongs to (the current device for the null stream).
inline hipError_t stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(s, &d);
  if (e != hipSuccess) return e;
  *dev = (int)d;
  return hipSuccess;
}

// The address of a file-scope __device__ array on device `dev` (each GPU
// holds its own copy at its own address): dev is made current for the
// lookup and the caller's current device restored.
inline hipError_t symbol_address_on(int dev, const void* symbol, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  e = hipGetSymbolAddress(out, symbol);
  if (cur != dev) {
    const hipError_t r = hipSetDevice(cur);
    if (e == hipSuccess) e = r;
  }
  return e;
}

hipError_t launch_fwd_dual(Dt dt, Act act, const GemmArgs& a, hipStream_t s);  // h = act(g) * u
// bf16 inputs, h = act(g) * u quantised per 1x32 block (n % 32 == 0).
hipError_t launch_fwd_dual_fp8(Act act, const GemmArgs& a, hipStream_t s);
hipError_t launch_bwd_dswiglu(Dt dt, Act act, const GemmArgs& a, hipStream_t s);   // D = [dg | du]
hipError_t launch_gemm_store(Dt dt, const GemmArgs& a, hipStream_t s);    // C = A B^T

// out[c, col_off + r] = in[r, c] for r < rows, 0 for rows <= r < rows_pad.
hipError_t launch_transpose(Dt dt, const void* in, int64_t ld_in, int rows, int cols,
                            void* out, int64_t ld_out, int col_off, int rows_pad,
                            hipStream_t s);

hipError_t launch_gemv(Act act, int M, int N, int K, const void* x, const void* wg, const void* wu,
                       void* h, float gmul, float umul, hipStream_t s);

// The decode kernel's read-only twin: the same grid, LDS and weight loads,
// no arithmetic; sink receives one word per column.
hipError_t launch_gemv_read_twin(int M, int N, int K, const void* x, const void* wg, const void* wu,
                                 uint32_t* sink, hipStream_t s);

// Clamp counts without same-address atomics (count.hip): a counting launch
// of at most kCountSlots workgroups writes workgroup b's count to slots[b],
// then launch_count_sum adds slots[0, nblocks) into *count (overwriting it).
constexpr int kCountSlots = 8192;
hipError_t count_slots(hipStream_t s, uint32_t** slots);   // this call's slots on the stream's device
hipError_t launch_count_sum(const uint32_t* slots, int nblocks, uint64_t* count, hipStream_t s);

hipError_t launch_act_bwd(Dt dt, int64_t rows, int64_t cols, const void* gate, const void* up,
                          const void* dy, const float* weights, float limit, bool clamp,
                          void* dgate, void* dup, float* wgrad, hipStream_t s);

// The same with dgate and dup as E4M3 codes and UE8M0 scales per 1x32 block.
hipError_t launch_act_bwd_fp8(Dt dt, int64_t rows, int64_t cols, const void* gate, const void* up,
                              const void* dy, const float* weights, float limit, bool clamp, uint8_t* q_dgate,
                              uint8_t* s_dgate, uint8_t* q_dup, uint8_t* s_dup, float* wgrad, hipStream_t s);

hipError_t launch_act_fwd(Act act, Dt out, int64_t rows, int64_t cols, const float* gate, const float* up,
                          float limit, bool clamp, void* h, uint64_t* count, hipStream_t s);

hipError_t launch_act_quant(Act act, int64_t rows, int64_t cols, const float* gate, const float* up,
                            float limit, bool clamp, uint8_t* q, uint8_t* scale,
                            uint64_t* count, float* hout, hipStream_t s);

// The quantiser's twin: its grid, loads and stores without arithmetic (the
// unclamped launch, no count, no h_out).
hipError_t launch_act_quant_twin(int64_t rows, int64_t cols, const float* gate, const float* up, uint8_t* q,
                                 uint8_t* scale, hipStream_t s);

hipError_t launch_probe_transitions(uint32_t first, uint32_t last, int kind, uint32_t* out, uint32_t capacity,
                                    uint32_t* count, hipStream_t s);

hipError_t launch_probe_mfma(int iters, int blocks, float* sink, hipStream_t s);

hipError_t launch_probe_read2(const void* a, const void* b, size_t bytes, uint32_t* sink,
                              hipStream_t s);

}  // namespace swg
