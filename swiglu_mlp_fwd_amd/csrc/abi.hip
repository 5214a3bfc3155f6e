// The C ABI of libswiglu: validation on the host, then kernel launches on the
// caller's stream.  No allocation, no synchronisation.
#include <math.h>

#include <mutex>

#include "gemm.hpp"
#include "swiglu.h"
#include "validate.hpp"

// Set by the build (a hash of the sources and flags); see swiglu_source_hash.
#ifndef SWIGLU_SOURCE_HASH
#define SWIGLU_SOURCE_HASH "unknown"
#endif

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SWIGLU_OK;
  g_last_hip_error = (int)e;
  return SWIGLU_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

swg::Dt as_dt(int dtype) { return dtype == SWIGLU_BF16 ? swg::Dt::kBF16 : swg::Dt::kF32; }

// Projection multipliers must be finite (NaN or infinity: SWIGLU_ERR_ARG).
bool finite_mult(float m) { return isfinite(m); }

// Zero-fill of a dense output through the transpose kernel's padding path
// (a kernel, not a memset node, so callers may capture it in a graph).
hipError_t fill_zero(int dtype, void* p, int64_t rows, int64_t cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  // Transposing a [0, rows] input with rows_pad = cols writes zeros into
  // out[c, r] for c < rows, r < cols, i.e. the whole [rows, cols] array.
  return swg::launch_transpose(as_dt(dtype), nullptr, 0, 0, (int)rows, p, cols, 0, (int)cols, s);
}

}  // namespace

// The backward's scratch for swiglu_bwd_noalloc: a file-scope device array,
// so the entry point never allocates.  In host code `scratch` is only a
// handle for the runtime: its device address on the current GPU comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[SWIGLU_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device `stream` belongs to (each GPU
// holds its own copy at its own address), looked up on the first call on
// that device.
hipError_t scratch_address(hipStream_t stream, void** out) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t result[kMaxDevices];
  int dev = 0;
  const hipError_t e = swg::stream_device(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    result[dev] = swg::symbol_address_on(dev, HIP_SYMBOL(scratch), &p);
    addr[dev] = p;
  });
  *out = addr[dev];
  return result[dev];
}

}  // namespace

namespace swg {
// probe.hip: threads in {256, 512}, chunks in {1, 2, 4, 8}, 1 <= max_blocks <= 65535.
hipError_t launch_probe_read2_cfg(const void* a, const void* b, size_t bytes, int threads, int chunks,
                                  int max_blocks, uint32_t* sink, hipStream_t s);
}  // namespace swg

extern "C" {

int swiglu_fwd_mult(int act, int dtype, int64_t M, int64_t N, int64_t K, const void* x,
                    const void* wg, const void* wu, float gate_mult, float up_mult, void* h,
                    void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  if (!finite_mult(gate_mult) || !finite_mult(up_mult)) return SWIGLU_ERR_ARG;
  int st = swg::validate_fwd(dtype, M, N, K, x, wg, wu, h);
  if (st != SWIGLU_OK || M == 0 || N == 0) return st;
  swg::GemmArgs a{};
  a.a = x; a.b0 = wg; a.b1 = wu;
  a.lda = K; a.ldb = K;
  a.arows = (int)M; a.brows = (int)N;
  a.m = (int)M; a.n = (int)N; a.r = (int)K;
  a.out0 = h; a.ldo = N; a.ncols = (int)N;
  a.gmul = gate_mult; a.umul = up_mult;
  return hip_status(swg::launch_fwd_dual(as_dt(dtype), static_cast<swg::Act>(act), a, as_stream(stream)));
}

int swiglu_fwd_act(int act, int dtype, int64_t M, int64_t N, int64_t K, const void* x,
                   const void* wg, const void* wu, void* h, void* stream) {
  return swiglu_fwd_mult(act, dtype, M, N, K, x, wg, wu, 1.0f, 1.0f, h, stream);
}

int swiglu_fwd(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
               const void* wu, void* h, void* stream) {
  return swiglu_fwd_act(SWIGLU_ACT_SILU, dtype, M, N, K, x, wg, wu, h, stream);
}

int swiglu_fwd_fp8(int act, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                   const void* wu, uint8_t* q, uint8_t* scale, float* h_out, void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  int st = swg::validate_fwd_fp8(M, N, K, x, wg, wu, q, scale, h_out);
  if (st != SWIGLU_OK || M == 0 || N == 0) return st;
  swg::GemmArgs a{};
  a.a = x; a.b0 = wg; a.b1 = wu;
  a.lda = K; a.ldb = K;
  a.arows = (int)M; a.brows = (int)N;
  a.m = (int)M; a.n = (int)N; a.r = (int)K;
  a.out0 = q; a.ldo = N; a.ncols = (int)N;
  a.q_scale = scale; a.q_h = h_out;
  return hip_status(swg::launch_fwd_dual_fp8(static_cast<swg::Act>(act), a, as_stream(stream)));
}

size_t swiglu_bwd_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K) {
  return swg::bwd_workspace_total(dtype, M, N, K);
}

int swiglu_bwd_act_mult(int act, int dtype, int64_t M, int64_t N, int64_t K, const void* x,
                        const void* wg, const void* wu, const void* dh, float gate_mult, float up_mult,
                        void* dx, void* dwg, void* dwu, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  if (!finite_mult(gate_mult) || !finite_mult(up_mult)) return SWIGLU_ERR_ARG;
  int st = swg::validate_bwd(dtype, M, N, K, x, wg, wu, dh, dx, dwg, dwu, workspace,
                             workspace_bytes);
  if (st != SWIGLU_OK || K == 0) return st;
  hipStream_t s = as_stream(stream);
  const swg::Dt dt = as_dt(dtype);
  if (M == 0 || N == 0) {
    // Empty sums: dx = 0 when N == 0, dWg = dWu = 0 when M == 0.
    hipError_t e = hipSuccess;
    if (N == 0) e = fill_zero(dtype, dx, M, K, s);
    if (e == hipSuccess && M == 0) e = fill_zero(dtype, dwg, N, K, s);
    if (e == hipSuccess && M == 0) e = fill_zero(dtype, dwu, N, K, s);
    return hip_status(e);
  }
  const swg::BwdLayout L = swg::bwd_layout(dtype, M, N, K);
  char* ws = static_cast<char*>(workspace);
  void* D = ws + L.off_d;
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K, Mp = (int)L.Mp, Np = (int)L.Np;
  hipError_t e;

  // 1. Recompute g, u and form D = [dg | du] (columns N..Np-1 of each half are zero).
  swg::GemmArgs b1{};
  b1.a = x; b1.b0 = wg; b1.b1 = wu; b1.lda = K; b1.ldb = K;
  b1.arows = Mi; b1.brows = Ni; b1.m = Mi; b1.n = Np; b1.r = Ki;
  b1.out0 = D; b1.ldo = 2 * (int64_t)Np; b1.ncols = Ni;
  b1.dh = dh; b1.lddh = N; b1.du_off = Np;
  b1.gmul = gate_mult; b1.umul = up_mult;
  void* DT = ws + L.off_dt;
  void* XT = ws + L.off_xt;
  if (dt == swg::Dt::kBF16) {
    b1.out1 = DT;            // the epilogue also writes D^T [2 Np, Mp]
    b1.ldt = Mp;
  }
  if ((e = swg::launch_bwd_dswiglu(dt, static_cast<swg::Act>(act), b1, s)) != hipSuccess) return hip_status(e);

  if (dt == swg::Dt::kBF16) {
    // 2. dX [M, K] = D [M, 2 Np] . ([Wg; Wu]^T [K, 2 Np])^T, reducing over
    //    the stacked N (the transposes are zero padded from N to Np).
    void* WTb = ws + L.off_wt;
    if ((e = swg::launch_transpose(dt, wg, K, Ni, Ki, WTb, 2 * (int64_t)Np, 0, Np, s)) != hipSuccess) return hip_status(e);
    if ((e = swg::launch_transpose(dt, wu, K, Ni, Ki, WTb, 2 * (int64_t)Np, Np, Np, s)) != hipSuccess) return hip_status(e);
    swg::GemmArgs b2{};
    b2.a = D; b2.b0 = WTb; b2.lda = 2 * (int64_t)Np; b2.ldb = 2 * (int64_t)Np;
    b2.arows = Mi; b2.brows = Ki; b2.m = Mi; b2.n = Ki; b2.r = 2 * Np;
    b2.out0 = dx; b2.ldo = K; b2.split = Mi; b2.lim0 = Mi; b2.lim1 = 0; b2.ncols = Ki;
    if ((e = swg::launch_gemm_store(dt, b2, s)) != hipSuccess) return hip_status(e);
    // 3. [dWg; dWu] [2 Np, K] = D^T [2 Np, Mp] . (x^T [K, Mp])^T, reducing
    //    over M: D^T came from the recompute's epilogue, x^T from a
    //    transpose (zero padded to Mp).
    if ((e = swg::launch_transpose(dt, x, K, Mi, Ki, XT, Mp, 0, Mp, s)) != hipSuccess) return hip_status(e);
    swg::GemmArgs b3{};
    b3.a = DT; b3.b0 = XT; b3.lda = Mp; b3.ldb = Mp;
    b3.arows = 2 * Np; b3.brows = Ki; b3.m = 2 * Np; b3.n = Ki; b3.r = Mp;
    b3.out0 = dwg; b3.out1 = dwu; b3.ldo = K; b3.split = Np; b3.lim0 = Ni; b3.lim1 = Ni;
    b3.ncols = Ki;
    return hip_status(swg::launch_gemm_store(dt, b3, s));
  }
  void* WT = ws + L.off_wt;

  // 2. Transposes: x -> XT [K, Mp]; Wg, Wu -> WT [K, 2 Np]; D -> DT [2 Np, Mp].
  if ((e = swg::launch_transpose(dt, x, K, Mi, Ki, XT, Mp, 0, Mp, s)) != hipSuccess) return hip_status(e);
  if ((e = swg::launch_transpose(dt, wg, K, Ni, Ki, WT, 2 * (int64_t)Np, 0, Np, s)) != hipSuccess) return hip_status(e);
  if ((e = swg::launch_transpose(dt, wu, K, Ni, Ki, WT, 2 * (int64_t)Np, Np, Np, s)) != hipSuccess) return hip_status(e);
  if ((e = swg::launch_transpose(dt, D, 2 * (int64_t)Np, Mi, 2 * Np, DT, Mp, 0, Mp, s)) != hipSuccess) return hip_status(e);

  // 3. dX [M, K] = D [M, 2 Np] . WT [K, 2 Np]^T  (reduction over the stacked N).
  swg::GemmArgs b2{};
  b2.a = D; b2.b0 = WT; b2.lda = 2 * (int64_t)Np; b2.ldb = 2 * (int64_t)Np;
  b2.arows = Mi; b2.brows = Ki; b2.m = Mi; b2.n = Ki; b2.r = 2 * Np;
  b2.out0 = dx; b2.ldo = K; b2.split = Mi; b2.lim0 = Mi; b2.lim1 = 0; b2.ncols = Ki;
  if ((e = swg::launch_gemm_store(dt, b2, s)) != hipSuccess) return hip_status(e);

  // 4. [dWg; dWu] [2 Np, K] = DT [2 Np, Mp] . XT [K, Mp]^T  (reduction over M).
  swg::GemmArgs b3{};
  b3.a = DT; b3.b0 = XT; b3.lda = Mp; b3.ldb = Mp;
  b3.arows = 2 * Np; b3.brows = Ki; b3.m = 2 * Np; b3.n = Ki; b3.r = Mp;
  b3.out0 = dwg; b3.out1 = dwu; b3.ldo = K; b3.split = Np; b3.lim0 = Ni; b3.lim1 = Ni;
  b3.ncols = Ki;
  return hip_status(swg::launch_gemm_store(dt, b3, s));
}

int swiglu_bwd_mult(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                    const void* wu, const void* dh, float gate_mult, float up_mult, void* dx, void* dwg,
                    void* dwu, void* workspace, size_t workspace_bytes, void* stream) {
  return swiglu_bwd_act_mult(SWIGLU_ACT_SILU, dtype, M, N, K, x, wg, wu, dh, gate_mult, up_mult, dx, dwg,
                             dwu, workspace, workspace_bytes, stream);
}

int swiglu_bwd(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
               const void* wu, const void* dh, void* dx, void* dwg, void* dwu, void* workspace,
               size_t workspace_bytes, void* stream) {
  return swiglu_bwd_act_mult(SWIGLU_ACT_SILU, dtype, M, N, K, x, wg, wu, dh, 1.0f, 1.0f, dx, dwg, dwu,
                             workspace, workspace_bytes, stream);
}

int swiglu_bwd_noalloc(int act, int dtype, int64_t M, int64_t N, int64_t K, const void* x,
                       const void* wg, const void* wu, const void* dh, float gate_mult, float up_mult,
                       void* dx, void* dwg, void* dwu, void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  if (!finite_mult(gate_mult) || !finite_mult(up_mult)) return SWIGLU_ERR_ARG;
  // Everything but the workspace is checked first, so the errors are those
  // of swiglu_bwd_act_mult; then the scratch bound.
  int st = swg::validate_bwd(dtype, M, N, K, x, wg, wu, dh, dx, dwg, dwu, nullptr, 0);
  if (st != SWIGLU_OK && st != SWIGLU_ERR_WORKSPACE) return st;
  if (st == SWIGLU_OK)          // a call that needs no workspace (K, M or N is 0)
    return swiglu_bwd_act_mult(act, dtype, M, N, K, x, wg, wu, dh, gate_mult, up_mult, dx, dwg, dwu,
                               nullptr, 0, stream);
  if (swg::bwd_workspace_total(dtype, M, N, K) > SWIGLU_NOALLOC_SCRATCH_BYTES) return SWIGLU_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_address(as_stream(stream), &ws);
  if (e != hipSuccess) return hip_status(e);
  return swiglu_bwd_act_mult(act, dtype, M, N, K, x, wg, wu, dh, gate_mult, up_mult, dx, dwg, dwu, ws,
                             SWIGLU_NOALLOC_SCRATCH_BYTES, stream);
}

int swiglu_gemv_fwd_mult(int act, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                         const void* wu, float gate_mult, float up_mult, void* h, void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  if (!finite_mult(gate_mult) || !finite_mult(up_mult)) return SWIGLU_ERR_ARG;
  int st = swg::validate_gemv(M, N, K, x, wg, wu, h);
  if (st != SWIGLU_OK || M == 0 || N == 0) return st;
  return hip_status(swg::launch_gemv(static_cast<swg::Act>(act), (int)M, (int)N, (int)K, x, wg, wu,
                                     h, gate_mult, up_mult, as_stream(stream)));
}

int swiglu_gemv_fwd_act(int act, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                        const void* wu, void* h, void* stream) {
  return swiglu_gemv_fwd_mult(act, M, N, K, x, wg, wu, 1.0f, 1.0f, h, stream);
}

int swiglu_gemv_fwd(int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                    const void* wu, void* h, void* stream) {
  return swiglu_gemv_fwd_act(SWIGLU_ACT_SILU, M, N, K, x, wg, wu, h, stream);
}

int swiglu_act_fwd(int act, int out_dtype, int64_t rows, int64_t cols, const float* gate, const float* up,
                   float clamp_limit, void* h, uint64_t* clamp_count, void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  int st = swg::validate_act_fwd(out_dtype, rows, cols, gate, up, clamp_limit, h, clamp_count);
  if (st != SWIGLU_OK) return st;
  const bool clamp = !isinf(clamp_limit);
  return hip_status(swg::launch_act_fwd(static_cast<swg::Act>(act), as_dt(out_dtype), rows, cols, gate, up,
                                        clamp_limit, clamp, h, clamp_count, as_stream(stream)));
}

int swiglu_act_quant_act(int act, int64_t rows, int64_t cols, const float* gate, const float* up,
                         float clamp_limit, uint8_t* q, uint8_t* scale, uint64_t* clamp_count,
                         float* h_out, void* stream) {
  if (act != SWIGLU_ACT_SILU && act != SWIGLU_ACT_GELU_TANH) return SWIGLU_ERR_ARG;
  int st = swg::validate_act_quant(rows, cols, gate, up, clamp_limit, q, scale, clamp_count, h_out);
  if (st != SWIGLU_OK) return st;
  const bool clamp = !isinf(clamp_limit);
  return hip_status(swg::launch_act_quant(static_cast<swg::Act>(act), rows, cols, gate, up, clamp_limit,
                                          clamp, q, scale, clamp_count, h_out, as_stream(stream)));
}

int swiglu_act_quant(int64_t rows, int64_t cols, const float* gate, const float* up,
                     float clamp_limit, uint8_t* q, uint8_t* scale, uint64_t* clamp_count,
                     float* h_out, void* stream) {
  return swiglu_act_quant_act(SWIGLU_ACT_SILU, rows, cols, gate, up, clamp_limit, q, scale,
                              clamp_count, h_out, stream);
}

int swiglu_act_bwd_dt(int dtype, int64_t rows, int64_t cols, const void* gate, const void* up,
                      const void* dy, const float* weights, float clamp_limit, void* dgate, void* dup,
                      float* weight_grad, void* stream) {
  int st = swg::validate_act_bwd(dtype, rows, cols, gate, up, dy, weights, clamp_limit, dgate, dup,
                                 weight_grad);
  if (st != SWIGLU_OK || rows == 0) return st;
  const bool clamp = !isinf(clamp_limit);
  return hip_status(swg::launch_act_bwd(as_dt(dtype), rows, cols, gate, up, dy, weights, clamp_limit,
                                        clamp, dgate, dup, weight_grad, as_stream(stream)));
}

int swiglu_act_bwd_fp8(int dtype, int64_t rows, int64_t cols, const void* gate, const void* up, const void* dy,
                       const float* weights, float clamp_limit, uint8_t* q_dgate, uint8_t* scale_dgate,
                       uint8_t* q_dup, uint8_t* scale_dup, float* weight_grad, void* stream) {
  int st = swg::validate_act_bwd_fp8(dtype, rows, cols, gate, up, dy, weights, clamp_limit, q_dgate, scale_dgate,
                                     q_dup, scale_dup, weight_grad);
  if (st != SWIGLU_OK || rows == 0) return st;
  const bool clamp = !isinf(clamp_limit);
  return hip_status(swg::launch_act_bwd_fp8(as_dt(dtype), rows, cols, gate, up, dy, weights, clamp_limit, clamp,
                                            q_dgate, scale_dgate, q_dup, scale_dup, weight_grad, as_stream(stream)));
}

int swiglu_act_bwd(int64_t rows, int64_t cols, const float* gate, const float* up, const float* dy,
                   const float* weights, float clamp_limit, float* dgate, float* dup,
                   float* weight_grad, void* stream) {
  return swiglu_act_bwd_dt(SWIGLU_F32, rows, cols, gate, up, dy, weights, clamp_limit, dgate, dup,
                           weight_grad, stream);
}

int swiglu_probe_mfma(int iters, int blocks, float* sink, void* stream) {
  if (iters < 0 || blocks < 0) return SWIGLU_ERR_SHAPE;
  if (iters == 0 || blocks == 0) return SWIGLU_OK;
  if (sink == nullptr) return SWIGLU_ERR_NULL;
  return hip_status(swg::launch_probe_mfma(iters, blocks, sink, as_stream(stream)));
}

int swiglu_probe_gemv_read(int64_t M, int64_t N, int64_t K, const void* x, const void* wg, const void* wu,
                           uint32_t* sink, void* stream) {
  // h is checked for 16-byte alignment by the GEMV's validation; the sink
  // only needs 4 (one word per column).
  int st = swg::validate_gemv(M, N, K, x, wg, wu, x);
  if (st != SWIGLU_OK || M == 0 || N == 0) return st;
  if (sink == nullptr) return SWIGLU_ERR_NULL;
  if (!swg::aligned(sink, 4)) return SWIGLU_ERR_ALIGN;
  return hip_status(swg::launch_gemv_read_twin((int)M, (int)N, (int)K, x, wg, wu, sink, as_stream(stream)));
}

int swiglu_probe_act_quant_stream(int64_t rows, int64_t cols, const float* gate, const float* up, uint8_t* q,
                                  uint8_t* scale, void* stream) {
  int st = swg::validate_act_quant(rows, cols, gate, up, INFINITY, q, scale, nullptr, nullptr);
  if (st != SWIGLU_OK || rows == 0 || cols == 0) return st;
  return hip_status(swg::launch_act_quant_twin(rows, cols, gate, up, q, scale, as_stream(stream)));
}

int swiglu_probe_fp8_transitions(int kind, uint32_t first, uint32_t last, uint32_t* out, uint32_t capacity,
                                 uint32_t* count, void* stream) {
  if (kind != 0 && kind != 1) return SWIGLU_ERR_ARG;
  if (last < first) return SWIGLU_ERR_SHAPE;
  if (out == nullptr || count == nullptr) return SWIGLU_ERR_NULL;
  if (!swg::aligned(out, 4) || !swg::aligned(count, 4)) return SWIGLU_ERR_ALIGN;
  return hip_status(swg::launch_probe_transitions(first, last, kind, out, capacity, count, as_stream(stream)));
}

int swiglu_probe_read2(const void* a, const void* b, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16 != 0) return SWIGLU_ERR_SHAPE;
  if (bytes == 0) return SWIGLU_OK;
  if (a == nullptr || b == nullptr || sink == nullptr) return SWIGLU_ERR_NULL;
  if (!swg::aligned(a, 16) || !swg::aligned(b, 16) || !swg::aligned(sink, 4)) return SWIGLU_ERR_ALIGN;
  return hip_status(swg::launch_probe_read2(a, b, bytes, sink, as_stream(stream)));
}

int swiglu_probe_read2_cfg(const void* a, const void* b, size_t bytes, int threads, int chunks, int max_blocks,
                           uint32_t* sink, void* stream) {
  if (threads != 256 && threads != 512) return SWIGLU_ERR_ARG;
  if (chunks != 1 && chunks != 2 && chunks != 4 && chunks != 8) return SWIGLU_ERR_ARG;
  if (max_blocks < 1 || max_blocks > 65535) return SWIGLU_ERR_ARG;
  if (bytes % 16 != 0) return SWIGLU_ERR_SHAPE;
  if (bytes == 0) return SWIGLU_OK;
  if (a == nullptr || b == nullptr || sink == nullptr) return SWIGLU_ERR_NULL;
  if (!swg::aligned(a, 16) || !swg::aligned(b, 16) || !swg::aligned(sink, 4)) return SWIGLU_ERR_ALIGN;
  return hip_status(swg::launch_probe_read2_cfg(a, b, bytes, threads, chunks, max_blocks, sink, as_stream(stream)));
}

const char* swiglu_status_str(int status) {
  switch (status) {
    case SWIGLU_OK: return "ok";
    case SWIGLU_ERR_NULL: return "null pointer";
    case SWIGLU_ERR_SHAPE: return "invalid shape";
    case SWIGLU_ERR_DTYPE: return "invalid dtype";
    case SWIGLU_ERR_ALIGN: return "misaligned pointer";
    case SWIGLU_ERR_WORKSPACE: return "workspace missing or too small";
    case SWIGLU_ERR_ARG: return "invalid argument";
    case SWIGLU_ERR_UNSUPPORTED: return "unsupported size";
    case SWIGLU_ERR_HIP: return "HIP launch error";
    case SWIGLU_ERR_SCRATCH: return "problem needs more scratch than the static buffer holds";
    default: return "unknown status";
  }
}

int swiglu_last_hip_error(void) { return g_last_hip_error; }

int swiglu_version(void) { return 100; }

const char* swiglu_source_hash(void) { return SWIGLU_SOURCE_HASH; }

}  // extern "C"
