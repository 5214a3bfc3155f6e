// Layout transposes for the backward contractions.
//
// The matrix cores want both operands of C = A B^T with the reduction index
// contiguous.  dX = dg Wg + du Wu reduces over N and dW = dg^T x reduces over
// M, so the backward first writes x^T, [Wg; Wu]^T and [dg | du]^T (each zero
// padded along the new contiguous axis to a multiple of 8 elements) and then
// runs the same reduction-contiguous GEMM kernel.
#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kT = 64;  // tile edge

// out[c * ld_out + col_off + r] = (r < rows) ? in[r * ld_in + c] : 0,
// for c < cols and r < rows_pad.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int64_t ld_in,
                                                        int rows, int cols, T* __restrict__ out,
                                                        int64_t ld_out, int col_off, int rows_pad) {
  __shared__ T tile[kT][kT + 1];
  const int r0 = blockIdx.y * kT;
  const int c0 = blockIdx.x * kT;
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;  // 0..3
#pragma unroll 4
  for (int i = ty; i < kT; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    T v = T(0.0f);
    if (r < rows && c < cols) v = in[(int64_t)r * ld_in + c];
    tile[i][tx] = v;
  }
  __syncthreads();
#pragma unroll 4
  for (int i = ty; i < kT; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_pad) out[(int64_t)c * ld_out + col_off + r] = tile[tx][i];
  }
}

}  // namespace

hipError_t launch_transpose(Dt dt, const void* in, int64_t ld_in, int rows, int cols, void* out,
                            int64_t ld_out, int col_off, int rows_pad, hipStream_t s) {
  if (cols == 0 || rows_pad == 0) return hipSuccess;
  dim3 grid((cols + kT - 1) / kT, (rows_pad + kT - 1) / kT);
  if (dt == Dt::kBF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(in),
                       ld_in, rows, cols, static_cast<bf16*>(out), ld_out, col_off, rows_pad);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(in),
                       ld_in, rows, cols, static_cast<float*>(out), ld_out, col_off, rows_pad);
  return hipGetLastError();
}

}  // namespace swg
