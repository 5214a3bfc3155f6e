// Layout transposes for the backward contractions.
//
// The matrix cores want both operands of C = A B^T with the reduction index
// contiguous.  dX = dg Wg + du Wu reduces over N and dW = dg^T x reduces over
// M.  The fp32 backward writes x^T, [Wg; Wu]^T and [dg | du]^T (each zero
// padded along the new contiguous axis to a multiple of 8 elements) and then
// runs the reduction-contiguous GEMM kernel; the bf16 backward transposes x
// only (the rest is read in place or written transposed by the recompute).
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

// bf16 transpose with 16-byte accesses on both sides.  A 64 x 64 tile is
// loaded as 16-byte row chunks into LDS (160-byte pitch: the 8 rows of a
// chunk group fall in 8 distinct 32-byte bank windows), then read back a
// column at a time with ds_read_b64_tr_b16: in a 16-lane group, lane i gets
// column i of the 4 x 16 block the group addresses, so two reads (rows
// +0..3 and +4..7) give a lane 8 consecutive rows of one column, i.e. one
// 16-byte chunk of an output row.  The two groups served together read
// opposite row halves first, so their windows never overlap.  Needs cols,
// ld_in, ld_out, col_off and rows_pad to be multiples of 8.
constexpr int kTPitch = 160;

typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ in, int64_t ld_in,
                                                             int rows, int cols, bf16* __restrict__ out,
                                                             int64_t ld_out, int col_off, int rows_pad) {
  __shared__ __attribute__((aligned(16))) char tile[kT * kTPitch];
  const int r0 = blockIdx.y * kT;
  const int c0 = blockIdx.x * kT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = tid + 256 * j;
    const int i = q >> 3, cc = q & 7;
    const int r = r0 + i, c = c0 + 8 * cc;
    u32x4 v = {0, 0, 0, 0};
    if (r < rows && c < cols) v = *reinterpret_cast<const u32x4*>(in + (int64_t)r * ld_in + c);
    *reinterpret_cast<u32x4*>(tile + i * kTPitch + cc * 16) = v;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, s16 = lane & 15, hsel = g & 1;
#pragma unroll
  for (int t = wave; t < 8; t += 4) {
    const int cb = t >> 1;                       // 16-column block
    const int rq = (t & 1) * 4 + g;              // 8-row chunk
    const int col = cb * 16 + 4 * (s16 & 3);
    const int ra = rq * 8 + 4 * hsel + (s16 >> 2), rb = rq * 8 + 4 * (1 - hsel) + (s16 >> 2);
    const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4_t*)((lds_char_t*)tile + ra * kTPitch + col * 2));
    const short4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4_t*)((lds_char_t*)tile + rb * kTPitch + col * 2));
    const u32x2 a = __builtin_bit_cast(u32x2, hsel ? v2 : v1);
    const u32x2 b = __builtin_bit_cast(u32x2, hsel ? v1 : v2);
    const int c = c0 + cb * 16 + s16, r = r0 + rq * 8;
    if (c < cols && r < rows_pad)
      *reinterpret_cast<u32x4*>(out + (int64_t)c * ld_out + col_off + r) = u32x4{a[0], a[1], b[0], b[1]};
  }
}

}  // namespace

hipError_t launch_transpose(Dt dt, const void* in, int64_t ld_in, int rows, int cols, void* out,
                            int64_t ld_out, int col_off, int rows_pad, hipStream_t s) {
  if (cols == 0 || rows_pad == 0) return hipSuccess;
  dim3 grid((cols + kT - 1) / kT, (rows_pad + kT - 1) / kT);
  if (dt == Dt::kBF16 && cols % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0 && col_off % 8 == 0 &&
      rows_pad % 8 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(out) % 16 == 0) {
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, static_cast<const bf16*>(in),
                       ld_in, rows, cols, static_cast<bf16*>(out), ld_out, col_off, rows_pad);
    return hipGetLastError();
  }
  if (dt == Dt::kBF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(in),
                       ld_in, rows, cols, static_cast<bf16*>(out), ld_out, col_off, rows_pad);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(in),
                       ld_in, rows, cols, static_cast<float*>(out), ld_out, col_off, rows_pad);
  return hipGetLastError();
}

}  // namespace swg
