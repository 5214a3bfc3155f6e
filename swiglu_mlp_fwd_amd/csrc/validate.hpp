// Host-side argument validation and workspace layout for the C ABI.
// Pure C++ (no HIP), so it can be compiled and tested without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "swiglu.h"

namespace swg {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

inline int elem_size(int dtype) { return dtype == SWIGLU_BF16 ? 2 : 4; }
// Elements per 16-byte row chunk: rows must be whole chunks for 128-bit loads.
inline int chunk_elems(int dtype) { return dtype == SWIGLU_BF16 ? 8 : 4; }

inline int check_dtype(int dtype) {
  return (dtype == SWIGLU_F32 || dtype == SWIGLU_BF16) ? SWIGLU_OK : SWIGLU_ERR_DTYPE;
}

inline int check_dims(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return SWIGLU_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SWIGLU_ERR_SHAPE;
  return SWIGLU_OK;
}

// GEMM tiles are 128 x 128; the launch grid must stay below 2^31 workgroups.
inline bool tiles_fit(int64_t m, int64_t n) {
  return ((m + 127) / 128) * ((n + 127) / 128) < (int64_t(1) << 31);
}

inline int check_ptr(const void* p) {
  if (p == nullptr) return SWIGLU_ERR_NULL;
  if (!aligned(p, 16)) return SWIGLU_ERR_ALIGN;
  return SWIGLU_OK;
}

// Backward workspace, regions starting on 256-byte boundaries.
//   D   [M, 2 Np]     dg in columns [0, Np), du in [Np, 2 Np), zero padded
//   DT  [2 Np, Mp]    transpose of D, zero padded along M
//   XT  [K, Mp]       transpose of x, zero padded along M
//   WT  [K, 2 Np]     [Wg; Wu] transposed, zero padded along N
// with Mp = round_up(M, 8); Np = round_up(N, 64) for bf16 (its tiles and
// 64-element reduction steps then never straddle the dg / du halves) and
// round_up(N, 8) for fp32.
struct BwdLayout {
  int64_t Mp, Np;
  size_t off_d, off_dt, off_xt, off_wt, total;
};

inline BwdLayout bwd_layout(int dtype, int64_t M, int64_t N, int64_t K) {
  BwdLayout L;
  const size_t es = (size_t)elem_size(dtype);
  const bool bf16 = dtype == SWIGLU_BF16;
  L.Mp = round_up(M, 8);
  L.Np = round_up(N, bf16 ? 64 : 8);
  auto a256 = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t off = 0;
  L.off_d = off;  off += a256((size_t)M * 2 * L.Np * es);
  L.off_dt = off; off += a256((size_t)2 * L.Np * L.Mp * es);
  L.off_xt = off; off += a256((size_t)K * L.Mp * es);
  L.off_wt = off; off += a256((size_t)K * 2 * L.Np * es);
  L.total = off;
  return L;
}

// The GEMM kernels address an operand tile through a buffer descriptor whose
// size and byte offsets are 32-bit: a tile spans at most 512 bytes per unit
// of row stride (256 bf16 rows or 128 fp32 rows), and the out-of-range
// offset 2^31 must lie past it, so every row stride a GEMM reads with (K for
// the forward products, 2 Np and Mp for the backward ones) is capped for
// both element types.  The cap is also the largest padded row count the
// transposes' grids cover (65,535 tiles of 64 rows).
constexpr int64_t kMaxLd = (int64_t(1) << 22) - 64;

inline int validate_fwd(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                        const void* wu, const void* h) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, N, K))) return st;
  if (K % chunk_elems(dtype) != 0) return SWIGLU_ERR_SHAPE;
  if (!tiles_fit(M, N)) return SWIGLU_ERR_UNSUPPORTED;
  if (K > kMaxLd) return SWIGLU_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return SWIGLU_OK;
  if ((st = check_ptr(h))) return st;
  if (K > 0) {
    if ((st = check_ptr(x))) return st;
    if ((st = check_ptr(wg))) return st;
    if ((st = check_ptr(wu))) return st;
  }
  return SWIGLU_OK;
}

// The sizes the backward accepts, pointers aside: valid dims, grids that fit,
// and every row stride its GEMMs read with (K, 2 Np, Mp) within kMaxLd.  Within
// these limits every region of bwd_layout is below 2^46 bytes, so its sizes
// cannot wrap.
inline int bwd_shape_status(int dtype, int64_t M, int64_t N, int64_t K) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, N, K))) return st;
  if (K % chunk_elems(dtype) != 0) return SWIGLU_ERR_SHAPE;
  const int64_t Mp = round_up(M, 8), Np = round_up(N, dtype == SWIGLU_BF16 ? 64 : 8);
  if (K > kMaxLd || 2 * Np > kMaxLd || Mp > kMaxLd) return SWIGLU_ERR_UNSUPPORTED;
  if (!tiles_fit(M, Np) || !tiles_fit(M, K) || !tiles_fit(2 * Np, K)) return SWIGLU_ERR_UNSUPPORTED;
  return SWIGLU_OK;
}

// Workspace bytes of a backward the library accepts; 0 for any other sizes.
inline size_t bwd_workspace_total(int dtype, int64_t M, int64_t N, int64_t K) {
  return bwd_shape_status(dtype, M, N, K) == SWIGLU_OK ? bwd_layout(dtype, M, N, K).total : 0;
}

inline int validate_bwd(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                        const void* wu, const void* dh, const void* dx, const void* dwg,
                        const void* dwu, const void* ws, size_t ws_bytes) {
  int st = bwd_shape_status(dtype, M, N, K);
  if (st) return st;
  const BwdLayout L = bwd_layout(dtype, M, N, K);
  if (K == 0) return SWIGLU_OK;                       // every output is empty
  if (M > 0 && (st = check_ptr(dx))) return st;
  if (N > 0 && (st = check_ptr(dwg))) return st;
  if (N > 0 && (st = check_ptr(dwu))) return st;
  if (M == 0 || N == 0) return SWIGLU_OK;             // outputs are zero-filled
  if ((st = check_ptr(x))) return st;
  if ((st = check_ptr(wg))) return st;
  if ((st = check_ptr(wu))) return st;
  if ((st = check_ptr(dh))) return st;
  if (ws == nullptr) return SWIGLU_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SWIGLU_ERR_ALIGN;
  if (ws_bytes < L.total) return SWIGLU_ERR_WORKSPACE;
  return SWIGLU_OK;
}

inline int validate_gemv(int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                         const void* wu, const void* h) {
  if (M < 0 || M > 8) return SWIGLU_ERR_SHAPE;
  int st = check_dims(M, N, K);
  if (st) return st;
  if (K % 8 != 0) return SWIGLU_ERR_SHAPE;
  if (M == 0 || N == 0) return SWIGLU_OK;
  if ((st = check_ptr(h))) return st;
  if (K > 0) {
    if ((st = check_ptr(x))) return st;
    if ((st = check_ptr(wg))) return st;
    if ((st = check_ptr(wu))) return st;
  }
  return SWIGLU_OK;
}

inline int validate_fwd_fp8(int64_t M, int64_t N, int64_t K, const void* x, const void* wg,
                            const void* wu, const void* q, const void* scale, const void* h_out) {
  int st;
  if ((st = check_dims(M, N, K))) return st;
  if (K % chunk_elems(SWIGLU_BF16) != 0 || N % 32 != 0) return SWIGLU_ERR_SHAPE;
  if (!tiles_fit(M, N)) return SWIGLU_ERR_UNSUPPORTED;
  if (K > kMaxLd) return SWIGLU_ERR_UNSUPPORTED;
  if (h_out != nullptr && !aligned(h_out, 16)) return SWIGLU_ERR_ALIGN;
  if (M == 0 || N == 0) return SWIGLU_OK;
  if ((st = check_ptr(q))) return st;
  if (scale == nullptr) return SWIGLU_ERR_NULL;
  if (K > 0) {
    if ((st = check_ptr(x))) return st;
    if ((st = check_ptr(wg))) return st;
    if ((st = check_ptr(wu))) return st;
  }
  return SWIGLU_OK;
}

inline int validate_act_fwd(int out_dtype, int64_t rows, int64_t cols, const float* gate, const float* up,
                            float L, const void* h, const void* count) {
  int st = check_dtype(out_dtype);
  if (st) return st;
  if (rows < 0 || cols < 0) return SWIGLU_ERR_SHAPE;
  if (cols % 8 != 0) return SWIGLU_ERR_SHAPE;         // the interface's row granularity (the kernel needs 4)
  if (rows > 0 && cols > (int64_t(1) << 40) / rows) return SWIGLU_ERR_SHAPE;
  if (!(L > 0.0f)) return SWIGLU_ERR_ARG;             // rejects NaN, zero and negatives
  if (count != nullptr && !aligned(count, 8)) return SWIGLU_ERR_ALIGN;
  if (rows == 0 || cols == 0) return SWIGLU_OK;
  if ((st = check_ptr(gate))) return st;
  if ((st = check_ptr(up))) return st;
  if ((st = check_ptr(h))) return st;
  return SWIGLU_OK;
}

inline int validate_act_quant(int64_t rows, int64_t cols, const float* gate, const float* up,
                              float L, const void* q, const void* scale, const void* count,
                              const void* hout) {
  if (rows < 0 || cols < 0) return SWIGLU_ERR_SHAPE;
  if (cols % 32 != 0) return SWIGLU_ERR_SHAPE;
  if (rows > 0 && cols > (int64_t(1) << 40) / rows) return SWIGLU_ERR_SHAPE;
  if (!(L > 0.0f)) return SWIGLU_ERR_ARG;             // rejects NaN, zero and negatives
  if (count != nullptr && !aligned(count, 8)) return SWIGLU_ERR_ALIGN;
  if (rows == 0 || cols == 0) return SWIGLU_OK;
  int st;
  if ((st = check_ptr(gate))) return st;
  if ((st = check_ptr(up))) return st;
  if ((st = check_ptr(q))) return st;
  if ((st = check_ptr(scale))) return st;
  if (hout != nullptr && !aligned(hout, 16)) return SWIGLU_ERR_ALIGN;
  return SWIGLU_OK;
}

inline int validate_act_bwd(int dtype, int64_t rows, int64_t cols, const void* gate, const void* up,
                            const void* dy, const float* weights, float L, const void* dgate,
                            const void* dup, const float* wgrad) {
  int st0 = check_dtype(dtype);
  if (st0) return st0;
  if (rows < 0 || cols < 0) return SWIGLU_ERR_SHAPE;
  if (cols % chunk_elems(dtype) != 0) return SWIGLU_ERR_SHAPE;   // 16-byte rows
  if (rows > 0 && cols > (int64_t(1) << 40) / rows) return SWIGLU_ERR_SHAPE;
  if (!(L > 0.0f)) return SWIGLU_ERR_ARG;             // rejects NaN, zero and negatives
  if (weights != nullptr && !aligned(weights, 4)) return SWIGLU_ERR_ALIGN;
  if (wgrad != nullptr && !aligned(wgrad, 4)) return SWIGLU_ERR_ALIGN;
  if (rows == 0) return SWIGLU_OK;
  if (cols > 0) {
    int st;
    if ((st = check_ptr(gate))) return st;
    if ((st = check_ptr(up))) return st;
    if ((st = check_ptr(dy))) return st;
    if ((st = check_ptr(dgate))) return st;
    if ((st = check_ptr(dup))) return st;
  }
  return SWIGLU_OK;
}

inline int validate_act_bwd_fp8(int dtype, int64_t rows, int64_t cols, const void* gate, const void* up,
                                const void* dy, const float* weights, float L, const void* qg, const void* sg,
                                const void* qu, const void* su, const float* wgrad) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (rows < 0 || cols < 0) return SWIGLU_ERR_SHAPE;
  if (cols % 32 != 0) return SWIGLU_ERR_SHAPE;        // whole 1x32 blocks per row
  if (rows > 0 && cols > (int64_t(1) << 40) / rows) return SWIGLU_ERR_SHAPE;
  if (!(L > 0.0f)) return SWIGLU_ERR_ARG;             // rejects NaN, zero and negatives
  if (weights != nullptr && !aligned(weights, 4)) return SWIGLU_ERR_ALIGN;
  if (wgrad != nullptr && !aligned(wgrad, 4)) return SWIGLU_ERR_ALIGN;
  if (rows == 0 || cols == 0) return SWIGLU_OK;
  if ((st = check_ptr(gate))) return st;
  if ((st = check_ptr(up))) return st;
  if ((st = check_ptr(dy))) return st;
  if ((st = check_ptr(qg))) return st;
  if ((st = check_ptr(qu))) return st;
  if (sg == nullptr || su == nullptr) return SWIGLU_ERR_NULL;
  return SWIGLU_OK;
}

}  // namespace swg
