// Elementwise SwiGLU backward on materialised gate/up, with an optional clamp
// and optional per-row (routing) weights.
//
// "quant: add SwiGLU forward/backward VMI kernels" (TileKernels-PTO PR 20):
// the performance section's backward table (gate/up given, clamp, routing
// weights with recompute) and the implementation notes (weight_grad is a
// reassociated reduction).  With the forward
//   y[r, c] = w[r] * SiLU(g'[r, c]) * u'[r, c],  g' = clamp(g), u' = clamp(u)
// (w = 1 without weights), the kernel computes from dy
//   dg = w dy u' s (1 + g' (1 - s))   where |g| <= L or g is NaN, else 0
//   du = w dy SiLU(g')                where |u| <= L or u is NaN, else 0
//   weight_grad[r] = sum_c dy SiLU(g') u'
// with s = sigma(g').  sigma and 1 - sigma come from the accurate fp32 form
// (each to a few ulps, the complement without cancellation); the products
// and the row sum are formed in fp64 and each output is rounded once to its
// type.  gate, up, dy, dgate and dup are all fp32 or all bf16 (the table's
// fp32 and bf16 formats); weights and weight_grad are fp32.
//
// Mapping with weight_grad: a workgroup of 4 waves per row (grid-stride over
// rows); lane l of the 256 handles the 16-byte chunks l, l + 256, ... of the
// row (4 fp32 or 8 bf16 elements), kUnroll chunks' loads issued before any
// is used; the row sum is reduced within each wave with xor shuffles, then
// across the 4 waves through LDS in a fixed order.  (4 waves per row
// measured faster than 1 or 2 at 4001 x 3584.)  Without weight_grad there is
// no row sum, and the array is walked flat (grid-stride over all chunks, as
// the forward kernels), which keeps more loads in flight per lane; a chunk's
// row (for its weight) comes from one division.
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kThreads = 256;         // 4 waves
constexpr int kMaxBlocks = 4096;

template <bool kClamp>
__device__ __forceinline__ void bwd_elem(float g, float u, float dy, double w, float L, double& dg,
                                         double& du, double& acc) {
  bool pg = true, pu = true;
  if (kClamp) {
    pg = !(fabsf(g) > L);
    pu = !(fabsf(u) > L);
    g = pg ? g : copysignf(L, g);
    u = pu ? u : copysignf(L, u);
  }
  float s, c;
  sigmoid_pair_f32(g, s, c);
  const double silu = (double)g * (double)s;
  const double dh = w * (double)dy;
  const double t = (double)s * (1.0 + (double)g * (double)c);
  dg = pg ? dh * (double)u * t : 0.0;
  du = pu ? dh * silu : 0.0;
  acc += (double)dy * (silu * (double)u);
}

template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int kN = 4;
  __device__ static void unpack(const u32x4& w, float (&v)[kN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = bits_f32(w[i]);
  }
  __device__ static u32x4 pack(const double (&v)[kN]) {
    return u32x4{f32_bits((float)v[0]), f32_bits((float)v[1]), f32_bits((float)v[2]), f32_bits((float)v[3])};
  }
};
template <> struct Chunk<bf16> {
  static constexpr int kN = 8;
  __device__ static void unpack(const u32x4& w, float (&v)[kN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bits_f32(w[i] << 16);
      v[2 * i + 1] = bits_f32(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static u32x4 pack(const double (&v)[kN]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_bits_rne(v[2 * i]) | (bf16_bits_rne(v[2 * i + 1]) << 16);
    return w;
  }
};

// Where dgate and dup go: tensors of the input type, or (kFp8) E4M3 codes
// [rows, cols] with a UE8M0 scale byte per 1x32 block [rows, cols / 32].
struct BwdOut {
  void* dgate;
  void* dup;
  uint8_t* sg;       // kFp8: scales of dgate
  uint8_t* su;       // kFp8: scales of dup
};

// One output chunk of kN values starting at flat element e0 (a multiple of
// kN).  kFp8: the values are rounded once to fp32 (the precision of the
// scale and code decisions, as in the quantiser); a 1x32 block spans the
// 32 / kN lanes that hold its consecutive chunks (whole blocks, since
// cols % 32 == 0 and those lanes take consecutive chunks), so its amax
// (NaN ignored) is reduced across them with xor-shuffles; the first lane of
// the block stores its scale byte.
template <typename T, bool kFp8>
__device__ __forceinline__ void put_chunk(void* base, uint8_t* scale, int64_t e0, const double (&v)[Chunk<T>::kN]) {
  constexpr int kN = Chunk<T>::kN;
  if constexpr (!kFp8) {
    __builtin_nontemporal_store(Chunk<T>::pack(v), reinterpret_cast<u32x4*>(base) + e0 / kN);
  } else {
    constexpr int kLanes = 32 / kN;
    float f[kN];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < kN; ++e) {
      f[e] = (float)v[e];
      amax = fmaxf(amax, fabsf(f[e]));                  // maxNum: NaN ignored
    }
#pragma unroll
    for (int off = 1; off < kLanes; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const int E = block_exponent(amax);
    const float sc = ldexpf(1.0f, -E);
    uint8_t* q = static_cast<uint8_t*>(base) + e0;
    if constexpr (kN == 8) {
      const uint32_t lo = e4m3_pair(f[0], f[1], sc) | (e4m3_pair(f[2], f[3], sc) << 16);
      const uint32_t hi = e4m3_pair(f[4], f[5], sc) | (e4m3_pair(f[6], f[7], sc) << 16);
      __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(q));
    } else {
      __builtin_nontemporal_store(e4m3_pair(f[0], f[1], sc) | (e4m3_pair(f[2], f[3], sc) << 16),
                                  reinterpret_cast<uint32_t*>(q));
    }
    if ((e0 & 31) == 0) scale[e0 >> 5] = (uint8_t)(E + 127);
  }
}

template <typename T, int kSplit, bool kClamp, bool kWeights, bool kGrad, bool kFp8>
__global__ __launch_bounds__(kThreads) void act_bwd_kernel(const T* __restrict__ gate,
                                                           const T* __restrict__ up,
                                                           const T* __restrict__ dy,
                                                           const float* __restrict__ weights, float L,
                                                           BwdOut out, float* __restrict__ wgrad, int64_t rows,
                                                           int64_t cols) {
  constexpr int kN = Chunk<T>::kN;
  constexpr int kUnroll = 4;                        // chunks per lane in flight
  constexpr int kRowsPerBlock = kThreads / 64 / kSplit;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = wave % kSplit;                  // which of the row's kSplit waves
  const int lp = part * 64 + lane;                 // lane index within the row's waves
  const int64_t nch = cols / kN;
  __shared__ double part_sum[kThreads / 64];
  for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock; r0 < rows; r0 += (int64_t)gridDim.x * kRowsPerBlock) {
    const int64_t r = r0 + wave / kSplit;
    if (r >= rows) {
      if (kGrad && kSplit > 1) { __syncthreads(); __syncthreads(); }
      continue;
    }
    const double w = kWeights ? (double)weights[r] : 1.0;
    const u32x4* g4 = reinterpret_cast<const u32x4*>(gate + r * cols);
    const u32x4* u4 = reinterpret_cast<const u32x4*>(up + r * cols);
    const u32x4* d4 = reinterpret_cast<const u32x4*>(dy + r * cols);
    double acc = 0.0;
    for (int64_t c0 = lp; c0 < nch; c0 += 64 * kSplit * kUnroll) {
      u32x4 G[kUnroll], U[kUnroll], D[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t c = c0 + 64 * kSplit * j;
        if (c < nch) {
          G[j] = __builtin_nontemporal_load(g4 + c);
          U[j] = __builtin_nontemporal_load(u4 + c);
          D[j] = __builtin_nontemporal_load(d4 + c);
        }
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t c = c0 + 64 * kSplit * j;
        if (c >= nch) break;
        float gv[kN], uv[kN], dv[kN];
        Chunk<T>::unpack(G[j], gv);
        Chunk<T>::unpack(U[j], uv);
        Chunk<T>::unpack(D[j], dv);
        double a[kN], b[kN];
#pragma unroll
        for (int e = 0; e < kN; ++e) bwd_elem<kClamp>(gv[e], uv[e], dv[e], w, L, a[e], b[e], acc);
        put_chunk<T, kFp8>(out.dgate, out.sg, r * cols + c * kN, a);
        put_chunk<T, kFp8>(out.dup, out.su, r * cols + c * kN, b);
      }
    }
    if (kGrad) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if constexpr (kSplit == 1) {
        if (lane == 0) wgrad[r] = (float)acc;
      } else {
        // The row's waves meet in LDS; its first wave adds the parts in
        // order (the same order on every run).
        __syncthreads();
        if (lane == 0) part_sum[wave] = acc;
        __syncthreads();
        if (part == 0 && lane == 0) {
          double t = 0.0;
#pragma unroll
          for (int k = 0; k < kSplit; ++k) t += part_sum[wave + k];
          wgrad[r] = (float)t;
        }
      }
    }
  }
}

// Flat mapping, no weight_grad.  Rows hold whole chunks (cols % kN == 0),
// so chunk c lies in row c / (cols / kN).
template <typename T, bool kClamp, bool kWeights, bool kFp8>
__global__ __launch_bounds__(kThreads) void act_bwd_flat_kernel(const T* __restrict__ gate,
                                                                const T* __restrict__ up,
                                                                const T* __restrict__ dy,
                                                                const float* __restrict__ weights, float L,
                                                                BwdOut out, int64_t nchunks, int64_t row_chunks) {
  constexpr int kN = Chunk<T>::kN;
  // bf16: one chunk per step.  A bf16 chunk carries 8 elements of fp64 work
  // against 4 for fp32, and 4 chunks in flight took 116-142 VGPRs (3-4 waves
  // per SIMD, too few to hide that work); one takes 68-76, and at 4001 x 3584
  // (about one chunk per lane anyway) the pass ran 8 % faster with bf16
  // outputs and 18 % faster with E4M3 outputs.  fp32 keeps 4 in flight.
  constexpr int kUnroll = sizeof(T) == 2 ? 1 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4* g4 = reinterpret_cast<const u32x4*>(gate);
  const u32x4* u4 = reinterpret_cast<const u32x4*>(up);
  const u32x4* d4 = reinterpret_cast<const u32x4*>(dy);
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < nchunks; c0 += kUnroll * stride) {
    u32x4 G[kUnroll], U[kUnroll], D[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = c0 + j * stride;
      if (c < nchunks) {
        G[j] = __builtin_nontemporal_load(g4 + c);
        U[j] = __builtin_nontemporal_load(u4 + c);
        D[j] = __builtin_nontemporal_load(d4 + c);
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = c0 + j * stride;
      if (c >= nchunks) break;
      const double w = kWeights ? (double)weights[c / row_chunks] : 1.0;
      float gv[kN], uv[kN], dv[kN];
      Chunk<T>::unpack(G[j], gv);
      Chunk<T>::unpack(U[j], uv);
      Chunk<T>::unpack(D[j], dv);
      double a[kN], b[kN], unused = 0.0;
#pragma unroll
      for (int e = 0; e < kN; ++e) bwd_elem<kClamp>(gv[e], uv[e], dv[e], w, L, a[e], b[e], unused);
      put_chunk<T, kFp8>(out.dgate, out.sg, c * kN, a);
      put_chunk<T, kFp8>(out.dup, out.su, c * kN, b);
    }
  }
}

template <typename T> constexpr int kSplitOf = 4;   // waves per row

template <typename T, bool kFp8, bool kClamp, bool kWeights, bool kGrad>
void launch_ab(unsigned grid, const void* gate, const void* up, const void* dy, const float* w,
               float L, const BwdOut& out, float* wgrad, int64_t rows, int64_t cols, hipStream_t s) {
  hipLaunchKernelGGL((act_bwd_kernel<T, kSplitOf<T>, kClamp, kWeights, kGrad, kFp8>), dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const T*>(gate), static_cast<const T*>(up), static_cast<const T*>(dy), w, L, out,
                     wgrad, rows, cols);
}

template <typename T, bool kFp8, bool kClamp, bool kWeights>
void launch_flat(const void* gate, const void* up, const void* dy, const float* w, float L, const BwdOut& out,
                 int64_t rows, int64_t cols, hipStream_t s) {
  constexpr int kFlatMaxBlocks = 8192;
  const int64_t nch = rows * (cols / Chunk<T>::kN);
  if (nch == 0) return;                                 // no elements (cols == 0)
  const int64_t want = (nch + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < kFlatMaxBlocks ? want : kFlatMaxBlocks);
  hipLaunchKernelGGL((act_bwd_flat_kernel<T, kClamp, kWeights, kFp8>), dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const T*>(gate), static_cast<const T*>(up), static_cast<const T*>(dy), w, L, out,
                     nch, cols / Chunk<T>::kN);
}

template <typename T, bool kFp8>
void launch_typed(bool clamp, const void* gate, const void* up, const void* dy,
                  const float* weights, float limit, const BwdOut& out, float* wgrad, int64_t rows,
                  int64_t cols, hipStream_t s) {
  const bool w = weights != nullptr, g = wgrad != nullptr;
  if (!g) {
    if (clamp) {
      if (w) launch_flat<T, kFp8, true, true>(gate, up, dy, weights, limit, out, rows, cols, s);
      else launch_flat<T, kFp8, true, false>(gate, up, dy, weights, limit, out, rows, cols, s);
    } else {
      if (w) launch_flat<T, kFp8, false, true>(gate, up, dy, weights, limit, out, rows, cols, s);
      else launch_flat<T, kFp8, false, false>(gate, up, dy, weights, limit, out, rows, cols, s);
    }
    return;
  }
  constexpr int kRowsPerBlock = kThreads / 64 / kSplitOf<T>;
  const int64_t want = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const unsigned grid = (unsigned)(want < kMaxBlocks ? want : kMaxBlocks);
#define SWG_AB(C, W) launch_ab<T, kFp8, C, W, true>(grid, gate, up, dy, weights, limit, out, wgrad, rows, cols, s)
  if (clamp) {
    if (w) SWG_AB(true, true); else SWG_AB(true, false);
  } else {
    if (w) SWG_AB(false, true); else SWG_AB(false, false);
  }
#undef SWG_AB
}

}  // namespace

hipError_t launch_act_bwd(Dt dt, int64_t rows, int64_t cols, const void* gate, const void* up,
                          const void* dy, const float* weights, float limit, bool clamp,
                          void* dgate, void* dup, float* wgrad, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const BwdOut out{dgate, dup, nullptr, nullptr};
  if (dt == Dt::kBF16)
    launch_typed<bf16, false>(clamp, gate, up, dy, weights, limit, out, wgrad, rows, cols, s);
  else
    launch_typed<float, false>(clamp, gate, up, dy, weights, limit, out, wgrad, rows, cols, s);
  return hipGetLastError();
}

hipError_t launch_act_bwd_fp8(Dt dt, int64_t rows, int64_t cols, const void* gate, const void* up,
                              const void* dy, const float* weights, float limit, bool clamp, uint8_t* q_dgate,
                              uint8_t* s_dgate, uint8_t* q_dup, uint8_t* s_dup, float* wgrad, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const BwdOut out{q_dgate, q_dup, s_dgate, s_dup};
  if (dt == Dt::kBF16)
    launch_typed<bf16, true>(clamp, gate, up, dy, weights, limit, out, wgrad, rows, cols, s);
  else
    launch_typed<float, true>(clamp, gate, up, dy, weights, limit, out, wgrad, rows, cols, s);
  return hipGetLastError();
}

}  // namespace swg
