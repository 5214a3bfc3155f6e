// GEMM-shaped kernels of the fused SwiGLU stage on gfx950 matrix cores.
//
// One kernel template computes C[m, n] = sum_r A[m, r] * B[n, r] with both
// operands reduction-contiguous.  With two B operands (Wg and Wu) it is the
// dual GEMM of the forward pass: the A tile (x) is staged in LDS once per
// k-step and feeds both weight tiles, and the epilogue works on the fp32
// accumulators ("Another MLP implementation along with multiplier support",
// Liger-Kernel issue 937, TL;DR approach 3: a dual GEMM with the activation;
// "[RFC] Testing Methodology for FP32 Convergence Tests on Fused
// SwiGLU/dSwiGLU Kernels", Liger-Kernel issue 1383, Background: gate/up GEMM
// and SwiGLU in one kernel so g and u never reach memory).
//
// Epilogues:
//   kSwiGLU  h = SiLU(g) * u, one rounding to the output type (the activation
//            is applied to the fp32 accumulator, as in the numerics follow-up
//            of "VisualGen MLP: cublasLt GELU-tanh epilogue for the
//            unquantized bf16 path", TensorRT-LLM PR 17693);
//   kDSwiGLU du = dh * SiLU(g), dg = dh * u * s * (1 + g (1 - s)), s = sigma(g)
//            (the backward of the same stage, Liger-Kernel issue 1383);
//   kStore   C itself, routed to one of two outputs by row.
//
// Tiling: a workgroup owns a BM x BN block tile (rows of A x rows of each
//   B), k-steps of 128 bytes per row (64 bf16 or 32 fp32), and its waves form
//   a grid in which each wave owns a sub-tile of every B operand made of
//   32 x 32 MFMA tiles.  The dual GEMMs use 256 x 128 with 8 waves (4 x 2,
//   64 x 64 per wave per weight), the single-operand GEMMs 256 x 256 with 8
//   waves (64 x 128 per wave); both were the fastest of the tile shapes
//   measured at the 8192 x 14336 x 4096 training shapes.  LDS holds two k-steps
//   (double buffer); rows are stored as eight 16-byte chunks with the chunk
//   index XOR-swizzled by (row & 7), so the 16-byte MFMA operand reads of 8
//   consecutive rows hit 8 distinct bank groups.
// MFMA operand mapping: lane l supplies row (l & 31) of its 32-row operand
// tile and the 16-byte chunk (2 kk + (l >> 5)) of the k-step; the same chunk
// mapping for A and B makes the products pair up correctly whatever order
// the matrix core uses within a chunk.
#include <mutex>

#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

constexpr int kChunks = 8;          // 16-byte chunks per row per k-step
constexpr int kGroupM = 8;          // tile raster: groups of 8 row-tiles

// Block tile kBM x kBN (rows of A x rows of each B), waves in a kWGM x kWGN
// grid, each wave owning (kBM / kWGM) x (kBN / kWGN) of every B operand.
template <int BM_, int BN_, int WGM_, int WGN_>
struct Tile {
  static constexpr int kBM = BM_, kBN = BN_, kWGM = WGM_, kWGN = WGN_;
  static constexpr int kThreads = 64 * WGM_ * WGN_;
  static constexpr int kWM = BM_ / WGM_, kWN = BN_ / WGN_;   // wave tile
  static constexpr int kTM = kWM / 32, kTN = kWN / 32;       // 32x32 MFMA tiles per wave
};

enum class Epi { kSwiGLU, kDSwiGLU, kStore };

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int kPerChunk = 4;
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bits_f32(a[t]), bits_f32(b[t]), acc, 0, 0, 0);
  }
};

template <typename T> __device__ __forceinline__ T cvt_out(float v);
template <> __device__ __forceinline__ bf16 cvt_out<bf16>(float v) { return to_bf16(v); }
template <> __device__ __forceinline__ float cvt_out<float>(float v) { return v; }

template <typename T> __device__ __forceinline__ float load_in(const T* p);
template <> __device__ __forceinline__ float load_in<bf16>(const bf16* p) { return from_bf16(*p); }
template <> __device__ __forceinline__ float load_in<float>(const float* p) { return *p; }

template <typename T, Epi E, int NB, class TL>
__global__ __launch_bounds__(TL::kThreads) void gemm_kernel(GemmArgs p) {
  constexpr int kBM = TL::kBM, kBN = TL::kBN, kThreads = TL::kThreads;
  constexpr int kTM = TL::kTM, kTN = TL::kTN, kWM = TL::kWM, kWN = TL::kWN;
  constexpr int kRows = kBM + NB * kBN;                 // LDS rows per k-step
  constexpr int kUnits = kRows * kChunks / kThreads;    // 16-byte loads per thread
  constexpr int kPer = Mma<T>::kPerChunk;
  extern __shared__ u32x4 lds[];                        // [2][kRows * kChunks]

  const int ntm = (p.m + kBM - 1) / kBM;
  const int ntn = (p.n + kBN - 1) / kBN;
  const int tile = xcd_remap(blockIdx.x, ntm * ntn);
  const int group = kGroupM * ntn;
  const int first_m = (tile / group) * kGroupM;
  const int gm = min(ntm - first_m, kGroupM);
  const int tm = first_m + (tile % group) % gm;
  const int tn = (tile % group) / gm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / TL::kWGN, wn = wave % TL::kWGN;

  const T* A = static_cast<const T*>(p.a);
  const T* B0 = static_cast<const T*>(p.b0);
  const T* B1 = static_cast<const T*>(p.b1);
  const int nchunk_r = p.r / kPer;                      // r % kPer == 0 (host-checked)
  const int nk = (nchunk_r + kChunks - 1) / kChunks;

  // Global -> register staging of one k-step.  Thread t moves the 16-byte
  // chunk (t & 7) of rows (t >> 3) + (kThreads / 8) i of each operand tile.
  constexpr int kRowsPerPass = kThreads / kChunks;
  constexpr int kUA = kBM / kRowsPerPass;               // loads for A
  constexpr int kUB = kBN / kRowsPerPass;               // loads per B
  static_assert(kUnits == kUA + NB * kUB, "staging split");
  const int trow = tid >> 3, tch = tid & 7;
  u32x4 stage[kUnits];
  auto gload = [&](int ks) {
    const int kc = ks * kChunks + tch;
    const bool kin = kc < nchunk_r;
    const int64_t koff = (int64_t)kc * kPer;
#pragma unroll
    for (int i = 0; i < kUA; ++i) {
      const int g = tm * kBM + trow + kRowsPerPass * i;
      stage[i] = (kin && g < p.arows) ? *reinterpret_cast<const u32x4*>(A + (int64_t)g * p.lda + koff)
                                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int w = 0; w < NB; ++w) {
      const T* B = w == 0 ? B0 : B1;
#pragma unroll
      for (int i = 0; i < kUB; ++i) {
        const int g = tn * kBN + trow + kRowsPerPass * i;
        stage[kUA + w * kUB + i] =
            (kin && g < p.brows) ? *reinterpret_cast<const u32x4*>(B + (int64_t)g * p.ldb + koff)
                                 : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
    u32x4* L = lds + buf * (kRows * kChunks);
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int row = trow + kRowsPerPass * i;          // rows of A, then B0, then B1
      L[row * kChunks + (tch ^ (row & 7))] = stage[i];
    }
  };

  f32x16 acc[NB][kTM][kTN];
#pragma unroll
  for (int w = 0; w < NB; ++w)
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[w][i][j][e] = 0.0f;

  if (nk > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
    if (nk > 1) gload(1);
  }
  const int r32 = lane & 31;
  const int half = lane >> 5;
  for (int ks = 0; ks < nk; ++ks) {
    const u32x4* L = lds + (ks & 1) * (kRows * kChunks);
#pragma unroll
    for (int kk = 0; kk < kChunks / 2; ++kk) {
      const int ch = 2 * kk + half;
      u32x4 av[kTM], bv[NB][kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int row = wm * kWM + i * 32 + r32;
        av[i] = L[row * kChunks + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int w = 0; w < NB; ++w)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          const int row = kBM + w * kBN + wn * kWN + j * 32 + r32;
          bv[w][j] = L[row * kChunks + (ch ^ (row & 7))];
        }
#pragma unroll
      for (int w = 0; w < NB; ++w)
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j) Mma<T>::run(acc[w][i][j], av[i], bv[w][j]);
    }
    if (ks + 1 < nk) lstore((ks + 1) & 1);
    if (ks + 2 < nk) gload(ks + 2);
    __syncthreads();
  }

  // Epilogue.  32 x 32 accumulator layout: lane l, element e holds
  // row 8 (e >> 2) + 4 (l >> 5) + (e & 3), column l & 31.
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = tm * kBM + wm * kWM + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        const int col = tn * kBN + wn * kWN + j * 32 + r32;
        if (row >= p.m || col >= p.n) continue;
        if constexpr (E == Epi::kSwiGLU) {
          if (col >= p.ncols) continue;
          const float g = acc[0][i][j][e];
          const float u = acc[NB - 1][i][j][e];
          T* out = static_cast<T*>(p.out0);
          out[(int64_t)row * p.ldo + col] = cvt_out<T>(silu_f32(g) * u);
        } else if constexpr (E == Epi::kDSwiGLU) {
          const float g = acc[0][i][j][e];
          const float u = acc[NB - 1][i][j][e];
          float dh = 0.0f;
          if (col < p.ncols) dh = load_in<T>(static_cast<const T*>(p.dh) + (int64_t)row * p.lddh + col);
          float s, sg;
          sigmoid_silu_f32(g, s, sg);
          const float du = dh * sg;
          const float dg = dh * u * (s * (1.0f + g * (1.0f - s)));
          T* out = static_cast<T*>(p.out0) + (int64_t)row * p.ldo;
          out[col] = cvt_out<T>(dg);
          out[p.du_off + col] = cvt_out<T>(du);
        } else {
          if (col >= p.ncols) continue;
          T* out;
          if (row < p.split) {
            if (row >= p.lim0) continue;
            out = static_cast<T*>(p.out0) + (int64_t)row * p.ldo;
          } else {
            if (row - p.split >= p.lim1) continue;
            out = static_cast<T*>(p.out1) + (int64_t)(row - p.split) * p.ldo;
          }
          out[col] = cvt_out<T>(acc[0][i][j][e]);
        }
      }
}

template <typename T, Epi E, int NB, class TL>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int ntm = (a.m + TL::kBM - 1) / TL::kBM;
  const int ntn = (a.n + TL::kBN - 1) / TL::kBN;
  const int64_t tiles = (int64_t)ntm * ntn;
  if (tiles == 0) return hipSuccess;
  const size_t lds = 2u * (TL::kBM + NB * TL::kBN) * kChunks * sizeof(u32x4);
  // Allow more than the default 64 KiB of dynamic LDS (idempotent; done once).
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [&] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<T, E, NB, TL>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_kernel<T, E, NB, TL>), dim3((unsigned)tiles), dim3(TL::kThreads), lds, s, a);
  return hipGetLastError();
}

using TileDual = Tile<256, 128, 4, 2>;   // 8 waves, 64 x 64 per wave per weight
using TileSingle = Tile<256, 256, 4, 2>; // 8 waves, 64 x 128 per wave

}  // namespace

hipError_t launch_fwd_dual(Dt dt, const GemmArgs& a, hipStream_t s) {
  return dt == Dt::kBF16 ? launch<bf16, Epi::kSwiGLU, 2, TileDual>(a, s)
                         : launch<float, Epi::kSwiGLU, 2, TileDual>(a, s);
}

hipError_t launch_bwd_dswiglu(Dt dt, const GemmArgs& a, hipStream_t s) {
  return dt == Dt::kBF16 ? launch<bf16, Epi::kDSwiGLU, 2, TileDual>(a, s)
                         : launch<float, Epi::kDSwiGLU, 2, TileDual>(a, s);
}

hipError_t launch_gemm_store(Dt dt, const GemmArgs& a, hipStream_t s) {
  return dt == Dt::kBF16 ? launch<bf16, Epi::kStore, 1, TileSingle>(a, s)
                         : launch<float, Epi::kStore, 1, TileSingle>(a, s);
}

}  // namespace swg
