// Decode forward, 1 <= M <= 8 tokens, bf16: h = act(x Wg^T) * (x Wu^T).
//
// The work is bound by reading Wg and Wu from HBM once ("Fused SwiGLU
// benchmark", AstrAI docs/developer/swiglu_benchmark.md, sections L20
// findings and HBM re-measurement: the wide shapes are weight-bandwidth
// dominated and the fused kernel sits at the dual-stream cold-read floor).
// Two kernels, each streaming every weight row once for all M tokens:
//
// M <= 3, vector ALU: each half-wave (32 lanes) owns one output column n
// and streams the rows Wg[n, :] and Wu[n, :] with 16-byte loads (lane j
// reads chunks j, j+32, ...), 512 contiguous bytes per row per instruction;
// x [M, K] is staged in LDS and each 16-byte chunk of it is reused for both
// weights.  The dot products use the bf16 dot2 instruction (two bf16
// products into fp32 per lane-op); per lane the 2M partial sums are reduced
// across the half-wave with butterfly shuffles, and lane 0 of the half
// applies act(g) * u and stores the M outputs of its column.  x up to
// 64 KiB is staged whole, larger x in K-phases of at most about 36 KiB
// (stage x[:, phase], stream that phase's weights, move on), so there is no
// limit on K.
//
// M >= 4, matrix cores: see gemv_mfma_kernel below.  From M = 4 the vector
// ALU kernel is bound by its M LDS reads of x and 8 M dot2 per 16-byte
// weight chunk; the matrix cores take a whole 16 x 16 x 32 product per
// instruction.
//
// Each kernel has a read-only twin (kTwin): the same grid, LDS footprint,
// staging and loads, and no arithmetic; each lane folds the loaded weight
// words into one value.  Its time is the floor of that access pattern, the
// counterpart on the same buffers of the benchmark page's pure-read loop.
#include "common.hpp"
#include "gemm.hpp"

namespace swg {

namespace {

// Vector-ALU kernel: 8 waves, x is staged once per 16 columns.
constexpr int kThreads = 512;
constexpr int kColsPerBlock = 16;  // 8 waves x 2 half-waves
// x up to this size is staged whole (at 64 KiB two workgroups still share
// a CU); beyond it, in phases of at most kPhaseBytes (four per CU).
constexpr int kWholeBytes = 64 * 1024;
constexpr int kPhaseBytes = 36 * 1024;

// One half-wave's pass over chunks [0, nc) of its column's weight rows
// rg, ru, against x chunks xs[m * stride + c]: dot products into ag, au,
// or, for the twin, a fold of the loaded words.
template <int M, bool kTwin>
__device__ __forceinline__ void stream_chunks(const u32x4* __restrict__ rg, const u32x4* __restrict__ ru,
                                              const u32x4* xs, int stride, int nc, int lane,
                                              float (&ag)[M], float (&au)[M], uint32_t& fold) {
  const int hl = lane & 31;
  if constexpr (kTwin) {
    // The weight stream of the branch below (same loads, same unrolling),
    // folded into one word.
    auto eat = [&](int c) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
      fold ^= vg[0] ^ vg[1] ^ vg[2] ^ vg[3] ^ vu[0] ^ vu[1] ^ vu[2] ^ vu[3];
    };
#pragma unroll 4
    for (int c = hl; c < nc; c += 32) eat(c);
  } else {
#pragma unroll 4
    for (int c = hl; c < nc; c += 32) {
      const u32x4 vg = __builtin_nontemporal_load(rg + c);
      const u32x4 vu = __builtin_nontemporal_load(ru + c);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4 xv = xs[m * stride + c];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 xx = as_bf16x2(xv[t]);
          ag[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vg[t]), xx, ag[m], false);
          au[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vu[t]), xx, au[m], false);
        }
      }
    }
  }
}

// The end of a half-wave's column: reduce the partial sums (or folds) over
// the 32 lanes, and lane 0 stores act(g) * u for the M rows (or the fold).
template <int M, Act A, bool kTwin>
__device__ __forceinline__ void finish_column(float (&ag)[M], float (&au)[M], uint32_t fold, bool live, int hl,
                                              int col, int N, float gmul, float umul, bf16* __restrict__ h,
                                              uint32_t* __restrict__ sink) {
  if constexpr (kTwin) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) fold ^= __shfl_xor(fold, off, 32);
    if (live && hl == 0) sink[col] = fold;
    return;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      ag[m] += __shfl_xor(ag[m], off, 32);
      au[m] += __shfl_xor(au[m], off, 32);
    }
  }
  if (live && hl == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float g = gmul * ag[m], u = umul * au[m];
      const float a = (A == Act::kGeluTanh) ? gelu_tanh_f32(g) : silu_f32(g);
      h[(int64_t)m * N + col] = to_bf16(a * u);
    }
  }
}

// x staged whole (M K * 2 <= kWholeBytes).
template <int M, Act A, bool kTwin>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const bf16* __restrict__ x,
                                                        const bf16* __restrict__ wg,
                                                        const bf16* __restrict__ wu,
                                                        bf16* __restrict__ h, int N, int K,
                                                        float gmul, float umul, uint32_t* __restrict__ sink) {
  extern __shared__ u32x4 xs[];  // [M][K / 8]
  const int nch = K >> 3;
  const int tid = threadIdx.x;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);
  for (int i = tid; i < M * nch; i += kThreads) xs[i] = xg[i];
  __syncthreads();

  const int lane = tid & 63;
  const int col0 = (blockIdx.x * (kThreads / 64) + (tid >> 6)) * 2;
  if (col0 >= N) return;                           // the whole wave is past the end
  const int col = col0 + (lane >> 5);
  const bool live = col < N;
  // A half-wave past the end streams the last column again and stores
  // nothing.
  const int ccol = live ? col : N - 1;

  const u32x4* rg = reinterpret_cast<const u32x4*>(wg + (int64_t)ccol * K);
  const u32x4* ru = reinterpret_cast<const u32x4*>(wu + (int64_t)ccol * K);
  float ag[M], au[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ag[m] = au[m] = 0.0f;
  uint32_t fold = 0;
  stream_chunks<M, kTwin>(rg, ru, xs, nch, nch, lane, ag, au, fold);
  finish_column<M, A, kTwin>(ag, au, fold, live, lane & 31, col, N, gmul, umul, h, sink);
}

// x staged in phases of pch chunks per row (a multiple of 32): stage
// x[:, phase], stream the weights of that phase, move on.
template <int M, Act A, bool kTwin>
__global__ __launch_bounds__(kThreads) void gemv_phased_kernel(const bf16* __restrict__ x,
                                                               const bf16* __restrict__ wg,
                                                               const bf16* __restrict__ wu,
                                                               bf16* __restrict__ h, int N, int K, int pch,
                                                               float gmul, float umul,
                                                               uint32_t* __restrict__ sink) {
  extern __shared__ u32x4 xs[];  // [M][pch]
  const int nch = K >> 3;
  const int tid = threadIdx.x;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);

  const int lane = tid & 63;
  const int col0 = (blockIdx.x * (kThreads / 64) + (tid >> 6)) * 2;
  // A wave past the end still takes part in the staging and the barriers.
  const bool wave_live = col0 < N;
  const int col = col0 + (lane >> 5);
  const bool live = col < N;
  const int ccol = live ? col : N - 1;

  const u32x4* rg = reinterpret_cast<const u32x4*>(wg + (int64_t)ccol * K);
  const u32x4* ru = reinterpret_cast<const u32x4*>(wu + (int64_t)ccol * K);
  float ag[M], au[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ag[m] = au[m] = 0.0f;
  uint32_t fold = 0;
  for (int k0 = 0; k0 < nch; k0 += pch) {
    const int nc = min(pch, nch - k0);          // chunks of each row in this phase
    if (k0 > 0) __syncthreads();                // every wave is done with the last phase's x
    for (int i = tid; i < M * nc; i += kThreads) {
      const int m = i / nc, c = i - m * nc;
      xs[i] = xg[(int64_t)m * nch + k0 + c];
    }
    __syncthreads();
    if (wave_live) stream_chunks<M, kTwin>(rg + k0, ru + k0, xs, nc, nc, lane, ag, au, fold);
  }
  if (!wave_live) return;
  finish_column<M, A, kTwin>(ag, au, fold, live, lane & 31, col, N, gmul, umul, h, sink);
}

// ---------------------------------------------------------------- matrix cores, M >= 4
//
// From M = 4 on, the dot products go to v_mfma_f32_16x16x32_bf16 with the
// weights as the first operand (16 output columns) and x as the second (16
// token rows, rows M..15 zero).  The MFMA operand layout gives each lane one
// row and 16 bytes of k, i.e. 64 contiguous bytes per row per instruction,
// which streams from HBM at only about 5 TB/s; so the weights are loaded
// coalesced instead (a quarter-wave per row, 256 contiguous bytes of Wg or
// Wu per row per instruction), written to a wave-private LDS tile, and read
// back in operand layout.  x comes from L2 straight into operand registers.
//
// A workgroup owns 16 columns and its W waves split the reduction into
// slabs of 128 k (wave w takes slabs [w S / W, (w + 1) S / W) of S); each
// wave keeps 16 x 16 partial sums of g and u (4 + 4 floats per lane), the
// partials meet in LDS, and wave 0 adds them in wave order, applies
// act(g) * u and stores h.  Weight rows past N and k past K load as zero.
// W is 8, except for short reductions (fewer than 32 slabs, kPairs): there
// W is the largest count from 4 to 8 that divides S, so every wave walks as
// many slabs, or, when no such count exists, 8 waves (one per slab below 8)
// with shares that differ by one slab; a wave requests two slabs' weights
// before the first goes through its LDS tile.  At (6912, 1536) that is 6
// waves of 2 slabs: 1.5-1.8 % faster at M = 8; the same form is up to 2 %
// slower at the longer reductions, which keep the plain loop.  Taking the
// largest divisor down to 1 left 13, 22 and 31 slabs with 1, 2 and 1 waves:
// 8 uneven waves run (6400, 1600), (5632, 2816) and (8192, 3968) 1.56, 1.14
// and 1.64 times faster at M = 4 and 8.
constexpr int kMxWaves = 8;
constexpr int kMxThreads = kMxWaves * 64;
constexpr int kMxSlabK = 128;                    // k per slab
constexpr int kMxCPR = kMxSlabK / 8;             // 16-byte chunks per row per slab (16)
constexpr int kMxRowsPerInst = 64 / kMxCPR;      // rows one load instruction covers (4)
constexpr int kMxInst = 16 / kMxRowsPerInst;     // load instructions per weight per slab (4)
constexpr int kMxSteps = kMxSlabK / 32;          // MFMA k-steps per slab (4)
constexpr int kMxTile = 16 * kMxCPR;             // 16-byte chunks in one weight's slab tile
constexpr size_t kMxLds = (size_t)kMxWaves * 2 * kMxTile * 16;   // 64 KiB
static_assert(kMxLds >= (size_t)2 * kMxWaves * 64 * 16, "the reduction fits the tiles' LDS");

// kTwin: the same loads, LDS tiles and exchange with no arithmetic; sink[n]
// receives the XOR of every word of Wg[n, :] and Wu[n, :] as read back from
// the LDS tiles (x is loaded as in the kernel and not folded).
template <Act A, bool kTwin, bool kPairs>
__global__ __launch_bounds__(kMxThreads) void gemv_mfma_kernel(const bf16* __restrict__ x,
                                                               const bf16* __restrict__ wg,
                                                               const bf16* __restrict__ wu,
                                                               bf16* __restrict__ h, int M, int N, int K,
                                                               float gmul, float umul,
                                                               uint32_t* __restrict__ sink) {
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  const int nch = K >> 3;                         // K % 8 == 0
  const int nslab = (nch + kMxCPR - 1) / kMxCPR;
  const int nw = kPairs ? (int)(blockDim.x >> 6) : kMxWaves;   // waves in this launch
  const int s0 = (int)((int64_t)wave * nslab / nw);
  const int s1 = (int)((int64_t)(wave + 1) * nslab / nw);
  u32x4* tg = lds + wave * 2 * kMxTile;           // this wave's tiles: Wg, then Wu
  u32x4* tu = tg + kMxTile;

  // Loads: instruction i covers rows 4 i + lane / 16, chunk lane % 16 of the slab.
  const int lc = lane % kMxCPR, lr = lane / kMxCPR;
  // Operands: lane l supplies row l % 16 and chunk 4 j + l / 16 of k-step j.
  const int r16 = lane & 15, q4 = lane >> 4;
  const bool xrow = r16 < M;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (int64_t)(xrow ? r16 : 0) * K);
  const u32x4* wg4 = reinterpret_cast<const u32x4*>(wg);
  const u32x4* wu4 = reinterpret_cast<const u32x4*>(wu);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  f32x4 acc_g = {0.0f, 0.0f, 0.0f, 0.0f}, acc_u = acc_g;
  uint32_t fold = 0;
  // One slab: request its weights (and x), then through the LDS tile into
  // the matrix cores (or, for the twin, the XOR fold).
  auto load_w = [&](int s, bool live, u32x4 (&vg)[kMxInst], u32x4 (&vu)[kMxInst]) {
    const int c = s * kMxCPR + lc;
#pragma unroll
    for (int i = 0; i < kMxInst; ++i) {
      const int n = n0 + i * kMxRowsPerInst + lr;
      const bool in = live && n < N && c < nch;
      const int64_t off = in ? (int64_t)n * nch + c : 0;
      vg[i] = in ? __builtin_nontemporal_load(wg4 + off) : zero;
      vu[i] = in ? __builtin_nontemporal_load(wu4 + off) : zero;
    }
  };
  auto load_x = [&](int s, u32x4 (&vx)[kMxSteps]) {
#pragma unroll
    for (int j = 0; j < kMxSteps; ++j) {
      const int cx = s * kMxCPR + 4 * j + q4;
      vx[j] = (xrow && cx < nch) ? xr[cx] : zero;
    }
  };
  auto consume = [&](const u32x4 (&vg)[kMxInst], const u32x4 (&vu)[kMxInst], const u32x4 (&vx)[kMxSteps]) {
    // Row r, chunk c of a tile sits at chunk c ^ (r & 15): the 16 lanes that
    // write one row and the 16 that read one chunk of 16 rows each hit 16
    // distinct 16-byte bank groups.
#pragma unroll
    for (int i = 0; i < kMxInst; ++i) {
      const int r = i * kMxRowsPerInst + lr;
      tg[r * kMxCPR + (lc ^ r)] = vg[i];
      tu[r * kMxCPR + (lc ^ r)] = vu[i];
    }
#pragma unroll
    for (int j = 0; j < kMxSteps; ++j) {
      const int pc = (4 * j + q4) ^ r16;
      const u32x4 ag = tg[r16 * kMxCPR + pc];
      const u32x4 au = tu[r16 * kMxCPR + pc];
      if constexpr (kTwin) {
        fold ^= ag[0] ^ ag[1] ^ ag[2] ^ ag[3] ^ au[0] ^ au[1] ^ au[2] ^ au[3];
        asm volatile("" ::"v"(vx[j]));          // x is loaded as in the kernel
      } else {
        const bf16x8 b = __builtin_bit_cast(bf16x8, vx[j]);
        acc_g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ag), b, acc_g, 0, 0, 0);
        acc_u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, au), b, acc_u, 0, 0, 0);
      }
    }
  };
  if constexpr (kPairs) {
    // Two slabs' weights in flight before the first is consumed; the second
    // slab's x (a few KiB, from L2) is requested after, which keeps the
    // kernel within 128 VGPRs (two workgroups per CU).
    for (int s = s0; s < s1; s += 2) {
      const bool two = s + 1 < s1;
      u32x4 vg0[kMxInst], vu0[kMxInst], vx0[kMxSteps], vg1[kMxInst], vu1[kMxInst], vx1[kMxSteps];
      load_w(s, true, vg0, vu0);
      load_x(s, vx0);
      load_w(s + 1, two, vg1, vu1);
      consume(vg0, vu0, vx0);
      if (two) {
        load_x(s + 1, vx1);
        consume(vg1, vu1, vx1);
      }
    }
  } else {
    for (int s = s0; s < s1; ++s) {
      const int c = s * kMxCPR + lc;
      u32x4 vg[kMxInst], vu[kMxInst], vx[kMxSteps];
#pragma unroll
      for (int i = 0; i < kMxInst; ++i) {
        const int n = n0 + i * kMxRowsPerInst + lr;
        const bool in = n < N && c < nch;
        const int64_t off = in ? (int64_t)n * nch + c : 0;
        vg[i] = in ? __builtin_nontemporal_load(wg4 + off) : zero;
        vu[i] = in ? __builtin_nontemporal_load(wu4 + off) : zero;
      }
#pragma unroll
      for (int j = 0; j < kMxSteps; ++j) {
        const int cx = s * kMxCPR + 4 * j + q4;
        vx[j] = (xrow && cx < nch) ? xr[cx] : zero;
      }
#pragma unroll
      for (int i = 0; i < kMxInst; ++i) {
        const int r = i * kMxRowsPerInst + lr;
        tg[r * kMxCPR + (lc ^ r)] = vg[i];
        tu[r * kMxCPR + (lc ^ r)] = vu[i];
      }
#pragma unroll
      for (int j = 0; j < kMxSteps; ++j) {
        const int pc = (4 * j + q4) ^ r16;
        const u32x4 ag = tg[r16 * kMxCPR + pc];
        const u32x4 au = tu[r16 * kMxCPR + pc];
        if constexpr (kTwin) {
          fold ^= ag[0] ^ ag[1] ^ ag[2] ^ ag[3] ^ au[0] ^ au[1] ^ au[2] ^ au[3];
          asm volatile("" ::"v"(vx[j]));        // x is loaded as in the kernel
        } else {
          const bf16x8 b = __builtin_bit_cast(bf16x8, vx[j]);
          acc_g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ag), b, acc_g, 0, 0, 0);
          acc_u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, au), b, acc_u, 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();                                // every wave is done with its tiles
  if constexpr (kTwin) {
    uint32_t* rf = reinterpret_cast<uint32_t*>(lds);
    rf[wave * 64 + lane] = fold;
    __syncthreads();
    if (wave != 0) return;
    uint32_t f = 0;
    for (int w = 0; w < nw; ++w) f ^= rf[w * 64 + lane];
    f ^= __shfl_xor(f, 16);                       // the 4 lanes of a row
    f ^= __shfl_xor(f, 32);
    if (lane < 16 && n0 + lane < N) sink[n0 + lane] = f;
    return;
  }
  f32x4* red = reinterpret_cast<f32x4*>(lds);
  red[wave * 64 + lane] = acc_g;
  red[(nw + wave) * 64 + lane] = acc_u;
  __syncthreads();
  if (wave != 0) return;
  f32x4 g = red[lane], u = red[nw * 64 + lane];
  for (int w = 1; w < nw; ++w) {
    g += red[w * 64 + lane];
    u += red[(nw + w) * 64 + lane];
  }
  if (!xrow) return;
  // Accumulator layout: lane l element e is column n0 + 4 (l / 16) + e of token row l % 16.
  const int nb = n0 + 4 * q4;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float gv = gmul * g[e], uv = umul * u[e];
    const float a = (A == Act::kGeluTanh) ? gelu_tanh_f32(gv) : silu_f32(gv);
    o[e] = __builtin_bit_cast(uint16_t, to_bf16(a * uv));
  }
  bf16* dst = h + (int64_t)r16 * N + nb;
  if ((N & 3) == 0 && nb + 3 < N) {               // 8-byte aligned: h is 16-byte aligned, N % 4 == 0
    *reinterpret_cast<u32x2*>(dst) = u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (nb + e < N) dst[e] = __builtin_bit_cast(bf16, (uint16_t)o[e]);
  }
}

// M from which the matrix-core kernel is used: at M = 8 it streams 22-34 %
// faster than the vector-ALU kernel at the benchmark shapes, at M = 4 0-4 %
// faster; at M = 1 the vector-ALU kernel is up to 12 % faster.
constexpr int kMfmaFromM = 4;

template <Act A, bool kTwin>
hipError_t launch_mfma(int M, int N, int K, const void* x, const void* wg, const void* wu, void* h,
                       float gm, float um, uint32_t* sink, hipStream_t s) {
  const unsigned blocks = (unsigned)((N + 15) / 16);
  const int nslab = (K / 8 + kMxCPR - 1) / kMxCPR;
  if (nslab < 4 * kMxWaves) {
    int nw = kMxWaves;
    while (nw > 1 && nslab % nw != 0) --nw;
    if (nw < 4) nw = nslab < kMxWaves ? nslab : kMxWaves;
    const size_t lds = (size_t)nw * 2 * kMxTile * 16;   // the tiles; the reduction needs less
    hipLaunchKernelGGL((gemv_mfma_kernel<A, kTwin, true>), dim3(blocks), dim3(nw * 64), lds, s,
                       static_cast<const bf16*>(x), static_cast<const bf16*>(wg), static_cast<const bf16*>(wu),
                       static_cast<bf16*>(h), M, N, K, gm, um, sink);
  } else {
    hipLaunchKernelGGL((gemv_mfma_kernel<A, kTwin, false>), dim3(blocks), dim3(kMxThreads), kMxLds, s,
                       static_cast<const bf16*>(x), static_cast<const bf16*>(wg), static_cast<const bf16*>(wu),
                       static_cast<bf16*>(h), M, N, K, gm, um, sink);
  }
  return hipGetLastError();
}

// Chunks of each x row per phase: the fewest equal phases of at most
// kPhaseBytes, each a multiple of 32 chunks (one pass of a half-wave), which
// may add up to 31 chunks per row to a phase.
inline int phase_chunks(int M, int K) {
  const int64_t nch = K / 8;
  const int64_t nph = ((int64_t)M * nch * 16 + kPhaseBytes - 1) / kPhaseBytes;
  const int64_t per = (nch + nph - 1) / nph;
  return (int)((per + 31) / 32 * 32);
}

template <int M, Act A, bool kTwin>
hipError_t launch_m(int N, int K, const void* x, const void* wg, const void* wu, void* h,
                    float gm, float um, uint32_t* sink, hipStream_t s) {
  const unsigned blocks = (unsigned)((N + kColsPerBlock - 1) / kColsPerBlock);
  const size_t whole = (size_t)M * K * 2;
  if (whole <= (size_t)kWholeBytes) {
    hipLaunchKernelGGL((gemv_kernel<M, A, kTwin>), dim3(blocks), dim3(kThreads), whole, s,
                       static_cast<const bf16*>(x), static_cast<const bf16*>(wg),
                       static_cast<const bf16*>(wu), static_cast<bf16*>(h), N, K, gm, um, sink);
  } else {
    const int pch = phase_chunks(M, K);
    const size_t lds = (size_t)M * pch * 16;     // at most 36 KiB + 31 chunks per row
    hipLaunchKernelGGL((gemv_phased_kernel<M, A, kTwin>), dim3(blocks), dim3(kThreads), lds, s,
                       static_cast<const bf16*>(x), static_cast<const bf16*>(wg),
                       static_cast<const bf16*>(wu), static_cast<bf16*>(h), N, K, pch, gm, um, sink);
  }
  return hipGetLastError();
}

template <Act A, bool kTwin>
hipError_t launch_act(int M, int N, int K, const void* x, const void* wg, const void* wu, void* h,
                      float gm, float um, uint32_t* sink, hipStream_t s) {
  if (M >= kMfmaFromM && M <= 8) return launch_mfma<A, kTwin>(M, N, K, x, wg, wu, h, gm, um, sink, s);
  switch (M) {
    case 1: return launch_m<1, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 2: return launch_m<2, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    case 3: return launch_m<3, A, kTwin>(N, K, x, wg, wu, h, gm, um, sink, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(Act act, int M, int N, int K, const void* x, const void* wg, const void* wu,
                       void* h, float gmul, float umul, hipStream_t s) {
  return act == Act::kGeluTanh ? launch_act<Act::kGeluTanh, false>(M, N, K, x, wg, wu, h, gmul, umul, nullptr, s)
                               : launch_act<Act::kSilu, false>(M, N, K, x, wg, wu, h, gmul, umul, nullptr, s);
}

hipError_t launch_gemv_read_twin(int M, int N, int K, const void* x, const void* wg, const void* wu,
                                 uint32_t* sink, hipStream_t s) {
  return launch_act<Act::kSilu, true>(M, N, K, x, wg, wu, nullptr, 1.0f, 1.0f, sink, s);
}

}  // namespace swg
