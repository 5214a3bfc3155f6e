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
//   kGeGLU   the same with GELU (tanh form) in place of SiLU;
//   kSwiGLUq, kGeGLUq  the same h quantised per 1x32 block (UE8M0 scale
//            byte, E4M3 codes), so it leaves as the down projection's FP8
//            operand;
//   kDSwiGLU du = dh * SiLU(g), dg = dh * u * s * (1 + g (1 - s)), s = sigma(g)
//            (the backward of the same stage, Liger-Kernel issue 1383);
//            bf16 can also write [dg | du] transposed for the dW product;
//   kDGeGLU  the same with GELU-tanh and its derivative;
//   kStore   C itself, routed to one of two outputs by row.
// The gated epilogues first scale the accumulators by the projection
// multipliers (g <- gmul g, u <- umul u; exact when they are 1), and the
// dSwiGLU epilogue applies the chain rule through them.
// sigma is the accurate fp32 form for fp32 and FP8 outputs and the short
// hardware exp2 / reciprocal form (common.hpp) where the result is rounded
// to bf16.
//
// Tiling: a workgroup owns a BM x BN block tile (rows of A x rows of each
//   B), k-steps of 128 bytes per row (64 bf16 or 32 fp32), and its waves form
//   a grid in which each wave owns a sub-tile of every B operand made of
//   MFMA tiles: 16 x 16 x 32 for every bf16 product (that form sustains
//   about 10 % more throughput on this chip than 32 x 32 x 16), 32 x 32 x 2
//   for fp32.
//   In bf16 the dual GEMMs use 256 x 128 with 8 waves (4 x 2, 64 x 64 per
//   wave per weight), the single-operand GEMMs 256 x 256 with 8 waves
//   (64 x 128 per wave); both were the fastest of the tile shapes measured
//   at the 8192 x 14336 x 4096 training shapes.  fp32 uses 128 x 64 and
//   128 x 128 with 4 waves, two workgroups per CU (TileDualF32 below).
//   LDS holds two k-steps (double buffer); rows are stored as eight 16-byte
//   chunks with the chunk index XOR-swizzled (see the LDS swizzle below) so
//   the 16-byte MFMA operand reads are free of bank conflicts.
// MFMA operand mapping (32 x 32): lane l supplies row (l & 31) of its 32-row
// operand tile and the 16-byte chunk (2 kk + (l >> 5)) of the k-step; the
// same chunk mapping for A and B makes the products pair up correctly
// whatever order the matrix core uses within a chunk.  16 x 16 x 32: row
// (l & 15) and chunk (4 kk + (l >> 4)).
#include "common.hpp"
#include "fp8.hpp"
#include "gemm.hpp"

namespace swg {

namespace {


// Block tile kBM x kBN (rows of A x rows of each B), waves in a kWGM x kWGN
// grid, each wave owning (kBM / kWGM) x (kBN / kWGN) of every B operand.
template <int BM_, int BN_, int WGM_, int WGN_, int OCC_ = 0>
struct Tile {
  static constexpr int kBM = BM_, kBN = BN_, kWGM = WGM_, kWGN = WGN_;
  static constexpr int kThreads = 64 * WGM_ * WGN_;
  // Waves per SIMD the register budget is sized for (default: one workgroup per CU).
  static constexpr int kOcc = OCC_ > 0 ? OCC_ : kThreads / 256;
  static constexpr int kWM = BM_ / WGM_, kWN = BN_ / WGN_;   // wave tile
};

enum class Epi { kSwiGLU, kGeGLU, kDSwiGLU, kStore, kSwiGLUq, kGeGLUq, kDGeGLU };

// Gated forward epilogues: h = act(g) * u.
constexpr bool gated_fwd(Epi e) { return e == Epi::kSwiGLU || e == Epi::kGeGLU; }
// ... with h quantised to E4M3 per 1x32 block (UE8M0 scales).
constexpr bool gated_q(Epi e) { return e == Epi::kSwiGLUq || e == Epi::kGeGLUq; }
// Backward epilogues of the gated forward: D = [dg | du].
constexpr bool gated_bwd(Epi e) { return e == Epi::kDSwiGLU || e == Epi::kDGeGLU; }

// Tile raster: consecutive workgroups walk groups of kGroupM row-tiles down
// the columns, so the 32 tiles an XCD runs at once share kGroupM tiles of
// the first operand and 32 / kGroupM of the second.  Measured side by side
// on the bf16 products at 8192 x 14336 x 4096: 8 for the dual products
// (forward: 4 is 0.5 % slower, 2: 2.5 %, 16: 3 %, 32: 20 %; the recompute of
// the backward: 4 is 1 % slower), 4 for the single products dX and dW (2.0 %
// faster than 8 over the whole backward).  The fp32 products keep 8.
template <typename T, Epi E>
constexpr int kGroupM = (sizeof(T) == 2 && E == Epi::kStore) ? 4 : 8;

// act(z) and act'(z) for the backward epilogues.  SiLU: a = z s,
// a' = s (1 + z (1 - s)), s = sigma(z).  GELU (tanh form): a = z s and
// a' = s + z s (1 - s) t'(z) with s = sigma(t), t = z (c1 + c3 z^2),
// t' = c1 + 3 c3 z^2.  kShort: the short sigma (results rounded to bf16);
// otherwise the accurate pair sigma, 1 - sigma.
template <Epi E, bool kShort>
__device__ __forceinline__ void act_and_grad(float z, float& a, float& da) {
  if constexpr (E == Epi::kDGeGLU) {
    const float z2 = z * z;
    const float t = z * __builtin_fmaf(kGeluC3, z2, kGeluC1);
    float s, c;
    if constexpr (kShort) {
      constexpr float kL2e = 1.44269504088896340736f;
      s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t * kL2e));
      c = 1.0f - s;
    } else {
      sigmoid_pair_f32(t, s, c);
    }
    a = z * s;
    da = s + a * c * __builtin_fmaf(3.0f * kGeluC3, z2, kGeluC1);
  } else {
    float s;
    if constexpr (kShort) sigmoid_silu_bf16out(z, s, a);
    else sigmoid_silu_f32(z, s, a);
    da = s * (1.0f + z * (1.0f - s));
  }
}

template <Epi E>
__device__ __forceinline__ float act_accurate(float g) {
  if constexpr (E == Epi::kGeGLU) return gelu_tanh_f32(g);
  else return silu_f32(g);
}

template <Epi E>
__device__ __forceinline__ float act_bf16out(float g) {
  if constexpr (E == Epi::kGeGLU) {
    return gelu_tanh_bf16out(g);
  } else {
    float s, sl;
    sigmoid_silu_bf16out(g, s, sl);
    return sl;
  }
}

// LDS swizzle: the physical 16-byte chunk of logical chunk c in LDS row r
// is c ^ ((r >> 1) & 7) for 128-byte rows.  gfx950 serves a 128-bit LDS read
// for 16 lanes per cycle across 64 four-byte banks, i.e. 16 distinct 16-byte
// bank groups (group = (8 r + chunk) mod 16 for 128-byte rows).  The MFMA
// operand reads put 16 consecutive rows at one logical chunk in a lane group;
// the XOR gives those 16 rows 16 distinct groups.

// Largest row count a block tile of either operand has.
template <int BM, int BN>
__device__ __forceinline__ constexpr int r_cap() { return BM > BN ? BM : BN; }

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

// MFMA accumulator layouts.  kMN = 32 (v_mfma_f32_32x32x*): 16 floats per
// lane, lane l element e at row 8 (e >> 2) + 4 (l >> 5) + (e & 3), column
// l & 31.  kMN = 16 (v_mfma_f32_16x16x32_bf16): 4 floats per lane, lane l
// element e at row 4 (l >> 4) + e, column l & 15.  In both, elements 4q ..
// 4q + 3 are 4 consecutive rows of one column, and the 16 lanes of a group
// hold one 16-column run of those rows.
template <int kMN> struct AccL;
template <> struct AccL<32> {
  using V = f32x16;
  static constexpr int kE = 16;
  __device__ __forceinline__ static int row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }
  __device__ __forceinline__ static int col(int lane) { return lane & 31; }
};
template <> struct AccL<16> {
  using V = f32x4;
  static constexpr int kE = 4;
  __device__ __forceinline__ static int row(int lane, int e) { return 4 * (lane >> 4) + e; }
  __device__ __forceinline__ static int col(int lane) { return lane & 15; }
};

template <typename T> __device__ __forceinline__ T cvt_out(float v);
template <> __device__ __forceinline__ bf16 cvt_out<bf16>(float v) { return to_bf16(v); }
template <> __device__ __forceinline__ float cvt_out<float>(float v) { return v; }

template <typename T> __device__ __forceinline__ float load_in(const T* p);
template <> __device__ __forceinline__ float load_in<bf16>(const bf16* p) { return from_bf16(*p); }
template <> __device__ __forceinline__ float load_in<float>(const float* p) { return *p; }

// Scalar epilogue (fp32 outputs, and bf16 outputs whose row stride is not a
// whole number of 16-byte chunks), for either accumulator layout.
template <typename T, Epi E, int NB, class TL, int kMN>
__device__ __forceinline__ void store_tile(const GemmArgs& p,
                                           typename AccL<kMN>::V (&acc)[NB][TL::kWM / kMN][TL::kWN / kMN],
                                           int tm, int tn, int wm, int wn, int lane) {
  constexpr int kBM = TL::kBM, kBN = TL::kBN, kWM = TL::kWM, kWN = TL::kWN;
  constexpr int kTM = kWM / kMN, kTN = kWN / kMN;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int e = 0; e < AccL<kMN>::kE; ++e) {
        const int row = tm * kBM + wm * kWM + i * kMN + AccL<kMN>::row(lane, e);
        const int col = tn * kBN + wn * kWN + j * kMN + AccL<kMN>::col(lane);
        if (row >= p.m || col >= p.n) continue;
        if constexpr (gated_fwd(E)) {
          if (col >= p.ncols) continue;
          const float g = p.gmul * acc[0][i][j][e];
          const float u = p.umul * acc[NB - 1][i][j][e];
          T* out = static_cast<T*>(p.out0);
          out[(int64_t)row * p.ldo + col] = cvt_out<T>(act_accurate<E>(g) * u);
        } else if constexpr (gated_bwd(E)) {
          const float g = p.gmul * acc[0][i][j][e];
          const float u = p.umul * acc[NB - 1][i][j][e];
          float dh = 0.0f;
          if (col < p.ncols) dh = load_in<T>(static_cast<const T*>(p.dh) + (int64_t)row * p.lddh + col);
          float a, da;
          act_and_grad<E, false>(g, a, da);
          const float du = (dh * a) * p.umul;
          const float dg = (dh * u * da) * p.gmul;
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

// Epilogue through LDS for 16-bit outputs (used by the DMA kernel once its
// LDS ring is idle).  The MFMA accumulator layout gives each lane one column
// and runs of 4 rows, so direct stores are 2 bytes per lane.  Instead:
//   - dSwiGLU only: the dh tile, staged in LDS (DhLds below), is read back
//     in accumulator layout with ds_read_b64_tr_b16 (16 lanes addressing a
//     4-row x 16-column block receive one column each, 4 rows deep --
//     exactly a lane's run of 4 accumulator rows);
//   - results are written to LDS (2-byte writes, rows padded so the two
//     half-waves hit different banks) and read back as 16-byte row chunks
//     that are stored with coalesced 16-byte global stores.
// Needs every output row pitch (and du_off) to be a multiple of 8 elements;
// the caller uses store_tile otherwise.
template <Epi E, class TL>
struct EpiLds {
  static constexpr int kCols = TL::kBN;                      // columns per output tile
  static constexpr int kPitch = kCols * (gated_q(E) ? 4 : 2) + 32;   // bytes per staged row
  static constexpr int kRegion = TL::kBM * kPitch;
  static constexpr int kBytes = (gated_bwd(E) ? 2 : 1) * kRegion;
};

typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// dSwiGLU: the dh tile (BM rows x BN columns of bf16) is staged densely in
// the ring slot that the last k-step leaves unused: row r at r * 2 BN bytes,
// its 16-byte chunk c at physical chunk c ^ (r & 15).  When dh's row pitch
// and base allow 16-byte chunks (dh_dma below), the main loop moves the tile
// there with the LDS DMA at its last step boundary, in place of the refill
// that would have no step to fill, so the tile needs no registers while the
// accumulators and operand fragments are live; the epilogue then only fixes
// the chunks that straddle or pass the last column.  Otherwise the epilogue
// loads the whole tile element by element.
template <class TL>
struct DhLds {
  static constexpr int kCPR = TL::kBN / 8;                  // 16-byte chunks per row
  static constexpr int kPitch = TL::kBN * 2;
  __device__ static int offset(int row, int col) {          // byte offset of element (row, col)
    return row * kPitch + (((col >> 3) ^ (row & 15)) << 4) + (col & 7) * 2;
  }
};

template <Epi E, int NB, class TL, int kMN>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& p,
                                               typename AccL<kMN>::V (&acc)[NB][TL::kWM / kMN][TL::kWN / kMN],
                                               int tm, int tn, int wm, int wn, int lane, int tid,
                                               char* lds, const char* dh_lds, bool dh_dma) {
  constexpr int kBM = TL::kBM, kWM = TL::kWM, kWN = TL::kWN;
  constexpr int kTM = kWM / kMN, kTN = kWN / kMN, kE = AccL<kMN>::kE;
  constexpr int kThreads = TL::kThreads;
  constexpr int kCols = EpiLds<E, TL>::kCols;
  constexpr int kPitch = EpiLds<E, TL>::kPitch;
  constexpr int kRegion = EpiLds<E, TL>::kRegion;
  constexpr int kCPR = kCols / 8;                           // 16-byte chunks per row
  const int grow0 = tm * kBM, gcol0 = tn * kCols;

  // Staged element (row, col) of region `reg`.
  auto at = [&](int reg, int row, int col) -> char* { return lds + reg * kRegion + row * kPitch + col * 2; };

  float dhv[kTM][kTN][kE];
  if constexpr (gated_bwd(E)) {
    static_assert(DhLds<TL>::kCPR == kCPR && kCPR == 16, "dh chunk mapping; the swizzle spans 16 chunks");
    const bf16* dh = static_cast<const bf16*>(p.dh);
    char* const dst = const_cast<char*>(dh_lds);
    // Chunks the DMA did not get right: with the DMA only those of rows
    // inside the matrix that reach past the last column (rows past the end
    // came in as zeros); without it every chunk.
    const bool tail = gcol0 + kCols > p.ncols;
    if (!dh_dma || tail) {
      for (int c = tid; c < kBM * kCPR; c += kThreads) {
        const int r = c / kCPR, ch = c % kCPR;
        const int grow = grow0 + r, gcol = gcol0 + ch * 8;
        if (dh_dma && (grow >= p.m || gcol + 8 <= p.ncols)) continue;
        uint16_t tmp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (grow < p.m && gcol < p.ncols) {
          const bf16* src = dh + (int64_t)grow * p.lddh + gcol;
          const int nq = min(8, p.ncols - gcol);
          for (int q = 0; q < nq; ++q) tmp[q] = __builtin_bit_cast(uint16_t, src[q]);
        }
        *reinterpret_cast<u32x4*>(dst + DhLds<TL>::offset(r, ch * 8)) = __builtin_bit_cast(u32x4, tmp);
      }
      __syncthreads();
    }
    // dh in accumulator layout: one transposing read per 4 consecutive rows
    // of a 16-column run (lane s16 of the group addresses row s16 / 4,
    // columns 4 (s16 % 4) .. + 3 of the 4 x 16 block; lane i receives
    // column i).
    const int s16 = lane & 15;
    const int run0 = AccL<kMN>::col(lane) - s16;            // first column of the lane's 16-column run
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int eq = 0; eq < kE / 4; ++eq) {
          const int row = wm * kWM + i * kMN + AccL<kMN>::row(lane, 4 * eq) + (s16 >> 2);
          const int col = wn * kWN + j * kMN + run0 + 4 * (s16 & 3);
          const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_short4_t*)(lds_char_t*)(dh_lds + DhLds<TL>::offset(row, col)));
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dhv[i][j][4 * eq + q] = bits_f32((uint32_t)(uint16_t)v[q] << 16);
        }
    __syncthreads();
  }

  // Results into LDS.
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int row = wm * kWM + i * kMN + AccL<kMN>::row(lane, e);
        const int col = wn * kWN + j * kMN + AccL<kMN>::col(lane);
        if constexpr (gated_fwd(E)) {
          const float g = p.gmul * acc[0][i][j][e], u = p.umul * acc[NB - 1][i][j][e];
          *reinterpret_cast<bf16*>(at(0, row, col)) = to_bf16(act_bf16out<E>(g) * u);
        } else if constexpr (gated_bwd(E)) {
          const float g = p.gmul * acc[0][i][j][e], u = p.umul * acc[NB - 1][i][j][e];
          const float dh = dhv[i][j][e];
          float a, da;
          act_and_grad<E, true>(g, a, da);
          *reinterpret_cast<bf16*>(at(0, row, col)) = to_bf16((dh * u * da) * p.gmul);
          *reinterpret_cast<bf16*>(at(1, row, col)) = to_bf16((dh * a) * p.umul);
        } else {
          *reinterpret_cast<bf16*>(at(0, row, col)) = to_bf16(acc[0][i][j][e]);
        }
      }
  __syncthreads();

  // 16-byte chunks out.
  auto put = [&](bf16* dst, const u32x4& v, int nvalid) {
    if (nvalid >= 8) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      uint16_t tmp[8];
      *reinterpret_cast<u32x4*>(tmp) = v;
      for (int q = 0; q < nvalid; ++q) reinterpret_cast<uint16_t*>(dst)[q] = tmp[q];
    }
  };
  for (int c = tid; c < kBM * kCPR; c += kThreads) {
    const int r = c / kCPR, ch = c % kCPR;
    const int grow = grow0 + r, gcol = gcol0 + ch * 8;
    if (grow >= p.m || gcol >= p.n) continue;
    if constexpr (gated_fwd(E)) {
      if (gcol >= p.ncols) continue;
      put(static_cast<bf16*>(p.out0) + (int64_t)grow * p.ldo + gcol,
          *reinterpret_cast<const u32x4*>(at(0, r, ch * 8)), min(8, p.ncols - gcol));
    } else if constexpr (gated_bwd(E)) {
      bf16* dst = static_cast<bf16*>(p.out0) + (int64_t)grow * p.ldo + gcol;
      const int nv = min(8, p.n - gcol);
      put(dst, *reinterpret_cast<const u32x4*>(at(0, r, ch * 8)), nv);
      put(dst + p.du_off, *reinterpret_cast<const u32x4*>(at(1, r, ch * 8)), nv);
    } else {
      if (gcol >= p.ncols) continue;
      bf16* dst;
      if (grow < p.split) {
        if (grow >= p.lim0) continue;
        dst = static_cast<bf16*>(p.out0) + (int64_t)grow * p.ldo + gcol;
      } else {
        if (grow - p.split >= p.lim1) continue;
        dst = static_cast<bf16*>(p.out1) + (int64_t)(grow - p.split) * p.ldo + gcol;
      }
      put(dst, *reinterpret_cast<const u32x4*>(at(0, r, ch * 8)), min(8, p.ncols - gcol));
    }
  }

  // dSwiGLU: [dg | du] transposed into out1 (row n of dg, row du_off + n of
  // du, columns m), for the dW product that reduces over m.  A 16-byte chunk
  // there is 8 consecutive rows m of one column n of the staged tile: two
  // transposing reads (rows +0..3, +4..7) give each lane of a 16-lane group
  // one column.  In a wave the 4 groups take 4 consecutive chunks of the
  // same 16 columns (64 contiguous bytes per output row and instruction);
  // the two groups served together read opposite row halves first (rows 0..3 and 4..7 of
  // their chunks sit in disjoint bank halves with the 288-byte pitch), and
  // swap halves on the second read.  Rows m in [p.m, ldt) of the tile hold
  // zeros (zero x rows and dh), so out1's padding columns are written zero.
  if constexpr (gated_bwd(E)) {
    if (p.out1 != nullptr) {
      bf16* dt = static_cast<bf16*>(p.out1);
      constexpr int kNB = kCols / 16, kMQ = kBM / 32;       // 16-column blocks, 32-row groups
      const int g = lane >> 4, s16 = lane & 15, hsel = g & 1;
      // A wave takes consecutive tasks: all 32-row groups of one 16-column
      // block in turn, so each output row it touches gets 512 contiguous
      // bytes over its iterations.
      constexpr int kTasks = 2 * kNB * kMQ, kPerWave = kTasks / (kThreads / 64);
      static_assert(kTasks % (kThreads / 64) == 0, "D^T tasks per wave");
#pragma unroll 4
      for (int it = 0; it < kPerWave; ++it) {
        const int t = (tid >> 6) * kPerWave + it;
        const int reg = t / (kNB * kMQ);
        const int nb = (t / kMQ) % kNB, mq = t % kMQ;
        const int m0 = (mq * 4 + g) * 8;
        const int c = nb * 16 + 4 * (s16 & 3);
        const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4_t*)(lds_char_t*)(at(reg, m0 + 4 * hsel + (s16 >> 2), c)));
        const short4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4_t*)(lds_char_t*)(at(reg, m0 + 4 * (1 - hsel) + (s16 >> 2), c)));
        const u32x2 a = __builtin_bit_cast(u32x2, hsel ? v2 : v1);   // rows m0 .. m0 + 3
        const u32x2 b = __builtin_bit_cast(u32x2, hsel ? v1 : v2);   // rows m0 + 4 .. m0 + 7
        const int n = gcol0 + nb * 16 + s16, m = grow0 + m0;
        if (n < p.n && m < p.ldt)
          *reinterpret_cast<u32x4*>(dt + ((int64_t)reg * p.du_off + n) * p.ldt + m) = u32x4{a[0], a[1], b[0], b[1]};
      }
    }
  }
}

// FP8-output epilogue of the gated forward ("quant: add SwiGLU
// forward/backward VMI kernels", TileKernels-PTO PR 20, implementation
// notes: 1x32 blocks along the hidden dimension, packed UE8M0 scale, E4M3
// without saturation): h = act(g) * u from the fp32 accumulators (the
// activation to a few fp32 ulps, then the fp32 product) is staged in LDS
// as fp32; each thread then takes whole 1x32 blocks of a row, forms the
// block amax (NaN ignored), the UE8M0 exponent and the 32 codes, and writes
// 32 code bytes, one scale byte and optionally the fp32 h.  Needs n % 32 == 0
// (whole blocks), row strides that keep 16-byte alignment.
template <Epi E, int NB, class TL, int kMN>
__device__ __forceinline__ void store_tile_fp8(const GemmArgs& p,
                                               typename AccL<kMN>::V (&acc)[NB][TL::kWM / kMN][TL::kWN / kMN],
                                               int tm, int tn, int wm, int wn, int lane, int tid,
                                               char* lds) {
  constexpr int kBM = TL::kBM, kWM = TL::kWM, kWN = TL::kWN;
  constexpr int kTM = kWM / kMN, kTN = kWN / kMN;
  constexpr int kThreads = TL::kThreads;
  constexpr int kCols = EpiLds<E, TL>::kCols;
  constexpr int kPitch = EpiLds<E, TL>::kPitch;
  const int grow0 = tm * kBM, gcol0 = tn * kCols;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int e = 0; e < AccL<kMN>::kE; ++e) {
        const int row = wm * kWM + i * kMN + AccL<kMN>::row(lane, e);
        const int col = wn * kWN + j * kMN + AccL<kMN>::col(lane);
        const float g = p.gmul * acc[0][i][j][e], u = p.umul * acc[NB - 1][i][j][e];
        const float h = (E == Epi::kGeGLUq ? gelu_tanh_f32(g) : silu_f32(g)) * u;
        *reinterpret_cast<float*>(lds + row * kPitch + col * 4) = h;
      }
  __syncthreads();
  // Block q: row q % kBM, 32-column block q / kBM, so 16 lanes read 16 rows
  // at one column offset.
  constexpr int kBlocks = kBM * (kCols / 32);
  uint8_t* codes = static_cast<uint8_t*>(p.out0);
  uint8_t* scale = static_cast<uint8_t*>(p.q_scale);
  const int64_t lds_ = p.n / 32;
  for (int qb = tid; qb < kBlocks; qb += kThreads) {
    const int r = qb % kBM, b = qb / kBM;
    const int grow = grow0 + r, gcol = gcol0 + b * 32;
    if (grow >= p.m || gcol >= p.n) continue;
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const f32x4*>(lds + r * kPitch + b * 128 + k * 16);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int t = 0; t < 4; ++t) amax = fmaxf(amax, fabsf(v[k][t]));   // maxNum: NaN ignored
    const int ex = block_exponent(amax);
    const float sc = ldexpf(1.0f, -ex);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = e4m3_pair(v[k][0], v[k][1], sc) | (e4m3_pair(v[k][2], v[k][3], sc) << 16);
    u32x4* dst = reinterpret_cast<u32x4*>(codes + (int64_t)grow * p.ldo + gcol);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    scale[(int64_t)grow * lds_ + gcol / 32] = (uint8_t)(ex + 127);
    if (p.q_h != nullptr) {
      f32x4* hd = reinterpret_cast<f32x4*>(p.q_h + (int64_t)grow * p.ldo + gcol);
#pragma unroll
      for (int k = 0; k < 8; ++k) hd[k] = v[k];
    }
  }
}

// s_waitcnt that only bounds the vector-memory counter (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] left at
// their maxima).  The LDS DMA loads below count as vector-memory operations.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Raw buffer descriptor over [base, base + bytes): reads past the end return
// zero.  Every field goes through readfirstlane so the descriptor is known to
// be wave-uniform and lives in scalar registers (a descriptor the compiler
// thinks divergent turns each buffer access into a waterfall loop).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const T* base, int64_t bytes) {
  const uint64_t bp = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)bp);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, n, 0x00020000);
}

// Workgroup barrier without the memory fence of __syncthreads (which waits
// for every outstanding vector-memory operation, i.e. would drain the DMA
// ring).  Each wave has already waited for its own DMA of the step with
// wait_vmcnt; the empty asm statements keep the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Loads the kernel arguments the epilogue uses into scalar registers before
// the main loop.  Left to itself the compiler issues some of these scalar
// loads just before the loop; a scalar load still in flight there shares the
// LDS wait counter and completes out of order, which forces every LDS wait in
// the loop down to zero and so exposes the latency of every fragment read.
__device__ __forceinline__ void pin_epilogue_args(const GemmArgs& p) {
  asm volatile("" ::"s"(p.out0), "s"(p.out1), "s"(p.ldo), "s"(p.dh), "s"(p.lddh));
  asm volatile("" ::"s"(p.split), "s"(p.lim0), "s"(p.lim1), "s"(p.ncols), "s"(p.du_off), "s"(p.m),
               "s"(p.n));
  asm volatile("" ::"s"(p.ldt), "s"(p.q_scale), "s"(p.q_h), "s"(p.gmul), "s"(p.umul));
}

// The GEMM kernel (bf16 and fp32): the operand tiles go from global memory
// straight into LDS (buffer_load_dwordx4 ... lds, the gfx950 16-byte LDS
// DMA), through an S-stage ring of KC-chunk k-steps, with no register
// staging.  Each wave moves a fixed slab of rows of the stage (all in one
// operand); a DMA instruction writes 1 KiB of LDS in lane order, so the
// XOR swizzle is applied on the global side: the lane that lands in
// physical chunk q of row r fetches logical chunk q ^ swizzle(r).  Buffer
// descriptors bound each operand's block-tile rows, so rows past the end and
// k-chunks past the reduction length (given an out-of-range offset) read as
// zero with no branch.  Per k-step: wait for this wave's DMA of the step,
// one barrier (every wave's data has landed, and every wave has finished the
// step whose ring slot is refilled next), issue the DMA of step ks + S - 1,
// then the MFMAs, with the operand fragments of the next sub-step read from
// LDS while the current ones are in the matrix cores.
template <typename T, Epi E, int NB, class TL, int KC, int S, int kIL, int kMN>
__global__ __launch_bounds__(TL::kThreads) __attribute__((amdgpu_waves_per_eu(TL::kOcc, TL::kOcc)))
void gemm_dma_kernel(GemmArgs p) {
  constexpr int kBM = TL::kBM, kBN = TL::kBN, kThreads = TL::kThreads;
  constexpr int kWaves = kThreads / 64;
  // kMN x kMN MFMA tiles (32 x 32 x 16 or 16 x 16 x 32): each wave's
  // sub-tile is kTM x kTN of them.
  constexpr int kWM = TL::kWM, kWN = TL::kWN, kTM = kWM / kMN, kTN = kWN / kMN;
  static_assert(kMN == 16 || kMN == 32, "MFMA shape");
  constexpr int kRows = kBM + NB * kBN;                 // LDS rows per k-step
  constexpr int kRowBytes = KC * 16;
  constexpr int kStageBytes = kRows * kRowBytes;
  constexpr int kRowsPerDma = 64 / KC;                  // rows one DMA instruction covers
  constexpr int kRowsPerWave = kRows / kWaves;
  constexpr int kDma = kRowsPerWave / kRowsPerDma;      // DMA instructions per wave per k-step
  constexpr int kSwzShift = (KC == 8) ? 1 : (KC == 4 ? 2 : 3);  // log2(16 / KC)
  constexpr int kPer = Mma<T>::kPerChunk;
  static_assert(KC == 4 || KC == 8, "chunks per row");
  static_assert(kRows % (kWaves * kRowsPerDma) == 0, "DMA split");
  static_assert(kBM % kRowsPerWave == 0 && kBN % kRowsPerWave == 0, "a wave's slab lies in one operand");
  extern __shared__ u32x4 lds[];
  char* const lds_bytes = reinterpret_cast<char*>(lds);

  const int ntm = (p.m + kBM - 1) / kBM;
  const int ntn = (p.n + kBN - 1) / kBN;
  const int tile = xcd_remap(blockIdx.x, ntm * ntn);
  const int group = kGroupM<T, E> * ntn;
  const int first_m = (tile / group) * kGroupM<T, E>;
  const int gm = min(ntm - first_m, kGroupM<T, E>);
  const int tm = first_m + (tile % group) % gm;
  const int tn = (tile % group) / gm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave index through readfirstlane: the compiler then knows it is uniform,
  // so LDS-DMA bases (M0) and buffer descriptors stay in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::kWGN, wn = wave % TL::kWGN;
  const int nchunk_r = p.r / kPer;                      // r % kPer == 0 (host-checked)
  const int nk = (nchunk_r + KC - 1) / KC;
  pin_epilogue_args(p);

  // This wave's DMA slab and its operand.
  const int row0 = wave * kRowsPerWave;
  const T* base;
  int64_t ld;
  int valid;
  int local0;
  if (row0 < kBM) {
    base = static_cast<const T*>(p.a) + (int64_t)tm * kBM * p.lda;
    ld = p.lda;
    valid = p.arows - tm * kBM;
    local0 = row0;
  } else {
    const int r = row0 - kBM;
    base = static_cast<const T*>(r < kBN ? p.b0 : p.b1) + (int64_t)tn * kBN * p.ldb;
    ld = p.ldb;
    valid = p.brows - tn * kBN;
    local0 = r % kBN;
  }
  valid = valid < 0 ? 0 : (valid > (r_cap<kBM, kBN>()) ? r_cap<kBM, kBN>() : valid);
  const __amdgpu_buffer_rsrc_t rsrc = uniform_rsrc(base, valid * ld * (int64_t)sizeof(T));
  // Lane i of DMA d fills physical chunk (i % KC) of stage row
  // rr = row0 + d * kRowsPerDma + i / KC and fetches logical chunk
  // (i % KC) ^ swz(rr), swz(rr) = (rr >> kSwzShift) & (KC - 1).  row0 is a
  // multiple of 32, so swz(rr) depends on d
  // only through d's low bits: one chunk index per residue of d, and a row
  // offset that is linear in d (kept in two registers per lane).
  constexpr int kLchPeriod = (KC == 8) ? 2 : 1;
  int lch[kLchPeriod];
#pragma unroll
  for (int d = 0; d < kLchPeriod; ++d) {
    const int rr = row0 + d * kRowsPerDma + lane / KC;
    lch[d] = (lane % KC) ^ ((rr >> kSwzShift) & (KC - 1));
  }
  const uint32_t voff0 = (uint32_t)((int64_t)(local0 + lane / KC) * ld * (int64_t)sizeof(T));
  const uint32_t dstride = (uint32_t)((int64_t)kRowsPerDma * ld * (int64_t)sizeof(T));
  auto issue = [&](int ks) {
    char* dst = lds_bytes + (ks % S) * kStageBytes + row0 * kRowBytes;
    uint32_t koff[kLchPeriod];
    bool kin[kLchPeriod];
#pragma unroll
    for (int q = 0; q < kLchPeriod; ++q) {
      const int kc = ks * KC + lch[q];
      kin[q] = kc < nchunk_r;
      koff[q] = voff0 + (uint32_t)(kc * kPer * (int)sizeof(T));
    }
#pragma unroll
    for (int d = 0; d < kDma; ++d) {
      const int q = d % kLchPeriod;
      const uint32_t off = kin[q] ? koff[q] + (uint32_t)d * dstride : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + d * 1024), 16, off, 0, 0, 0);
    }
  };

  // dSwiGLU (bf16): the dh tile goes by DMA into the ring slot of step
  // nk - 2, which no step refills, when dh's pitch and base allow whole
  // 16-byte chunks; the epilogue writes D from the fp32 accumulators only
  // through the LDS path (vec), so the tile is not moved otherwise.
  constexpr bool kDhDma = gated_bwd(E) && sizeof(T) == 2;
  const bool dh_dma = kDhDma && nk >= 1 && p.lddh % 8 == 0 && (reinterpret_cast<uintptr_t>(p.dh) & 15) == 0 &&
                      p.ldo % 8 == 0 && p.du_off % 8 == 0;
  const int dh_slot = nk % S;   // S == 2: the slot of step nk - 2 (slot 1 when nk == 1)
  // Wave w moves rows 32 w .. 32 w + 31 of the tile (the same 8 KiB of the
  // slot as its ring slab): DMA d takes rows 32 w + 4 d .. + 3, lane i lands
  // in row 32 w + 4 d + i / 16, physical chunk i % 16, and fetches logical
  // chunk (i % 16) ^ (row & 15).  Rows past the matrix read as zero through
  // the descriptor; chunks past the last column are fixed by the epilogue.
  auto issue_dh = [&]() {
    static_assert(!kDhDma || (S == 2 && kBM * DhLds<TL>::kPitch == kStageBytes &&
                              kBM * DhLds<TL>::kPitch / kWaves == kDma * 1024),
                  "the dh tile fills one ring slot, 8 DMAs per wave");
    const bf16* dh_tile = static_cast<const bf16*>(p.dh) + (int64_t)tm * kBM * p.lddh + (int64_t)tn * kBN;
    int rows = p.m - tm * kBM;
    rows = rows < 0 ? 0 : (rows > kBM ? kBM : rows);
    int cols = p.ncols - tn * kBN;
    cols = cols < 0 ? 0 : (cols > kBN ? kBN : cols);
    // The descriptor ends at the tile's last element inside dh, so no read
    // leaves dh: earlier rows' chunks past the last column read the next
    // row (fixed by the epilogue), the last row's read zeros.
    const int64_t bytes = (rows > 0 && cols > 0) ? ((int64_t)(rows - 1) * p.lddh + cols) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rd = uniform_rsrc(dh_tile, bytes);
    char* dst = lds_bytes + dh_slot * kStageBytes + wave * (kBM / kWaves) * DhLds<TL>::kPitch;
    const int pc = lane & 15, rq = lane >> 4;
    const uint32_t rowb = (uint32_t)(p.lddh * 2);
    const uint32_t base = (uint32_t)(wave * (kBM / kWaves) + rq) * rowb;
#pragma unroll
    for (int d = 0; d < kDma; ++d) {
      const uint32_t off = base + (uint32_t)(4 * d) * rowb + (uint32_t)((pc ^ ((4 * d + rq) & 15)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t*)(dst + d * 1024), 16, off, 0, 0, 0);
    }
  };
  // The refill at a step boundary, or at the last boundary the dh tile.
  auto refill = [&](int ks, bool last) {
    if (kDhDma && last && dh_dma) issue_dh();
    else issue(ks);
  };

  static_assert(sizeof(T) == 2 || kMN == 32, "fp32 operands use the 32 x 32 x 2 MFMA");
  typename AccL<kMN>::V acc[NB][kTM][kTN];
#pragma unroll
  for (int w = 0; w < NB; ++w)
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int e = 0; e < AccL<kMN>::kE; ++e) acc[w][i][j][e] = 0.0f;

  // MFMA operand mapping: a sub-step covers kCPS = 64 / kMN 16-byte chunks
  // of the k-step (16 bf16 k for 32 x 32 x 16, 32 for 16 x 16 x 32, 8 fp32 k
  // for 32 x 32 x 2 taken 4 MFMAs at a time); lane l supplies row l % kMN of
  // its operand tile and chunk kCPS kk + l / kMN of the k-step.
  // The same chunk mapping for A and B pairs the products.
  constexpr int kCPS = 64 / kMN;
  const int rl = lane % kMN;
  const int ql = lane / kMN;
  auto frag = [&](const char* L, int row, int ch) -> u32x4 {
    const int pc = ch ^ ((row >> kSwzShift) & (KC - 1));
    return *reinterpret_cast<const u32x4*>(L + row * kRowBytes + pc * 16);
  };

  // Operand fragments of one sub-step, double-buffered in registers.
  u32x4 av[2][kTM], bv[2][NB][kTN];
  auto read_frags = [&](int buf, const char* L, int kk) {
    const int ch = kCPS * kk + ql;
#pragma unroll
    for (int i = 0; i < kTM; ++i) av[buf][i] = frag(L, wm * kWM + i * kMN + rl, ch);
#pragma unroll
    for (int w = 0; w < NB; ++w)
#pragma unroll
      for (int j = 0; j < kTN; ++j) bv[buf][w][j] = frag(L, kBM + w * kBN + wn * kWN + j * kMN + rl, ch);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int w = 0; w < NB; ++w)
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          if constexpr (kMN == 16)
            acc[w][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[buf][i]),
                                                                   __builtin_bit_cast(bf16x8, bv[buf][w][j]),
                                                                   acc[w][i][j], 0, 0, 0);
          else
            Mma<T>::run(acc[w][i][j], av[buf][i], bv[buf][w][j]);
        }
  };
  // Wait until at most `later` of this wave's DMA steps are still in flight
  // (DMA completes in issue order, so every earlier step has landed), and
  // until its own LDS reads are done, so no slot it read is still being read
  // when the barrier lets another wave's DMA refill it.
  auto wait_dma = [&](int later) {
    static_assert(S <= 5 && (S - 2) * kDma < 64, "wait table");
    if (later <= 0) wait_vmcnt<0>();
    else if (later == 1) wait_vmcnt<kDma>();
    else if (later == 2) wait_vmcnt<2 * kDma < 64 ? 2 * kDma : 0>();
    else wait_vmcnt<3 * kDma < 64 ? 3 * kDma : 0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0), other counters free
  };

  // Schedule.  The ring holds S steps; the prologue fills it.  The
  // fragments of sub-step kk + 1 are read before the MFMAs of sub-step kk
  // (scheduling fences keep the two register sets apart), and the step
  // boundary sits inside the last sub-step: wait for the next step's DMA,
  // barrier, refill the slot of the step just consumed with step ks + S, and
  // read the next step's first fragments before the last MFMAs of this
  // step.  So no LDS read latency is exposed in the steady state.
  constexpr int kKK = KC / kCPS;                        // sub-steps per k-step
  static_assert(kKK % 2 == 0, "the next step's first fragments go to buffer 0");
#pragma unroll
  for (int s0 = 0; s0 < S; ++s0)
    if (kIL >= 1 || s0 < nk) issue(s0);   // with kIL every ring step is issued
  if (nk > 0) {
    wait_dma(min(S - 1, nk - 1));
    barrier_no_fence();
    read_frags(0, lds_bytes, 0);
  }
  // One k-step; `more` (a constant after inlining) says whether a next step
  // follows.  The last step is peeled off so the steady-state loop has no
  // branch around the next step's fragment reads: at such a join the
  // compiler's LDS wait counts would have to cover both paths, and the last
  // MFMAs of every step would wait for the next step's reads.
  auto kstep = [&](int ks, bool more, bool last) {
    const char* L = lds_bytes + (ks % S) * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      constexpr int kMf = NB * kTM * kTN;
      constexpr int kRd = kTM + NB * kTN;
      if (kk + 1 < kKK) {
        if constexpr (kIL >= 2) {
          // Fragment reads of the next sub-step spread between the MFMAs.
          __builtin_amdgcn_sched_barrier(0);
          read_frags((kk + 1) & 1, L, kk + 1);
          mfmas(kk & 1);
#pragma unroll
          for (int t = 0; t < kRd; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        read_frags((kk + 1) & 1, L, kk + 1);
      } else if (more) {
        if constexpr (kIL >= 1) {
          // The refill is issued for every step (steps past the end read
          // nothing: their offsets are out of range and land zeros in a dead
          // slot), so the wait is always for the newest step in flight.
          wait_dma(S - 2);
          barrier_no_fence();
          if constexpr (kIL == 3) {
            // After the barrier: a few MFMAs of this sub-step, then the next
            // step's first fragment reads, then the refill DMAs, then the
            // rest of the MFMAs.  The compiler keeps every fragment read
            // before every refill DMA (it cannot tell the two ring slots
            // apart), so the reads and DMAs go in bursts.  Against the plain
            // boundary below: 3.3 % faster for the forward dual GEMM at
            // 8192 x 14336 x 4096 and 1.5 % for the whole backward through
            // its recompute, 0.9 % slower for the single products,
            // bit-identical either way.  Other orders, written in source
            // order, were slower or equal: a read and a DMA between each
            // group of MFMAs, or the DMAs first.
            __builtin_amdgcn_sched_barrier(0);
            read_frags(0, lds_bytes + ((ks + 1) % S) * kStageBytes, 0);
            refill(ks + S, last);
            mfmas(kk & 1);
            constexpr int kLead = kMf / kDma > 0 ? kMf / kDma : 1;
            __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, kDma, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, kMf - kLead, 0);
            __builtin_amdgcn_sched_barrier(0);
            continue;
          }
          read_frags(0, lds_bytes + ((ks + 1) % S) * kStageBytes, 0);
          // The DMA instructions of the refill go one by one between the
          // MFMAs of this sub-step instead of stalling the matrix core.
          __builtin_amdgcn_sched_barrier(0);
          refill(ks + S, last);
          mfmas(kk & 1);
          constexpr int kPerDma = kMf / kDma > 0 ? kMf / kDma : 1;
#pragma unroll
          for (int t = 0; t < kDma; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, kPerDma, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        } else {
          wait_dma(min(S - 2, nk - 2 - ks));   // step ks + 1 has landed
          barrier_no_fence();                  // and every wave has read step ks
          if (ks + S < nk) issue(ks + S);      // refills the slot of step ks
          read_frags(0, lds_bytes + ((ks + 1) % S) * kStageBytes, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(kk & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (kDhDma) {
    // The last step boundary (that of step nk - 2) is peeled off to move the
    // dh tile; with a single step the tile goes after the prologue, whose
    // barrier has retired every wave's DMA into the unused slot.
    static_assert(kIL >= 1, "the refill at the last boundary is unconditional");
    for (int ks = 0; ks + 2 < nk; ++ks) kstep(ks, true, false);
    if (nk >= 2) kstep(nk - 2, true, true);
    else if (nk == 1 && dh_dma) issue_dh();
  } else {
    for (int ks = 0; ks + 1 < nk; ++ks) kstep(ks, true, false);
  }
  if (nk > 0) kstep(nk - 1, false, false);

  if constexpr (gated_q(E)) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier_no_fence();
    store_tile_fp8<E, NB, TL, kMN>(p, acc, tm, tn, wm, wn, lane, tid, lds_bytes);
  } else {
    if constexpr (sizeof(T) == 2) {
      const bool vec = (p.ldo % 8 == 0) && (!gated_bwd(E) || p.du_off % 8 == 0);
      if (vec) {
        wait_vmcnt<0>();                      // no DMA still landing in the ring
        __builtin_amdgcn_s_waitcnt(0xC07F);   // own LDS reads done
        barrier_no_fence();                   // every wave is done with the ring
        store_tile_lds<E, NB, TL, kMN>(p, acc, tm, tn, wm, wn, lane, tid, lds_bytes,
                                       lds_bytes + dh_slot * kStageBytes, dh_dma);
        return;
      }
    }
    // No ring DMA (a refill with no step to fill) may still be landing in
    // this workgroup's LDS when its waves end.
    wait_vmcnt<0>();
    store_tile<T, E, NB, TL, kMN>(p, acc, tm, tn, wm, wn, lane);
  }
}

template <typename T, Epi E, int NB, class TL, int KC, int S, int kIL = 0, int kMN = 16>
hipError_t launch_dma(const GemmArgs& a, hipStream_t s) {
  const int ntm = (a.m + TL::kBM - 1) / TL::kBM;
  const int ntn = (a.n + TL::kBN - 1) / TL::kBN;
  const int64_t tiles = (int64_t)ntm * ntn;
  if (tiles == 0) return hipSuccess;
  const size_t ring = (size_t)S * (TL::kBM + NB * TL::kBN) * KC * 16;
  const size_t epi = sizeof(T) == 2 ? (size_t)EpiLds<E, TL>::kBytes : 0;
  const size_t lds = ring > epi ? ring : epi;
  const hipError_t attr = allow_lds<&gemm_dma_kernel<T, E, NB, TL, KC, S, kIL, kMN>>(lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_dma_kernel<T, E, NB, TL, KC, S, kIL, kMN>), dim3((unsigned)tiles), dim3(TL::kThreads), lds, s, a);
  return hipGetLastError();
}

using TileDual = Tile<256, 128, 4, 2>;   // 8 waves, 64 x 64 per wave per weight
using TileSingle = Tile<256, 256, 4, 2>; // 8 waves, 64 x 128 per wave
// fp32: the matrix cores take 16 times longer per operand byte, so small
// tiles cost little in operand traffic, and they fill the 256 CUs more
// evenly (4001 x 3584: 1,792 tiles of 128 x 64 against 448 of 256 x 128);
// 4 waves, two workgroups per CU.
using TileDualF32 = Tile<128, 64, 2, 2, 2>;     // 64 x 32 per wave per weight
using TileSingleF32 = Tile<128, 128, 2, 2, 2>;  // 64 x 64 per wave

}  // namespace

// The bf16 dual products (forward and recompute) use the interleaved step
// boundary (kIL = 3), the single products the plain one (kIL = 2): each the
// faster at the training shape.
hipError_t launch_fwd_dual(Dt dt, Act act, const GemmArgs& a, hipStream_t s) {
  if (act == Act::kGeluTanh)
    return dt == Dt::kBF16 ? launch_dma<bf16, Epi::kGeGLU, 2, TileDual, 8, 2, 3>(a, s)
                           : launch_dma<float, Epi::kGeGLU, 2, TileDualF32, 8, 2, 2, 32>(a, s);
  return dt == Dt::kBF16 ? launch_dma<bf16, Epi::kSwiGLU, 2, TileDual, 8, 2, 3>(a, s)
                         : launch_dma<float, Epi::kSwiGLU, 2, TileDualF32, 8, 2, 2, 32>(a, s);
}

hipError_t launch_fwd_dual_fp8(Act act, const GemmArgs& a, hipStream_t s) {
  return act == Act::kGeluTanh ? launch_dma<bf16, Epi::kGeGLUq, 2, TileDual, 8, 2, 3>(a, s)
                               : launch_dma<bf16, Epi::kSwiGLUq, 2, TileDual, 8, 2, 3>(a, s);
}

hipError_t launch_bwd_dswiglu(Dt dt, Act act, const GemmArgs& a, hipStream_t s) {
  if (act == Act::kGeluTanh)
    return dt == Dt::kBF16 ? launch_dma<bf16, Epi::kDGeGLU, 2, TileDual, 8, 2, 3>(a, s)
                           : launch_dma<float, Epi::kDGeGLU, 2, TileDualF32, 8, 2, 2, 32>(a, s);
  return dt == Dt::kBF16 ? launch_dma<bf16, Epi::kDSwiGLU, 2, TileDual, 8, 2, 3>(a, s)
                         : launch_dma<float, Epi::kDSwiGLU, 2, TileDualF32, 8, 2, 2, 32>(a, s);
}

hipError_t launch_gemm_store(Dt dt, const GemmArgs& a, hipStream_t s) {
  return dt == Dt::kBF16 ? launch_dma<bf16, Epi::kStore, 1, TileSingle, 8, 2, 2>(a, s)
                         : launch_dma<float, Epi::kStore, 1, TileSingleF32, 8, 2, 2, 32>(a, s);
}

}  // namespace swg
