/*
 * libswiglu -- the fused SwiGLU gate/up stage on AMD Instinct MI355X (gfx950).
 *
 *   h = SiLU(x Wg^T) (*) (x Wu^T),  SiLU(z) = z * sigmoid(z)
 *
 * Plain C ABI: device pointers, sizes and a HIP stream passed as void*.  No
 * torch types, no allocation, no synchronisation: every call validates its
 * arguments on the host and then only enqueues kernels on `stream`.
 *
 * Common conventions
 *   - All tensor pointers are DEVICE pointers to dense row-major arrays.
 *   - Weights use the nn.Linear layout Wg, Wu [N, K] and are applied as
 *     x @ W^T ("VisualGen MLP: cublasLt GELU-tanh epilogue for the
 *     unquantized bf16 path", TensorRT-LLM PR 17693, section Change: the
 *     up-projection is addmm(bias, x2d, weight.t()) on a [M, in] view).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is ordered on
 *     it; the call returns before the work is done.
 *   - The caller owns every buffer.  Outputs must not alias inputs or each
 *     other.  Tensor pointers must be 16-byte aligned (the kernels use
 *     128-bit loads and stores) unless an entry point states otherwise.
 *   - Devices: calls run on the current HIP device; buffers and `stream` must
 *     belong to it.
 *   - Return value: SWIGLU_OK or an error code.  On an error nothing has been
 *     enqueued and no output has been written.  Sizes of zero are valid and
 *     enqueue only what is needed to give the outputs their defined values.
 *   - Calls are thread-safe: the library's only global state is a
 *     thread-local record of the last HIP error, a once-per-device kernel
 *     attribute (the larger dynamic LDS size), the addresses of two static
 *     device arrays on each device (swiglu_bwd_noalloc's scratch buffer and
 *     the clamp count's slots), all set under call_once, and the counter
 *     that hands the count slots' regions out in turn.  A call's device
 *     arrays are those of the device its stream belongs to.
 *     swiglu_bwd_noalloc and the counting calls of swiglu_act_quant and
 *     swiglu_act_fwd alone share device memory between calls (see there).
 */
#ifndef SWIGLU_H_
#define SWIGLU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum swiglu_status {
  SWIGLU_OK = 0,
  SWIGLU_ERR_NULL = 1,        /* a required pointer is NULL                     */
  SWIGLU_ERR_SHAPE = 2,       /* a size is negative or breaks a layout rule     */
  SWIGLU_ERR_DTYPE = 3,       /* unknown dtype code                             */
  SWIGLU_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
  SWIGLU_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
  SWIGLU_ERR_ARG = 6,         /* any other invalid argument (e.g. clamp limit)  */
  SWIGLU_ERR_UNSUPPORTED = 7, /* valid request the library does not implement   */
  SWIGLU_ERR_HIP = 8,         /* a HIP launch failed; see swiglu_last_hip_error */
  SWIGLU_ERR_SCRATCH = 9      /* needs more scratch than swiglu_bwd_noalloc's
                                 static buffer (SWIGLU_NOALLOC_SCRATCH_BYTES)  */
};

/* Element type of x, Wg, Wu, dh and of every output of a call.  Accumulation
 * is always fp32.  SWIGLU_F32 is true IEEE fp32 on the fp32 matrix cores (no
 * reduced-precision operand truncation): "[RFC] Testing Methodology for FP32
 * Convergence Tests on Fused SwiGLU/dSwiGLU Kernels" (Liger-Kernel issue
 * 1383), section Root Cause, traces fp32 convergence failures to TF32. */
enum swiglu_dtype { SWIGLU_F32 = 0, SWIGLU_BF16 = 1 };

/* Forward of the fused gate/up stage: the dual GEMM g = x Wg^T, u = x Wu^T
 * with the SiLU-gate epilogue applied to the fp32 accumulators and one
 * rounding of h to `dtype`; g and u are never written to memory.
 * Sources: Liger-Kernel issue 1383, Background (gate/up GEMM + SwiGLU fused
 * in one kernel to cut intermediate-tensor traffic); "Another MLP
 * implementation along with multiplier support" (Liger-Kernel issue 937),
 * TL;DR approach 3 (dual GEMM with activation); TensorRT-LLM PR 17693,
 * follow-up commit on numerics (activation on the fp32 accumulator).
 *
 *   x  [M, K], wg [N, K], wu [N, K]  (inputs, dtype)
 *   h  [M, N]                        (output, dtype)
 * Layout rule: K % 8 == 0 for bf16 and K % 4 == 0 for fp32 (16-byte rows),
 * and K <= 2^22 - 64 for both (the kernels address an operand tile of 512
 * bytes per unit of row stride with 32-bit offsets; else
 * SWIGLU_ERR_UNSUPPORTED).  K == 0 gives h = 0. */
int swiglu_fwd(int dtype, int64_t M, int64_t N, int64_t K,
               const void* x, const void* wg, const void* wu, void* h,
               void* stream);

/* Gate activations of the gated forward. */
enum swiglu_act {
  SWIGLU_ACT_SILU = 0,       /* SwiGLU: SiLU(z) = z * sigmoid(z)                    */
  SWIGLU_ACT_GELU_TANH = 1   /* GeGLU: z / 2 * (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))) */
};

/* The gated forward with a choice of gate activation:
 *   h = act(x Wg^T) * (x Wu^T)
 * act = SWIGLU_ACT_SILU is swiglu_fwd; SWIGLU_ACT_GELU_TANH is the GeGLU
 * variant ("Another MLP implementation along with multiplier support",
 * Liger-Kernel issue 937, feature pitch: the MLP modules fuse swiglu and
 * geglu; "VisualGen MLP: cublasLt GELU-tanh epilogue for the unquantized
 * bf16 path", TensorRT-LLM PR 17693: the tanh-approximated GELU applied to
 * the fp32 accumulator).  Arguments, layouts and errors as swiglu_fwd; an
 * unknown act gives SWIGLU_ERR_ARG. */
int swiglu_fwd_act(int act, int dtype, int64_t M, int64_t N, int64_t K,
                   const void* x, const void* wg, const void* wu, void* h,
                   void* stream);

/* The gated forward with scalar multipliers on the two projections
 * ("Another MLP implementation along with multiplier support", Liger-Kernel
 * issue 937: the dual GEMM with activation takes a gate multiplier, and the
 * Falcon-H1 MLP has gate and up multipliers):
 *   h = act(gate_mult * (x Wg^T)) * (up_mult * (x Wu^T))
 * The pages do not place the multipliers; this form scales each projection's
 * fp32 accumulator before the activation and the product, which is the same
 * as scaling Wg and Wu and, for up_mult, as a multiplier after the
 * activation.  Multipliers of 1 give swiglu_fwd_act exactly.  Non-finite
 * multipliers: SWIGLU_ERR_ARG; the rest as swiglu_fwd_act. */
int swiglu_fwd_mult(int act, int dtype, int64_t M, int64_t N, int64_t K,
                    const void* x, const void* wg, const void* wu,
                    float gate_mult, float up_mult, void* h, void* stream);

/* Bytes of device workspace swiglu_bwd needs for these sizes: 0 for sizes
 * swiglu_bwd rejects (invalid, or past its limits), so the result never
 * wraps.  It holds [dg | du], its transpose, x^T and the transposed weight
 * pair. */
size_t swiglu_bwd_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K);

/* Backward of the fused stage ("Fused SwiGLU/dSwiGLU", Liger-Kernel issue
 * 1383, Background: the full forward and backward dataflow).  With
 * s = sigmoid(g) and g, u recomputed from x, Wg, Wu:
 *   du = dh * g * s,   dg = dh * u * s * (1 + g * (1 - s))
 *   dx = dg Wg + du Wu,   dwg = dg^T x,   dwu = du^T x
 * dg and du are rounded to `dtype` once (they are matrix-core operands);
 * every contraction accumulates in fp32 and rounds its output once.
 * Kernels run in order on `stream`: the recompute dual GEMM with the
 * dSwiGLU epilogue (bf16: it also writes [dg | du] transposed; fp32 uses a
 * transpose kernel), transposes of x and the weights, the dX GEMM and the
 * stacked dW GEMM.
 *
 *   x [M, K], wg/wu [N, K], dh [M, N]         (inputs, dtype)
 *   dx [M, K], dwg [N, K], dwu [N, K]         (outputs, dtype; overwritten)
 *   workspace: device buffer of at least swiglu_bwd_workspace_bytes(...)
 *              bytes, 256-byte aligned; contents are scratch.
 * Layout rule: K % 8 == 0 for bf16, K % 4 == 0 for fp32; M and N are free
 * (padded operands are zero-filled).  K, 2 * Np and round_up(M, 8) must be
 * at most 2^22 - 64, with Np = round_up(N, 64) for bf16 and round_up(N, 8)
 * for fp32 (32-bit tile offsets, as for swiglu_fwd; else
 * SWIGLU_ERR_UNSUPPORTED). */
int swiglu_bwd(int dtype, int64_t M, int64_t N, int64_t K,
               const void* x, const void* wg, const void* wu, const void* dh,
               void* dx, void* dwg, void* dwu,
               void* workspace, size_t workspace_bytes, void* stream);

/* Backward of swiglu_fwd_mult with act = SiLU: with G = gate_mult * g,
 * U = up_mult * u and S = sigmoid(G),
 *   dg = gate_mult * dh * U * S * (1 + G * (1 - S)),   du = up_mult * dh * G * S,
 * then dx, dwg, dwu from dg, du as in swiglu_bwd (same workspace, layouts
 * and errors; non-finite multipliers: SWIGLU_ERR_ARG).  Multipliers of 1
 * give swiglu_bwd exactly. */
int swiglu_bwd_mult(int dtype, int64_t M, int64_t N, int64_t K,
                    const void* x, const void* wg, const void* wu, const void* dh,
                    float gate_mult, float up_mult,
                    void* dx, void* dwg, void* dwu,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Backward of swiglu_fwd_mult with either gate activation: act = SiLU is
 * swiglu_bwd_mult; act = SWIGLU_ACT_GELU_TANH (GeGLU) uses, with
 * t = 2 sqrt(2/pi) (G + 0.044715 G^3) and S = sigmoid(t),
 *   GELU(G) = G S,   GELU'(G) = S + G S (1 - S) * 2 sqrt(2/pi) (1 + 3 * 0.044715 G^2),
 *   dg = gate_mult * dh * U * GELU'(G),   du = up_mult * dh * GELU(G)
 * (product and chain rule on the forward of swiglu_fwd_act).  Workspace,
 * layouts and errors as swiglu_bwd; unknown act: SWIGLU_ERR_ARG. */
int swiglu_bwd_act_mult(int act, int dtype, int64_t M, int64_t N, int64_t K,
                        const void* x, const void* wg, const void* wu, const void* dh,
                        float gate_mult, float up_mult,
                        void* dx, void* dwg, void* dwu,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Size of swiglu_bwd_noalloc's scratch buffer: 128 MiB of device memory on
 * every GPU the library runs on, held until the process ends. */
#define SWIGLU_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* swiglu_bwd_act_mult without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid allocation.  The backward's scratch
 * (the [dg | du] tile, its transpose, x^T and [Wg; Wu]^T) lives in a static
 * device array of SWIGLU_NOALLOC_SCRATCH_BYTES inside the library; the call
 * allocates nothing (no hipMalloc, no library allocator) and the caller still
 * passes every input and output.  Results are bit-identical to
 * swiglu_bwd_act_mult.
 * Limits and sharing:
 *   - a problem whose swiglu_bwd_workspace_bytes(dtype, M, N, K) exceeds
 *     SWIGLU_NOALLOC_SCRATCH_BYTES returns SWIGLU_ERR_SCRATCH (nothing is
 *     enqueued);
 *   - every call on one GPU uses that GPU's one buffer, and the buffer keeps
 *     whatever the last call left in it (nothing in it needs to start at
 *     zero: every call writes each scratch element it reads).  Calls whose
 *     work overlaps on one GPU (concurrent streams, or threads without an
 *     ordering between their streams) race on the buffer and give wrong
 *     results; order them on one stream or use swiglu_bwd_act_mult with
 *     separate workspaces.
 * Arguments, layouts and the other errors as swiglu_bwd_act_mult. */
int swiglu_bwd_noalloc(int act, int dtype, int64_t M, int64_t N, int64_t K,
                       const void* x, const void* wg, const void* wu, const void* dh,
                       float gate_mult, float up_mult,
                       void* dx, void* dwg, void* dwu, void* stream);

/* Decode forward for 1 <= M <= 8 tokens, bf16 only: the same h as
 * swiglu_fwd, computed by a weight-streaming kernel that reads each row of
 * Wg and Wu from HBM once for all M tokens ("Fused SwiGLU benchmark",
 * AstrAI docs/developer/swiglu_benchmark.md, sections L20 findings and HBM
 * re-measurement: a fused BF16 SwiGLU primitive for M = 1, 2, 4, 8 bound by
 * the cold weight read).  M <= 3 reduces on the vector units, M >= 4 on the
 * matrix cores; fp32 accumulation in a fixed order either way, so results
 * are deterministic.
 *
 *   x [M, K], wg/wu [N, K] (bf16 inputs), h [M, N] (bf16 output)
 * Layout rule: K % 8 == 0; no other limit on K. */
int swiglu_gemv_fwd(int64_t M, int64_t N, int64_t K,
                    const void* x, const void* wg, const void* wu, void* h,
                    void* stream);

/* swiglu_gemv_fwd with a choice of gate activation (see swiglu_fwd_act). */
int swiglu_gemv_fwd_act(int act, int64_t M, int64_t N, int64_t K,
                        const void* x, const void* wg, const void* wu, void* h,
                        void* stream);

/* swiglu_gemv_fwd with an activation choice and the projection multipliers
 * of swiglu_fwd_mult. */
int swiglu_gemv_fwd_mult(int act, int64_t M, int64_t N, int64_t K,
                         const void* x, const void* wg, const void* wu,
                         float gate_mult, float up_mult, void* h, void* stream);

/* Gated forward with the FP8 block quantisation fused into the dual GEMM's
 * epilogue, so h leaves the kernel as the down projection's FP8 operand
 * (the quantisation of swiglu_act_quant below applied to the h of
 * swiglu_fwd_act; "quant: add SwiGLU forward/backward VMI kernels",
 * TileKernels-PTO PR 20, implementation notes, for the 1x32 UE8M0 / E4M3
 * format):
 *   h = act(x Wg^T) * (x Wu^T), fp32 accumulation; act(g) to a few fp32
 *       ulps, then the fp32 product;
 *   per row and 1x32 block of N: amax, E, scale byte and E4M3FN codes
 *   exactly as in swiglu_act_quant (no clamp).
 *
 *   act        SWIGLU_ACT_SILU or SWIGLU_ACT_GELU_TANH
 *   x, wg, wu  bf16 [M, K], [N, K], [N, K] (16-byte aligned)
 *   q          [M, N] uint8 E4M3FN codes (output, 16-byte aligned)
 *   scale      [M, N / 32] uint8 UE8M0 bytes (output)
 *   h_out      NULL, or [M, N] fp32 receiving the h that was quantised
 * Layout rules: bf16 only, K % 8 == 0, N % 32 == 0, K <= 2^22 - 64.
 * Returns SWIGLU_ERR_SHAPE / _ALIGN / _NULL / _UNSUPPORTED as swiglu_fwd. */
int swiglu_fwd_fp8(int act, int64_t M, int64_t N, int64_t K,
                   const void* x, const void* wg, const void* wu,
                   uint8_t* q, uint8_t* scale, float* h_out, void* stream);

/* Elementwise gated activation without quantisation (the fp32 and bf16
 * output formats of the forward table in "quant: add SwiGLU forward/backward
 * VMI kernels", TileKernels-PTO PR 20, performance section):
 *   g' = clamp(gate, -L, L), u' = clamp(up, -L, L)   (NaN passes through)
 *   h  = act(g') * u', formed in fp64 and rounded once to out_dtype
 *
 *   act          SWIGLU_ACT_SILU or SWIGLU_ACT_GELU_TANH
 *   out_dtype    SWIGLU_F32 or SWIGLU_BF16 (the type of h)
 *   gate, up     [rows, cols] fp32 inputs
 *   clamp_limit  L > 0, or +INFINITY for no clamp (NaN or L <= 0: error)
 *   h            [rows, cols] output
 *   clamp_count  NULL, or one uint64 (8-byte aligned) overwritten with the
 *                number of gate and up values with |v| > L (NaN not counted);
 *                counted as in swiglu_act_quant
 * Layout rule: cols % 8 == 0.  Unknown act: SWIGLU_ERR_ARG; unknown
 * out_dtype: SWIGLU_ERR_DTYPE. */
int swiglu_act_fwd(int act, int out_dtype, int64_t rows, int64_t cols,
                   const float* gate, const float* up, float clamp_limit,
                   void* h, uint64_t* clamp_count, void* stream);

/* Elementwise SwiGLU with FP8 block quantisation, one pass ("quant: add
 * SwiGLU forward/backward VMI kernels", TileKernels-PTO PR 20, sections
 * overview and implementation notes):
 *   g' = clamp(gate, -L, L), u' = clamp(up, -L, L)   (NaN passes through)
 *   h  = SiLU(g') * u'                               (fp32)
 *   per row and 1x32 block along cols: amax = max |h| ignoring NaN,
 *   E = smallest integer with amax <= 448 * 2^E, clamped to [-127, 127]
 *       (E = 128 when amax is +inf), scale byte = E + 127 (UE8M0),
 *   q = E4M3FN(h * 2^-E), round to nearest even, no saturation,
 *       NaN and +-inf -> NaN.
 *
 *   gate, up     [rows, cols] fp32 inputs
 *   clamp_limit  L > 0, or +INFINITY for no clamp (NaN or L <= 0: error)
 *   q            [rows, cols] uint8 E4M3FN codes (output)
 *   scale        [rows, cols / 32] uint8 UE8M0 bytes (output)
 *   clamp_count  NULL, or one uint64 overwritten with the number of gate and
 *                up values with |v| > L (NaN not counted).  With the clamp on,
 *                each workgroup's count goes to a slot of a library-owned
 *                device array and a second launch sums the slots into
 *                *clamp_count.  Counting calls take the array's 16 regions
 *                in turn, so at most 16 counting calls of this function
 *                and swiglu_act_fwd may be in flight on one GPU at once.
 *   h_out        NULL, or [rows, cols] fp32 that also receives h itself (the
 *                page's kernel likewise keeps a non-quantised output mode)
 * Layout rule: cols % 32 == 0 (the 1x32 blocks tile each row). */
int swiglu_act_quant(int64_t rows, int64_t cols,
                     const float* gate, const float* up, float clamp_limit,
                     uint8_t* q, uint8_t* scale, uint64_t* clamp_count,
                     float* h_out, void* stream);

/* swiglu_act_quant with a choice of gate activation: SWIGLU_ACT_SILU, or
 * SWIGLU_ACT_GELU_TANH for h = GELU_tanh(g') * u' (the GeGLU variant; see
 * swiglu_fwd_act).  Either way h is formed from the fp32 inputs and rounded
 * to fp32 once before the quantisation; unknown act: SWIGLU_ERR_ARG. */
int swiglu_act_quant_act(int act, int64_t rows, int64_t cols,
                         const float* gate, const float* up, float clamp_limit,
                         uint8_t* q, uint8_t* scale, uint64_t* clamp_count,
                         float* h_out, void* stream);

/* Elementwise SwiGLU backward on materialised gate/up ("quant: add SwiGLU
 * forward/backward VMI kernels", TileKernels-PTO PR 20: the performance
 * section's backward table -- gate/up given, optional clamp, optional routing
 * weights with recompute -- and the implementation notes on weight_grad, a
 * reassociated per-row reduction).  For the forward
 *   y[r, c] = w[r] * SiLU(g') * u',   g' = clamp(gate, -L, L), u' = clamp(up, -L, L)
 * (w = 1 when weights is NULL; NaN passes the clamp), given dy:
 *   dgate = w dy u' s (1 + g' (1 - s)), s = sigmoid(g'), where |gate| <= L
 *           (or NaN), 0 where the clamp acted;
 *   dup   = w dy SiLU(g') where |up| <= L (or NaN), 0 where the clamp acted;
 *   weight_grad[r] = sum_c dy[r, c] * SiLU(g') * u'   (dL/dw[r]).
 *
 *   gate, up, dy   [rows, cols] fp32 inputs
 *   weights        NULL, or [rows] fp32
 *   clamp_limit    L > 0, or +INFINITY for no clamp (NaN or L <= 0: error)
 *   dgate, dup     [rows, cols] fp32 outputs
 *   weight_grad    NULL, or [rows] fp32 output
 * Products and the row sum are formed in fp64, each output rounded once.
 * Layout rule: cols % 4 == 0 (16-byte rows). */
int swiglu_act_bwd(int64_t rows, int64_t cols,
                   const float* gate, const float* up, const float* dy,
                   const float* weights, float clamp_limit,
                   float* dgate, float* dup, float* weight_grad, void* stream);

/* swiglu_act_bwd with a choice of tensor format (the backward table's fmt
 * column, read as the type of gate, up, dy, dgate and dup): SWIGLU_F32, or
 * SWIGLU_BF16 with bf16 tensors, fp32 arithmetic as above and each output
 * rounded once (to nearest even) to bf16.  weights and weight_grad stay
 * fp32.  Layout rule: rows are whole 16-byte chunks (cols % 4 == 0 for fp32,
 * cols % 8 == 0 for bf16); unknown dtype: SWIGLU_ERR_DTYPE. */
int swiglu_act_bwd_dt(int dtype, int64_t rows, int64_t cols,
                      const void* gate, const void* up, const void* dy,
                      const float* weights, float clamp_limit,
                      void* dgate, void* dup, float* weight_grad, void* stream);

/* swiglu_act_bwd_dt with dgate and dup in E4M3 (the backward table's fmt
 * e4m3, read as the format of dgate and dup, as fmt is the format of h in the
 * forward table; the implementation notes' FP8 output cast without
 * saturation, keeping NaN).  Each output leaves as the quantiser's 1x32
 * blocks: its exact value is rounded once to fp32, the block's amax (NaN
 * ignored) gives the smallest E with amax <= 448 * 2^E (byte E + 127, 0xFF
 * when amax is infinite), and each value is coded as E4M3FN(v * 2^-E), ties
 * to even, NaN and infinities as NaN.
 *
 *   gate, up, dy        [rows, cols] inputs of `dtype` (SWIGLU_F32 or SWIGLU_BF16)
 *   weights, weight_grad as swiglu_act_bwd (fp32, NULL allowed)
 *   q_dgate, q_dup      [rows, cols] uint8 E4M3FN codes (16-byte aligned)
 *   scale_dgate, scale_dup  [rows, cols / 32] uint8 UE8M0 bytes
 * Layout rule: cols % 32 == 0 (whole blocks), else SWIGLU_ERR_SHAPE. */
int swiglu_act_bwd_fp8(int dtype, int64_t rows, int64_t cols,
                       const void* gate, const void* up, const void* dy,
                       const float* weights, float clamp_limit,
                       uint8_t* q_dgate, uint8_t* scale_dgate, uint8_t* q_dup, uint8_t* scale_dup,
                       float* weight_grad, void* stream);

/* Measurement aid: the decode kernel's read-only twin.  The same launch as
 * swiglu_gemv_fwd for (M, N, K) -- the same kernel's grid, LDS footprint,
 * x loads and weight loads (and, for M >= 4, the weights' trip through LDS),
 * in the same order and unrolling -- with no arithmetic: sink[n] receives
 * the XOR of every 32-bit word of Wg[n, :] and Wu[n, :], for sink [N].  Its time is the floor of the decode kernel's access pattern
 * on the same buffers ("Fused SwiGLU benchmark", section HBM
 * re-measurement: the fused kernel against a pure-read loop over the same
 * rotated weights).  Arguments and errors as swiglu_gemv_fwd (sink in place
 * of h, 4-byte aligned). */
int swiglu_probe_gemv_read(int64_t M, int64_t N, int64_t K,
                           const void* x, const void* wg, const void* wu, uint32_t* sink,
                           void* stream);

/* Measurement aid: the quantiser's twin.  The launch of swiglu_act_quant
 * without clamp, count or h_out -- grid, loads of gate and up, stores of q
 * and scale, in the same mapping -- with no arithmetic: the stored bytes are
 * folds of the loaded words.  Its time is the floor of the quantiser's byte
 * pattern (8 bytes read, 1 + 1/32 written per element) on the same buffers.
 * Arguments, layouts and errors as swiglu_act_quant. */
int swiglu_probe_act_quant_stream(int64_t rows, int64_t cols, const float* gate, const float* up,
                                  uint8_t* q, uint8_t* scale, void* stream);

/* Test aid for the FP8 encoders shared by every quantising path: scans the
 * fp32 bit patterns first..last (inclusive) and appends to `out` the pair
 * (p, result) for p = first and for each pattern p > first whose result
 * differs from that of p - 1, incrementing *count once per pair (the caller
 * zeroes *count; `out` holds 2 * capacity uint32, at most `capacity` pairs
 * are stored, in no particular order).  kind 0: the E4M3FN code of
 * the value at scale 1 (nearest, ties to even, NOSAT, NaN kept); kind 1: the
 * UE8M0 scale byte of the value taken as a block amax.  Over patterns of one
 * sign the value is monotone in the pattern, so the returned list is the
 * whole function, which a test compares with an independent encoder over
 * all 2^32 patterns.  Errors: kind not 0 or 1 (SWIGLU_ERR_ARG), last < first
 * (SWIGLU_ERR_SHAPE), NULL or misaligned out / count. */
int swiglu_probe_fp8_transitions(int kind, uint32_t first, uint32_t last, uint32_t* out, uint32_t capacity,
                                 uint32_t* count, void* stream);

/* Measurement aid: a pure streaming read of two device buffers of `bytes`
 * bytes each (16-byte multiples), the cold-read floor against which the
 * decode kernel is measured ("Fused SwiGLU benchmark", section HBM
 * re-measurement: the fused kernel is compared with a dual-stream pure-read
 * loop over rotated weight copies).  Writes one word per workgroup to `sink`
 * (>= 4096 uint32 words) so the reads cannot be elided. */
int swiglu_probe_read2(const void* a, const void* b, size_t bytes,
                       uint32_t* sink, void* stream);

/* Measurement aid: the same dual-stream read with a chosen launch shape,
 * so that the floor can be the fastest of several: `threads` per workgroup
 * (256 or 512), `chunks` 16-byte chunks of each buffer in flight per lane
 * (1, 2, 4 or 8), a grid of at most `max_blocks` workgroups (1..65535;
 * grid-stride beyond).  `sink` (>= 4096 uint32 words) receives a word only
 * when a lane's fold of its loaded words equals 0x9E3779B9; it exists so
 * that the loads cannot be elided.  Other arguments and errors as
 * swiglu_probe_read2; an unsupported shape is SWIGLU_ERR_ARG. */
int swiglu_probe_read2_cfg(const void* a, const void* b, size_t bytes, int threads, int chunks, int max_blocks,
                           uint32_t* sink, void* stream);

/* Measurement aid: the dense bf16 matrix-core rate the chip sustains.
 * `blocks` workgroups of 8 waves each run `iters` iterations of eight
 * independent v_mfma_f32_16x16x32_bf16 (the form the bf16 forward uses) on
 * register operands (no memory traffic): 2 * 16 * 16 * 32 * 8 * 8 * iters *
 * blocks flop per call.  The
 * roofline peak of the bf16 kernels is the published one; this gives the
 * ceiling the chip reaches under its power and clock limits beside it.
 * `sink` receives one float per workgroup (>= blocks floats). */
int swiglu_probe_mfma(int iters, int blocks, float* sink, void* stream);

/* Human-readable name of a status code (static string). */
const char* swiglu_status_str(int status);

/* hipError_t of the last SWIGLU_ERR_HIP returned on this thread (0 if none). */
int swiglu_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int swiglu_version(void);

/* Hash of the sources and compiler flags this library was built from (16
 * hex digits, static string), so a caller can tell a stale build from a
 * current one. */
const char* swiglu_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H_ */
