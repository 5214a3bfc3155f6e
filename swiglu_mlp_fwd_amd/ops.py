"""PyTorch-facing wrappers of libswiglu.

Argument marshalling only: shapes, dtypes and devices of inputs and of any
caller-supplied output are checked before the library is called (the C ABI
sees raw pointers, so a wrong shape would be read or written past its
tensor), inputs are made contiguous, outputs are allocated with torch.empty
on the input's device, and the library is called on the current HIP stream.
Every step of the computation runs in the HIP kernels behind the C ABI.

Inputs of rank >= 3 are viewed as [M, K] and the output restored to the
leading shape ("VisualGen MLP: cublasLt GELU-tanh epilogue for the
unquantized bf16 path", TensorRT-LLM PR 17693, section Change: rank >= 3
inputs are flattened to [M, in] and restored afterward).
"""
from __future__ import annotations

import math

import torch

from ._lib import SWIGLU_ACT_GELU_TANH, SWIGLU_ACT_SILU, SWIGLU_BF16, SWIGLU_F32, check, lib

_DT = {torch.bfloat16: SWIGLU_BF16, torch.float32: SWIGLU_F32}
_ACT = {"silu": SWIGLU_ACT_SILU, "gelu_tanh": SWIGLU_ACT_GELU_TANH}


def _act_code(act: str) -> int:
    try:
        return _ACT[act]
    except KeyError:
        raise ValueError(f"act must be one of {sorted(_ACT)}, got {act!r}") from None


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"libswiglu supports bfloat16 and float32, got {t.dtype}") from None


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _same(*ts):
    """Inputs of one call share dtype and device."""
    d, dev = ts[0].dtype, ts[0].device
    for t in ts[1:]:
        if t.dtype != d:
            raise TypeError(f"dtype mismatch: {t.dtype} vs {d}")
        if t.device != dev:
            raise ValueError(f"device mismatch: {t.device} vs {dev}")


def _on_gpu(t: torch.Tensor) -> None:
    """Checked after every shape check, so a malformed call fails the same way
    with or without a GPU; the library itself only ever sees device pointers."""
    if t.device.type != "cuda":
        raise ValueError("libswiglu operates on GPU tensors only")


def _weights(wg: torch.Tensor, wu: torch.Tensor, K: int) -> int:
    """N of Wg, Wu [N, K] (the nn.Linear layout)."""
    if wg.dim() != 2:
        raise ValueError(f"Wg must be [N, K], got {tuple(wg.shape)}")
    N = wg.shape[0]
    if tuple(wg.shape) != (N, K) or tuple(wu.shape) != (N, K):
        raise ValueError(f"weights must be [N, K] = [{N}, {K}], got {tuple(wg.shape)}, {tuple(wu.shape)}")
    return N


def _check_out(t: torch.Tensor | None, name: str, shape, dtype: torch.dtype, device: torch.device) -> None:
    """A caller-supplied output: the kernels write exactly `shape` elements of
    `dtype` through its data pointer, so anything else would be written past
    or beside the tensor."""
    if t is None:
        raise ValueError(f"{name}: an output tensor is required here")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _p(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def fwd(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, out: torch.Tensor | None = None,
        act: str = "silu", gate_mult: float = 1.0, up_mult: float = 1.0) -> torch.Tensor:
    """h = act(gate_mult * x Wg^T) * (up_mult * x Wu^T), act "silu" (SwiGLU) or
    "gelu_tanh" (GeGLU).  x [..., K], Wg/Wu [N, K] -> h [..., N]."""
    _same(x, wg, wu)
    _dtype_code(x)
    lead, K = x.shape[:-1], x.shape[-1]
    N = _weights(wg, wu, K)
    M = math.prod(lead)
    if out is not None:
        _check_out(out, "out", (M, N), x.dtype, x.device)
    _on_gpu(x)
    x2 = x.reshape(M, K).contiguous()
    wg, wu = wg.contiguous(), wu.contiguous()
    h = out if out is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
    check("swiglu_fwd_mult", lib().swiglu_fwd_mult(_act_code(act), _dtype_code(x), M, N, K, _p(x2), _p(wg), _p(wu),
                                                   float(gate_mult), float(up_mult), _p(h), _stream(x)))
    return h.reshape(*lead, N)


def fwd_fp8(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, act: str = "silu", h_out: bool = False,
            out=None):
    """Gated forward with h quantised in the GEMM epilogue (bf16 inputs).

    Returns (q uint8 [M, N] E4M3FN codes, scale uint8 [M, N/32] UE8M0 bytes,
    h fp32 [M, N] or None); `out` may pass preallocated (q, scale, h).
    """
    _same(x, wg, wu)
    if x.dtype != torch.bfloat16:
        raise TypeError("fwd_fp8 takes bf16 inputs")
    lead, K = x.shape[:-1], x.shape[-1]
    N = _weights(wg, wu, K)
    M = math.prod(lead)
    dev = x.device
    if out is not None:
        q, scale, h = out
        _check_out(q, "q", (M, N), torch.uint8, dev)
        _check_out(scale, "scale", (M, N // 32 if N % 32 == 0 else 0), torch.uint8, dev)
        if h is not None:
            _check_out(h, "h", (M, N), torch.float32, dev)
    _on_gpu(x)
    x2 = x.reshape(M, K).contiguous()
    wg, wu = wg.contiguous(), wu.contiguous()
    if out is None:
        q = torch.empty((M, N), dtype=torch.uint8, device=dev)
        scale = torch.empty((M, N // 32 if N % 32 == 0 else 0), dtype=torch.uint8, device=dev)
        h = torch.empty((M, N), dtype=torch.float32, device=dev) if h_out else None
    check("swiglu_fwd_fp8", lib().swiglu_fwd_fp8(_act_code(act), M, N, K, _p(x2), _p(wg), _p(wu), _p(q), _p(scale),
                                                 _p(h), _stream(x)))
    return q, scale, h


def bwd_workspace_bytes(dtype: torch.dtype, M: int, N: int, K: int) -> int:
    return int(lib().swiglu_bwd_workspace_bytes(_DT[dtype], M, N, K))


def bwd(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, dh: torch.Tensor,
        workspace: torch.Tensor | None = None, gate_mult: float = 1.0, up_mult: float = 1.0,
        act: str = "silu", out=None):
    """(dx, dwg, dwu) of L = sum(dh * h), h = act(gate_mult x Wg^T) * (up_mult x Wu^T).
    Shapes as in fwd; dh [..., N].  `out` may pass preallocated (dx [M, K],
    dwg [N, K], dwu [N, K]); `workspace` a uint8 device buffer of at least
    bwd_workspace_bytes(...) bytes (a smaller or missing one is replaced)."""
    _same(x, wg, wu, dh)
    dt = _dtype_code(x)
    lead, K = x.shape[:-1], x.shape[-1]
    N = _weights(wg, wu, K)
    M = math.prod(lead)
    if tuple(dh.shape) != (*lead, N):
        raise ValueError(f"dh must be {(*lead, N)}, got {tuple(dh.shape)}")
    if out is not None:
        dx, dwg, dwu = out
        _check_out(dx, "dx", (M, K), x.dtype, x.device)
        _check_out(dwg, "dwg", (N, K), x.dtype, x.device)
        _check_out(dwu, "dwu", (N, K), x.dtype, x.device)
    if workspace is not None and (workspace.device != x.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the device of x")
    _on_gpu(x)
    x2 = x.reshape(M, K).contiguous()
    dh2 = dh.reshape(M, N).contiguous()
    wg, wu = wg.contiguous(), wu.contiguous()
    need = int(lib().swiglu_bwd_workspace_bytes(dt, M, N, K))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        dx = torch.empty((M, K), dtype=x.dtype, device=x.device)
        dwg = torch.empty((N, K), dtype=x.dtype, device=x.device)
        dwu = torch.empty((N, K), dtype=x.dtype, device=x.device)
    check("swiglu_bwd_act_mult", lib().swiglu_bwd_act_mult(_act_code(act), dt, M, N, K, _p(x2), _p(wg), _p(wu),
                                                           _p(dh2), float(gate_mult), float(up_mult), _p(dx),
                                                           _p(dwg), _p(dwu), _p(workspace),
                                                           workspace.numel() * workspace.element_size(),
                                                           _stream(x)))
    return dx.reshape(*lead, K), dwg, dwu


def bwd_noalloc(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, dh: torch.Tensor, out,
                gate_mult: float = 1.0, up_mult: float = 1.0, act: str = "silu"):
    """bwd into preallocated (dx, dwg, dwu) with the library's static scratch
    instead of a workspace: the library allocates nothing.  Inputs must
    already be contiguous (no copies are made).  Calls that overlap on one
    GPU share the scratch and race; problems larger than the scratch raise
    (SWIGLU_ERR_SCRATCH)."""
    _same(x, wg, wu, dh)
    dt = _dtype_code(x)
    lead, K = x.shape[:-1], x.shape[-1]
    N = _weights(wg, wu, K)
    M = math.prod(lead)
    if tuple(dh.shape) != (*lead, N):
        raise ValueError(f"dh must be {(*lead, N)}, got {tuple(dh.shape)}")
    dx, dwg, dwu = out
    _check_out(dx, "dx", (M, K), x.dtype, x.device)
    _check_out(dwg, "dwg", (N, K), x.dtype, x.device)
    _check_out(dwu, "dwu", (N, K), x.dtype, x.device)
    for t, name in ((x, "x"), (wg, "wg"), (wu, "wu"), (dh, "dh")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _on_gpu(x)
    check("swiglu_bwd_noalloc", lib().swiglu_bwd_noalloc(_act_code(act), dt, M, N, K, _p(x), _p(wg), _p(wu), _p(dh),
                                                         float(gate_mult), float(up_mult), _p(dx), _p(dwg),
                                                         _p(dwu), _stream(x)))
    return dx, dwg, dwu


def gemv_fwd(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, out: torch.Tensor | None = None,
             act: str = "silu", gate_mult: float = 1.0, up_mult: float = 1.0) -> torch.Tensor:
    """Decode forward for M <= 8 tokens (bf16): same result as fwd."""
    _same(x, wg, wu)
    if x.dtype != torch.bfloat16:
        raise TypeError("gemv_fwd is bf16 only")
    lead, K = x.shape[:-1], x.shape[-1]
    N = _weights(wg, wu, K)
    M = math.prod(lead)
    if out is not None:
        _check_out(out, "out", (M, N), x.dtype, x.device)
    _on_gpu(x)
    x2 = x.reshape(M, K).contiguous()
    wg, wu = wg.contiguous(), wu.contiguous()
    h = out if out is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
    check("swiglu_gemv_fwd_mult", lib().swiglu_gemv_fwd_mult(_act_code(act), M, N, K, _p(x2), _p(wg), _p(wu),
                                                             float(gate_mult), float(up_mult), _p(h), _stream(x)))
    return h.reshape(*lead, N)


def act_fwd(gate: torch.Tensor, up: torch.Tensor, clamp_limit: float = math.inf, act: str = "silu",
            out_dtype: torch.dtype = torch.float32, count: bool = True, out=None):
    """Elementwise act(clamp(gate)) * clamp(up) without quantisation, fp32 in,
    fp32 or bf16 out.  Returns (h, clamp_count int64 tensor [1] or None);
    `out` may pass preallocated (h, count)."""
    _same(gate, up)
    if gate.dtype != torch.float32:
        raise TypeError("act_fwd takes fp32 gate/up")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    cols = gate.shape[-1]
    rows = math.prod(gate.shape[:-1])
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"act_fwd writes float32 or bfloat16 h, got {out_dtype}")
    if out is not None:
        h, cnt = out
        if h is None or h.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out h must be a float32 or bfloat16 tensor")
        _check_out(h, "h", (rows, cols), h.dtype, gate.device)
        if cnt is not None:
            _check_out(cnt, "count", (1,), torch.int64, gate.device)
    _on_gpu(gate)
    g2 = gate.reshape(rows, cols).contiguous()
    u2 = up.reshape(rows, cols).contiguous()
    if out is None:
        h = torch.empty((rows, cols), dtype=out_dtype, device=gate.device)
        cnt = torch.empty(1, dtype=torch.int64, device=gate.device) if count else None
    check("swiglu_act_fwd", lib().swiglu_act_fwd(_act_code(act), _DT[h.dtype], rows, cols, _p(g2), _p(u2),
                                                 float(clamp_limit), _p(h), _p(cnt), _stream(gate)))
    return h.reshape(gate.shape), cnt


def act_quant(gate: torch.Tensor, up: torch.Tensor, clamp_limit: float = math.inf,
              count: bool = True, h_out: bool = False, out=None, act: str = "silu"):
    """Elementwise SwiGLU (act "silu") or GeGLU ("gelu_tanh") + 1x32 UE8M0/E4M3
    quantisation.

    Returns (q uint8 [rows, cols], scale uint8 [rows, cols/32],
    clamp_count int64 tensor [1] or None, h fp32 or None).
    `out` may pass preallocated (q, scale, count, h) tensors.
    """
    _same(gate, up)
    if gate.dtype != torch.float32:
        raise TypeError("act_quant takes fp32 gate/up")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    cols = gate.shape[-1]
    rows = math.prod(gate.shape[:-1])
    dev = gate.device
    if out is not None:
        q, scale, cnt, h = out
        _check_out(q, "q", (rows, cols), torch.uint8, dev)
        _check_out(scale, "scale", (rows, cols // 32 if cols % 32 == 0 else 0), torch.uint8, dev)
        if cnt is not None:
            _check_out(cnt, "count", (1,), torch.int64, dev)
        if h is not None:
            _check_out(h, "h", (rows, cols), torch.float32, dev)
    _on_gpu(gate)
    g2 = gate.reshape(rows, cols).contiguous()
    u2 = up.reshape(rows, cols).contiguous()
    if out is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scale = torch.empty((rows, cols // 32 if cols % 32 == 0 else 0), dtype=torch.uint8, device=dev)
        cnt = torch.empty(1, dtype=torch.int64, device=dev) if count else None
        h = torch.empty((rows, cols), dtype=torch.float32, device=dev) if h_out else None
    check("swiglu_act_quant_act", lib().swiglu_act_quant_act(_act_code(act), rows, cols, _p(g2), _p(u2),
                                                             float(clamp_limit), _p(q), _p(scale), _p(cnt), _p(h),
                                                             _stream(gate)))
    return q, scale, cnt, h


def act_bwd(gate: torch.Tensor, up: torch.Tensor, dy: torch.Tensor, clamp_limit: float = math.inf,
            weights: torch.Tensor | None = None, weight_grad: bool = False, out=None):
    """Elementwise SwiGLU backward of y = w * SiLU(clamp(gate)) * clamp(up).

    gate, up, dy are fp32 or bf16 (dgate, dup come out in the same type);
    weights ([rows] or None) and weight_grad are fp32.
    Returns (dgate, dup, weight_grad or None); `out` may pass preallocated
    (dgate, dup, weight_grad) tensors.
    """
    _same(gate, up, dy)
    if gate.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("act_bwd takes fp32 or bf16 gate/up/dy")
    if gate.shape != up.shape or gate.shape != dy.shape:
        raise ValueError("gate, up and dy must have the same shape")
    cols = gate.shape[-1]
    rows = math.prod(gate.shape[:-1])
    if weights is not None:
        if weights.dtype != torch.float32 or weights.device != gate.device:
            raise TypeError("weights must be an fp32 tensor on the device of gate")
        if weights.numel() != rows:
            raise ValueError(f"weights must have {rows} elements")
    dev = gate.device
    if out is not None:
        dg, du, wg = out
        _check_out(dg, "dgate", (rows, cols), gate.dtype, dev)
        _check_out(du, "dup", (rows, cols), gate.dtype, dev)
        if wg is not None:
            _check_out(wg, "weight_grad", (rows,), torch.float32, dev)
    _on_gpu(gate)
    g2 = gate.reshape(rows, cols).contiguous()
    u2 = up.reshape(rows, cols).contiguous()
    d2 = dy.reshape(rows, cols).contiguous()
    w = None if weights is None else weights.reshape(rows).contiguous()
    if out is None:
        dg = torch.empty((rows, cols), dtype=gate.dtype, device=dev)
        du = torch.empty((rows, cols), dtype=gate.dtype, device=dev)
        wg = torch.empty(rows, dtype=torch.float32, device=dev) if weight_grad else None
    check("swiglu_act_bwd_dt", lib().swiglu_act_bwd_dt(_dtype_code(gate), rows, cols, _p(g2), _p(u2), _p(d2), _p(w),
                                                       float(clamp_limit), _p(dg), _p(du), _p(wg), _stream(gate)))
    return dg.reshape(gate.shape), du.reshape(gate.shape), wg


def act_bwd_fp8(gate: torch.Tensor, up: torch.Tensor, dy: torch.Tensor, clamp_limit: float = math.inf,
                weights: torch.Tensor | None = None, weight_grad: bool = False, out=None):
    """act_bwd with dgate and dup quantised per 1x32 block (E4M3FN codes, UE8M0
    scales).  gate, up, dy are fp32 or bf16; weights and weight_grad fp32.
    Returns (q_dgate, scale_dgate, q_dup, scale_dup, weight_grad or None);
    `out` may pass those five preallocated (weight_grad may be None)."""
    _same(gate, up, dy)
    if gate.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("act_bwd_fp8 takes fp32 or bf16 gate/up/dy")
    if gate.shape != up.shape or gate.shape != dy.shape:
        raise ValueError("gate, up and dy must have the same shape")
    cols = gate.shape[-1]
    rows = math.prod(gate.shape[:-1])
    if weights is not None:
        if weights.dtype != torch.float32 or weights.device != gate.device:
            raise TypeError("weights must be an fp32 tensor on the device of gate")
        if weights.numel() != rows:
            raise ValueError(f"weights must have {rows} elements")
    dev = gate.device
    nb = cols // 32 if cols % 32 == 0 else 0
    if out is not None:
        qg, sg, qu, su, wg = out
        _check_out(qg, "q_dgate", (rows, cols), torch.uint8, dev)
        _check_out(sg, "scale_dgate", (rows, nb), torch.uint8, dev)
        _check_out(qu, "q_dup", (rows, cols), torch.uint8, dev)
        _check_out(su, "scale_dup", (rows, nb), torch.uint8, dev)
        if wg is not None:
            _check_out(wg, "weight_grad", (rows,), torch.float32, dev)
    _on_gpu(gate)
    g2 = gate.reshape(rows, cols).contiguous()
    u2 = up.reshape(rows, cols).contiguous()
    d2 = dy.reshape(rows, cols).contiguous()
    w = None if weights is None else weights.reshape(rows).contiguous()
    if out is None:
        qg = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        qu = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        sg = torch.empty((rows, nb), dtype=torch.uint8, device=dev)
        su = torch.empty((rows, nb), dtype=torch.uint8, device=dev)
        wg = torch.empty(rows, dtype=torch.float32, device=dev) if weight_grad else None
    check("swiglu_act_bwd_fp8", lib().swiglu_act_bwd_fp8(_dtype_code(gate), rows, cols, _p(g2), _p(u2), _p(d2), _p(w),
                                                         float(clamp_limit), _p(qg), _p(sg), _p(qu), _p(su), _p(wg),
                                                         _stream(gate)))
    return qg, sg, qu, su, wg


def probe_mfma(iters: int, blocks: int, sink: torch.Tensor) -> int:
    """Register-only bf16 MFMA loop; returns the flops one call performs."""
    if sink.dtype != torch.float32 or sink.numel() < blocks:
        raise ValueError("sink must be an fp32 tensor of at least `blocks` elements")
    check("swiglu_probe_mfma", lib().swiglu_probe_mfma(int(iters), int(blocks), _p(sink), _stream(sink)))
    return 2 * 16 * 16 * 32 * 8 * 8 * int(iters) * int(blocks)


def probe_gemv_read(x: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor, sink: torch.Tensor) -> None:
    """The decode kernel's read-only twin on these buffers (same launch as
    gemv_fwd, no arithmetic): one int32 word per column into sink [N]."""
    _same(x, wg, wu)
    if x.dtype != torch.bfloat16:
        raise TypeError("probe_gemv_read is bf16 only")
    lead, K = x.shape[:-1], x.shape[-1]
    N = _weights(wg, wu, K)
    M = math.prod(lead)
    if sink.dtype != torch.int32 or sink.numel() < N or not sink.is_contiguous() or sink.device != x.device:
        raise ValueError(f"sink must be a contiguous int32 tensor of at least {N} elements on the device of x")
    if not (x.is_contiguous() and wg.is_contiguous() and wu.is_contiguous()):
        raise ValueError("probe_gemv_read takes contiguous tensors")
    _on_gpu(x)
    check("swiglu_probe_gemv_read", lib().swiglu_probe_gemv_read(M, N, K, _p(x), _p(wg), _p(wu), _p(sink),
                                                                 _stream(x)))


def probe_act_quant_stream(gate: torch.Tensor, up: torch.Tensor, q: torch.Tensor, scale: torch.Tensor) -> None:
    """The quantiser's twin on these buffers (its loads and stores, no
    arithmetic); q and scale receive folds of the input words."""
    _same(gate, up)
    if gate.dtype != torch.float32 or gate.shape != up.shape or gate.dim() != 2:
        raise ValueError("gate and up must be fp32 [rows, cols]")
    rows, cols = gate.shape
    _check_out(q, "q", (rows, cols), torch.uint8, gate.device)
    _check_out(scale, "scale", (rows, cols // 32 if cols % 32 == 0 else 0), torch.uint8, gate.device)
    if not (gate.is_contiguous() and up.is_contiguous()):
        raise ValueError("probe_act_quant_stream takes contiguous inputs")
    _on_gpu(gate)
    check("swiglu_probe_act_quant_stream", lib().swiglu_probe_act_quant_stream(rows, cols, _p(gate), _p(up), _p(q),
                                                                               _p(scale), _stream(gate)))


def probe_read2(a: torch.Tensor, b: torch.Tensor, sink: torch.Tensor, shape: tuple[int, int, int] | None = None) -> None:
    """Pure read of two equally sized buffers (cold-read floor measurement);
    `shape` = (threads, chunks in flight per lane, max workgroups) picks the
    launch shape of swiglu_probe_read2_cfg."""
    nbytes = a.numel() * a.element_size()
    if b.numel() * b.element_size() != nbytes:
        raise ValueError("probe buffers must have equal size")
    if sink.numel() * sink.element_size() < 4096 * 4:
        raise ValueError("sink must hold at least 4096 words")
    if shape is None:
        check("swiglu_probe_read2", lib().swiglu_probe_read2(_p(a), _p(b), nbytes, _p(sink), _stream(a)))
    else:
        t, c, m = shape
        check("swiglu_probe_read2_cfg", lib().swiglu_probe_read2_cfg(_p(a), _p(b), nbytes, int(t), int(c), int(m),
                                                                     _p(sink), _stream(a)))


class SwiGLUFunction(torch.autograd.Function):
    """Autograd wrapper: forward = fwd, backward = bwd (g and u are recomputed)."""

    @staticmethod
    def forward(ctx, x, wg, wu, gate_mult=1.0, up_mult=1.0, act="silu"):
        ctx.save_for_backward(x, wg, wu)
        ctx.cfg = (gate_mult, up_mult, act)
        return fwd(x, wg, wu, gate_mult=gate_mult, up_mult=up_mult, act=act)

    @staticmethod
    def backward(ctx, dh):
        x, wg, wu = ctx.saved_tensors
        gm, um, act = ctx.cfg
        dx, dwg, dwu = bwd(x, wg, wu, dh, gate_mult=gm, up_mult=um, act=act)
        return dx, dwg, dwu, None, None, None


def swiglu(x, wg, wu, gate_mult: float = 1.0, up_mult: float = 1.0, act: str = "silu"):
    """Differentiable fused gate/up stage, act "silu" (SwiGLU) or "gelu_tanh"
    (GeGLU); the scalar projection multipliers are constants, not trained."""
    return SwiGLUFunction.apply(x, wg, wu, gate_mult, up_mult, act)
