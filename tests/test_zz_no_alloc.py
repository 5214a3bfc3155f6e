"""The allocation-free backward (swiglu_bwd_noalloc) against swiglu_bwd_act_mult.

Both are called through the C ABI with the same inputs; the allocation-free
entry point must give the same bits.  Two calls follow each other on one
GPU, the second with a smaller problem, so the second runs on a scratch
buffer that still holds the first call's values (nothing in it may be
assumed to start at zero).  Outputs sit in guarded buffers.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from parity_util import check_guards, guarded

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import swiglu_mlp_fwd_amd as S  # noqa: E402
from swiglu_mlp_fwd_amd import _lib  # noqa: E402

DEV = torch.device("cuda:0")


def _inputs(dt, M, N, K, seed):
    if dt == "bf16":
        d = synth.train_bf16(M, N, K, seed=seed)
        return {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(DEV) for k, v in d.items()}
    d = synth.gemm_fp32(M, N, K, seed=seed)
    d["dh"] = synth.normal_f32((M, N), 1.0, seed, synth.STREAM_DH)
    return {k: torch.from_numpy(v).to(DEV) for k, v in d.items()}


def _both(dt, M, N, K, seed, act, mult):
    """Returns the bf16/fp32 bit patterns of (dx, dwg, dwu) from both entry points."""
    t = _inputs(dt, M, N, K, seed)
    tdt = t["x"].dtype
    code = _lib.SWIGLU_BF16 if dt == "bf16" else _lib.SWIGLU_F32
    L = S.lib()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    p = {k: v.data_ptr() for k, v in t.items()}
    a_code = _lib.SWIGLU_ACT_SILU if act == "silu" else _lib.SWIGLU_ACT_GELU_TANH
    ref = [guarded((M, K), tdt), guarded((N, K), tdt), guarded((N, K), tdt)]
    need = L.swiglu_bwd_workspace_bytes(code, M, N, K)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    st = L.swiglu_bwd_act_mult(a_code, code, M, N, K, p["x"], p["wg"], p["wu"], p["dh"], mult[0], mult[1],
                               ref[0].t.data_ptr(), ref[1].t.data_ptr(), ref[2].t.data_ptr(), ws.data_ptr(),
                               need, stream)
    assert st == 0, L.swiglu_status_str(st)
    got = [guarded((M, K), tdt), guarded((N, K), tdt), guarded((N, K), tdt)]
    st = L.swiglu_bwd_noalloc(a_code, code, M, N, K, p["x"], p["wg"], p["wu"], p["dh"], mult[0], mult[1],
                              got[0].t.data_ptr(), got[1].t.data_ptr(), got[2].t.data_ptr(), stream)
    assert st == 0, L.swiglu_status_str(st)
    torch.cuda.synchronize()
    check_guards(f"noalloc {dt} {M}x{N}x{K}", *ref, *got)
    ib = torch.int16 if dt == "bf16" else torch.int32
    return [g.t.view(ib).cpu() for g in ref], [g.t.view(ib).cpu() for g in got]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_backward_on_two_calls(dt):
    # first call larger, second smaller: the second reads a scratch buffer
    # full of the first call's values
    for (M, N, K), seed, act, mult in (((300, 520, 264), 31, "silu", (1.0, 1.0)),
                                       ((129, 127, 72), 32, "gelu_tanh", (0.7, 1.3))):
        ref, got = _both(dt, M, N, K, seed, act, mult)
        for name, a, b in zip(("dx", "dwg", "dwu"), ref, got):
            assert torch.equal(a, b), f"noalloc {dt} {M}x{N}x{K} {name} differs from swiglu_bwd_act_mult"
        print(f"noalloc {dt} {M}x{N}x{K} {act}: bit-identical", flush=True)


def test_noalloc_rejects_problems_beyond_the_scratch():
    L = S.lib()
    A = 0x10000
    M, N, K = 4096, 8192, 4096
    need = L.swiglu_bwd_workspace_bytes(_lib.SWIGLU_BF16, M, N, K)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    st = L.swiglu_bwd_noalloc(0, _lib.SWIGLU_BF16, M, N, K, A, A, A, A, 1.0, 1.0, A, A, A, None)
    assert st == _lib.SWIGLU_ERR_SCRATCH
    assert b"scratch" in L.swiglu_status_str(st)
    assert ctypes.c_int(st).value == 9
