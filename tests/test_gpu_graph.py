"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

Every entry point enqueues kernels only on the caller's stream, allocates
nothing and never synchronizes, so a whole training step can be captured once
and replayed.  The graph is replayed several times with eager work and
synchronizations in between, and every replay must reproduce the eager
results bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import synth
from parity_util import dev_bf16, dev_f32

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import swiglu_mlp_fwd_amd as S  # noqa: E402

DEV = torch.device("cuda:0")


def test_training_step_and_quantiser_replay_in_a_graph():
    M, N, K = 520, 700, 328
    d = synth.train_bf16(M, N, K, seed=21)
    x, wg, wu, dh = (dev_bf16(d[k]) for k in ("x", "wg", "wu", "dh"))
    ws = torch.empty(S.bwd_workspace_bytes(torch.bfloat16, M, N, K), dtype=torch.uint8, device=DEV)
    a = synth.act_quant_f32(64, 512, seed=22)
    gate, up = dev_f32(a["gate"]), dev_f32(a["up"])
    dec = synth.decode_bf16(4, 264, 512, seed=23)
    xd, wgd, wud = (dev_bf16(dec[k]) for k in ("x", "wg", "wu"))

    # Outputs written in place by both the eager run and the graph.
    h = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((64, 512), dtype=torch.uint8, device=DEV)
    sc = torch.empty((64, 16), dtype=torch.uint8, device=DEV)
    cnt = torch.empty(1, dtype=torch.int64, device=DEV)
    hd = torch.empty((4, 264), dtype=torch.bfloat16, device=DEV)
    grads = {}

    def step():
        S.fwd(x, wg, wu, out=h)
        grads["b"] = S.bwd(x, wg, wu, dh, workspace=ws)
        S.act_quant(gate, up, 7.0, out=(q, sc, cnt, None))
        S.gemv_fwd(xd, wgd, wud, out=hd)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (h, *grads["b"], q, sc, cnt, hd)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the caching allocator outside capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    captured = (h, *grads["b"], q, sc, cnt, hd)
    for rep in range(3):
        for t in captured:                        # scribble over the outputs eagerly
            t.zero_() if t.dtype != torch.bfloat16 else t.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(captured, eager)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}, output {i}"
        # eager work between replays, counting calls among it (they take the
        # other regions of the library's count slots)
        _ = S.fwd(x, wg, wu)
        for _ in range(rep + 1):
            _ = S.act_quant(gate, up, 0.5)
        torch.cuda.synchronize()
    assert math.isfinite(float(eager[0].float().abs().max()))
