"""Host-side tests of the PyTorch wrappers (no GPU): malformed calls are
rejected before the library is touched.

The C ABI receives raw pointers, so the wrappers are what stands between a
wrong weight shape or a short out= tensor and a kernel reading or writing past
an allocation.  Here the library accessor is replaced by one that fails the
test if it is reached: every case must raise in the wrapper itself.  A
well-formed call on CPU tensors must stop at the device check, also before
the library.
"""
import pytest
import torch

import swiglu_mlp_fwd_amd.ops as ops


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def fail():
        raise AssertionError("the library was reached by a call that should have been rejected")
    monkeypatch.setattr(ops, "lib", fail)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


GPU_ONLY = "GPU tensors only"


# ----------------------------------------------------------------- fwd

def test_fwd_weight_shapes():
    with pytest.raises(ValueError, match="weights"):
        ops.fwd(bf(4, 64), bf(128, 64), bf(128, 72))
    with pytest.raises(ValueError, match="weights"):
        ops.fwd(bf(4, 64), bf(128, 72), bf(128, 72))
    with pytest.raises(ValueError, match=r"\[N, K\]"):
        ops.fwd(bf(4, 64), bf(128), bf(128))


@pytest.mark.parametrize("bad,exc", [
    (bf(4, 127), ValueError),                                  # short
    (bf(5, 128), ValueError),                                  # long
    (f32(4, 128), TypeError),                                  # dtype
    (bf(128, 4).t(), ValueError),                              # not contiguous
])
def test_fwd_out(bad, exc):
    with pytest.raises(exc):
        ops.fwd(bf(4, 64), bf(128, 64), bf(128, 64), out=bad)


def test_fwd_dtypes():
    with pytest.raises(TypeError):
        ops.fwd(bf(4, 64), f32(128, 64), f32(128, 64))
    with pytest.raises(TypeError):
        ops.fwd(torch.zeros(4, 64, dtype=torch.float16), torch.zeros(128, 64, dtype=torch.float16),
                torch.zeros(128, 64, dtype=torch.float16))


def test_fwd_well_formed_stops_at_the_device_check():
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.fwd(bf(2, 3, 64), bf(128, 64), bf(128, 64), out=bf(6, 128))


# ----------------------------------------------------------------- fwd_fp8

@pytest.mark.parametrize("which,bad", [
    (0, u8(4, 96)), (0, bf(4, 128)), (1, u8(4, 3)), (1, u8(5, 4)), (2, f32(4, 96)), (2, bf(4, 128)),
])
def test_fwd_fp8_out(which, bad):
    out = [u8(4, 128), u8(4, 4), f32(4, 128)]
    out[which] = bad
    with pytest.raises((ValueError, TypeError)):
        ops.fwd_fp8(bf(4, 64), bf(128, 64), bf(128, 64), out=tuple(out))


def test_fwd_fp8_weights_and_missing_outputs():
    with pytest.raises(ValueError, match="weights"):
        ops.fwd_fp8(bf(4, 64), bf(128, 64), bf(96, 64))
    with pytest.raises(ValueError, match="required"):
        ops.fwd_fp8(bf(4, 64), bf(128, 64), bf(128, 64), out=(None, u8(4, 4), None))
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.fwd_fp8(bf(4, 64), bf(128, 64), bf(128, 64), out=(u8(4, 128), u8(4, 4), None))


# ----------------------------------------------------------------- bwd

def test_bwd_weight_and_dh_shapes():
    with pytest.raises(ValueError, match="weights"):
        ops.bwd(bf(4, 64), bf(128, 64), bf(120, 64), bf(4, 128))
    with pytest.raises(ValueError, match="weights"):
        ops.bwd(bf(4, 64), bf(128, 64), bf(128, 56), bf(4, 128))
    with pytest.raises(ValueError, match="dh"):
        ops.bwd(bf(4, 64), bf(128, 64), bf(128, 64), bf(4, 120))


@pytest.mark.parametrize("which,bad", [
    (0, bf(4, 56)), (0, f32(4, 64)), (1, bf(120, 64)), (1, bf(64, 128).t()), (2, bf(128, 72)), (2, f32(128, 64)),
])
def test_bwd_out(which, bad):
    out = [bf(4, 64), bf(128, 64), bf(128, 64)]
    out[which] = bad
    with pytest.raises((ValueError, TypeError)):
        ops.bwd(bf(4, 64), bf(128, 64), bf(128, 64), bf(4, 128), out=tuple(out))


def test_bwd_workspace_must_be_contiguous():
    ws = u8(64, 64).t()
    with pytest.raises(ValueError, match="workspace"):
        ops.bwd(bf(4, 64), bf(128, 64), bf(128, 64), bf(4, 128), workspace=ws)
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.bwd(bf(4, 64), bf(128, 64), bf(128, 64), bf(4, 128), out=(bf(4, 64), bf(128, 64), bf(128, 64)))


# ----------------------------------------------------------------- gemv

def test_gemv_weight_shapes_and_out():
    with pytest.raises(ValueError, match="weights"):
        ops.gemv_fwd(bf(2, 64), bf(128, 64), bf(128, 32))
    with pytest.raises(ValueError, match="weights"):
        ops.gemv_fwd(bf(2, 64), bf(128, 56), bf(128, 56))
    with pytest.raises(ValueError):
        ops.gemv_fwd(bf(2, 64), bf(128, 64), bf(128, 64), out=bf(2, 127))
    with pytest.raises(TypeError):
        ops.gemv_fwd(bf(2, 64), bf(128, 64), bf(128, 64), out=f32(2, 128))
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.gemv_fwd(bf(2, 64), bf(128, 64), bf(128, 64), out=bf(2, 128))


# ----------------------------------------------------------------- elementwise

def test_act_quant_out():
    g, u = f32(3, 64), f32(3, 64)
    good = [u8(3, 64), u8(3, 2), torch.zeros(1, dtype=torch.int64), f32(3, 64)]
    for which, bad in ((0, u8(3, 32)), (1, u8(3, 1)), (2, torch.zeros(1, dtype=torch.int32)), (3, f32(3, 32)),
                       (0, f32(3, 64))):
        out = list(good)
        out[which] = bad
        with pytest.raises((ValueError, TypeError)):
            ops.act_quant(g, u, 7.0, out=tuple(out))
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.act_quant(g, u, 7.0, out=tuple(good))


def test_act_fwd_out():
    g, u = f32(3, 64), f32(3, 64)
    with pytest.raises(ValueError):
        ops.act_fwd(g, u, out=(f32(3, 56), None))
    with pytest.raises(TypeError):
        ops.act_fwd(g, u, out=(u8(3, 64), None))
    with pytest.raises(TypeError):
        ops.act_fwd(g, u, out=(f32(3, 64), torch.zeros(1, dtype=torch.float32)))
    with pytest.raises(TypeError):
        ops.act_fwd(g, u, out_dtype=torch.float16)
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.act_fwd(g, u, out=(bf(3, 64), torch.zeros(1, dtype=torch.int64)))


def test_act_bwd_out_and_weights():
    g = f32(3, 64)
    with pytest.raises(ValueError):
        ops.act_bwd(g, g, g, out=(f32(3, 60), f32(3, 64), None))
    with pytest.raises(TypeError):
        ops.act_bwd(g, g, g, out=(f32(3, 64), bf(3, 64), None))
    with pytest.raises(ValueError):
        ops.act_bwd(g, g, g, weights=f32(3), out=(f32(3, 64), f32(3, 64), f32(2)))
    with pytest.raises(ValueError):
        ops.act_bwd(g, g, g, weights=f32(4))
    with pytest.raises(ValueError, match=GPU_ONLY):
        ops.act_bwd(g, g, g, weights=f32(3), out=(f32(3, 64), f32(3, 64), f32(3)))
