"""Host-side tests of the C-ABI library (no GPU): it loads, exports every
symbol the header declares, and rejects invalid arguments before any launch.

Every call here fails validation, so no kernel is enqueued and no HIP call is
made (validation runs on the host before anything else).
"""
import ctypes
import math
import os
import re

import pytest

import swiglu_mlp_fwd_amd as S
from swiglu_mlp_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swiglu.h")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EARG, EUNSUP = 0, 1, 2, 3, 4, 5, 6, 7
A = 0x10000  # a 16-byte-aligned fake device address; never dereferenced
MIS = 0x10008


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from swiglu_mlp_fwd_amd import build
        build.build()
    return S.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(swiglu_\w+)\s*\(", src, flags=re.M)


def test_header_declares_the_entry_points():
    names = set(header_functions())
    for n in ("swiglu_fwd", "swiglu_bwd", "swiglu_bwd_workspace_bytes", "swiglu_gemv_fwd",
              "swiglu_act_quant", "swiglu_status_str", "swiglu_last_hip_error"):
        assert n in names


def test_library_resolves_every_symbol_at_load():
    """Loading with immediate binding resolves every function the library
    calls, so no entry point can fail later on an undefined symbol (a
    declaration given C linkage by mistake, say)."""
    ctypes.CDLL(_lib.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_library_exports_every_header_symbol(L):
    names = header_functions()
    assert names
    for n in names:
        assert hasattr(L, n), n
    # ...and the binding's signature table covers exactly those symbols.
    assert set(names) == set(_lib.SIGNATURES)


def test_version_and_status_strings(L):
    assert L.swiglu_version() >= 100
    assert L.swiglu_status_str(0) == b"ok"
    for s in range(1, 10):
        assert L.swiglu_status_str(s) not in (b"ok", b"unknown status")
    assert L.swiglu_status_str(99) == b"unknown status"
    assert L.swiglu_last_hip_error() == 0


def test_fwd_validation(L):
    f = L.swiglu_fwd
    assert f(2, 4, 4, 8, A, A, A, A, None) == EDTYPE
    assert f(1, -1, 4, 8, A, A, A, A, None) == ESHAPE
    assert f(1, 4, 4, 12, A, A, A, A, None) == ESHAPE          # bf16 needs K % 8 == 0
    assert f(0, 4, 4, 6, A, A, A, A, None) == ESHAPE           # fp32 needs K % 4 == 0
    assert f(1, 4, 4, 8, None, A, A, A, None) == ENULL
    assert f(1, 4, 4, 8, A, A, A, None, None) == ENULL
    assert f(1, 4, 4, 8, A, MIS, A, A, None) == EALIGN
    assert f(1, 1 << 31, 4, 8, A, A, A, A, None) == ESHAPE
    assert f(1, 0, 4, 8, None, None, None, None, None) == OK   # empty: nothing to do
    assert f(1, 4, 0, 8, None, None, None, None, None) == OK


def test_bwd_validation(L):
    f = L.swiglu_bwd
    need = L.swiglu_bwd_workspace_bytes(1, 100, 60, 64)
    assert need > 0 and need % 256 == 0
    assert L.swiglu_bwd_workspace_bytes(5, 1, 1, 8) == 0
    assert L.swiglu_bwd_workspace_bytes(1, -1, 1, 8) == 0
    args = [1, 100, 60, 64, A, A, A, A, A, A, A]
    assert f(*args, A, need - 1, None) == EWS
    assert f(*args, None, need, None) == EWS
    assert f(*args, 0x10010, need, None) == EALIGN             # workspace needs 256-byte alignment
    assert f(1, 100, 60, 64, A, A, A, None, A, A, A, A, need, None) == ENULL
    assert f(1, 100, 60, 60, A, A, A, A, A, A, A, A, need, None) == ESHAPE
    assert f(1, 100, 60, 64, A, A, A, A, A, MIS, A, A, need, None) == EALIGN
    assert f(1, 100, 60, 0, None, None, None, None, None, None, None, None, 0, None) == OK


def test_workspace_layout_formula(L):
    # D [M, 2Np] + DT [2Np, Mp] + XT [K, Mp] + WT [K, 2Np], each 256-byte
    # aligned; Np = round_up(N, 8) for fp32 and round_up(N, 64) for bf16.
    def a256(v):
        return (v + 255) // 256 * 256
    for (M, N, K) in ((100, 60, 64), (8192, 14336, 4096), (1, 1, 8)):
        Mp, Np = -(-M // 8) * 8, -(-N // 8) * 8
        want = a256(M * 2 * Np * 4) + a256(2 * Np * Mp * 4) + a256(K * Mp * 4) + a256(K * 2 * Np * 4)
        assert L.swiglu_bwd_workspace_bytes(0, M, N, K) == want
        Np = -(-N // 64) * 64
        want = a256(M * 2 * Np * 2) + a256(2 * Np * Mp * 2) + a256(K * Mp * 2) + a256(K * 2 * Np * 2)
        assert L.swiglu_bwd_workspace_bytes(1, M, N, K) == want


@pytest.mark.parametrize("dt", [0, 1])
def test_leading_dimension_limit(L, dt):
    # Both element types: an operand tile spans 512 bytes per unit of row
    # stride (256 bf16 rows, 128 fp32 rows) and is addressed with 32-bit
    # offsets, so every stride a GEMM reads with is capped at 2^22 - 64.
    EUNSUP = 7
    lim = (1 << 22) - 64
    npad = 64 if dt == 1 else 8
    # forward: K at the limit is accepted (validation only: M = 0), K past it is not
    assert L.swiglu_fwd(dt, 0, 4, lim, None, None, None, None, None) == OK
    assert L.swiglu_fwd(dt, 4, 4, lim + 64, A, A, A, A, None) == EUNSUP
    assert L.swiglu_fwd_act(0, dt, 4, 4, lim + 8, A, A, A, A, None) == EUNSUP
    assert L.swiglu_fwd_mult(0, dt, 4, 4, lim + 8, A, A, A, 1.0, 1.0, A, None) == EUNSUP
    # backward: K, 2 Np and Mp
    assert L.swiglu_bwd_workspace_bytes(dt, 4, 4, lim + 64) == 0
    assert L.swiglu_bwd(dt, 4, 4, lim + 64, A, A, A, A, A, A, A, A, 1 << 62, None) == EUNSUP
    n_ok = (lim // 2) // npad * npad              # largest N with 2 Np <= lim
    assert L.swiglu_bwd_workspace_bytes(dt, 4, n_ok, 8) > 0
    n_big = n_ok + 1                              # 2 Np = 2 n_ok + 2 npad > lim
    assert L.swiglu_bwd_workspace_bytes(dt, 4, n_big, 8) == 0    # sizes the backward rejects have no size
    assert L.swiglu_bwd(dt, 4, n_big, 8, A, A, A, A, A, A, A, A, 1 << 62, None) == EUNSUP
    m_big = lim + 8                               # Mp = lim + 8
    assert L.swiglu_bwd_workspace_bytes(dt, m_big, 4, 8) == 0
    assert L.swiglu_bwd(dt, m_big, 4, 8, A, A, A, A, A, A, A, A, 1 << 62, None) == EUNSUP
    assert L.swiglu_bwd_act_mult(0, dt, m_big, 4, 8, A, A, A, A, 1.0, 1.0, A, A, A, A, 1 << 62, None) == EUNSUP
    assert L.swiglu_bwd_workspace_bytes(dt, lim, 4, 8) > 0                 # Mp = lim is accepted
    # huge sizes never wrap to a small workspace
    assert L.swiglu_bwd_workspace_bytes(dt, (1 << 31) - 1, (1 << 31) - 1, 8) == 0


def test_gemv_validation(L):
    f = L.swiglu_gemv_fwd
    assert f(9, 16, 64, A, A, A, A, None) == ESHAPE
    assert f(-1, 16, 64, A, A, A, A, None) == ESHAPE
    assert f(2, 16, 60, A, A, A, A, None) == ESHAPE
    # No limit on K beyond K % 8 (x is staged in phases along K); N = 0
    # keeps these calls from launching.
    assert f(8, 0, 1 << 20, A, A, A, A, None) == OK
    assert f(1, 0, (1 << 31) - 8, A, A, A, A, None) == OK
    assert f(1, 0, 1 << 31, A, A, A, A, None) == ESHAPE         # past the int range of a dimension
    p = L.swiglu_probe_gemv_read
    assert p(8, 0, 1 << 20, A, A, A, A, None) == OK
    assert p(9, 16, 64, A, A, A, A, None) == ESHAPE
    assert p(2, 16, 64, A, A, A, None, None) == ENULL
    assert p(2, 16, 64, A, A, A, 0x10002, None) == EALIGN       # sink: 4-byte aligned
    assert p(2, 16, 64, MIS, A, A, A, None) == EALIGN
    assert p(0, 16, 64, None, None, None, None, None) == OK
    assert f(2, 16, 64, A, None, A, A, None) == ENULL
    assert f(2, 16, 64, A, A, A, MIS, None) == EALIGN
    assert f(0, 16, 64, None, None, None, None, None) == OK


def test_act_quant_validation(L):
    f = L.swiglu_act_quant
    assert f(4, 48, A, A, 7.0, A, A, None, None, None) == ESHAPE   # cols % 32
    assert f(-1, 64, A, A, 7.0, A, A, None, None, None) == ESHAPE
    assert f(4, 64, A, A, 0.0, A, A, None, None, None) == EARG
    assert f(4, 64, A, A, -1.0, A, A, None, None, None) == EARG
    assert f(4, 64, A, A, math.nan, A, A, None, None, None) == EARG
    assert f(4, 64, None, A, 7.0, A, A, None, None, None) == ENULL
    assert f(4, 64, A, A, 7.0, A, None, None, None, None) == ENULL
    assert f(4, 64, A, A, 7.0, A, A, 0x10004, None, None) == EALIGN  # count needs 8-byte alignment
    assert f(4, 64, A, A, math.inf, MIS, A, None, None, None) == EALIGN


def test_activation_choice_validation(L):
    # An unknown activation is rejected before anything else.
    assert L.swiglu_fwd_act(2, 1, 4, 4, 8, A, A, A, A, None) == EARG
    assert L.swiglu_fwd_act(-1, 1, 4, 4, 8, A, A, A, A, None) == EARG
    assert L.swiglu_gemv_fwd_act(7, 1, 4, 8, A, A, A, A, None) == EARG
    # Known activations reach the usual validation.
    assert L.swiglu_fwd_act(1, 1, 4, 4, 12, A, A, A, A, None) == ESHAPE     # K % 8
    assert L.swiglu_gemv_fwd_act(1, 9, 4, 8, A, A, A, A, None) == ESHAPE    # M <= 8
    assert L.swiglu_fwd_act(1, 1, 0, 4, 8, None, None, None, None, None) == OK


def test_act_quant_activation_validation(L):
    f = L.swiglu_act_quant_act
    assert f(2, 4, 64, A, A, 7.0, A, A, None, None, None) == EARG
    assert f(1, 4, 48, A, A, 7.0, A, A, None, None, None) == ESHAPE
    assert f(1, 4, 64, A, A, 0.0, A, A, None, None, None) == EARG


def test_multiplier_validation(L):
    inf, nan = math.inf, math.nan
    assert L.swiglu_fwd_mult(0, 1, 4, 4, 8, A, A, A, inf, 1.0, A, None) == EARG
    assert L.swiglu_fwd_mult(0, 1, 4, 4, 8, A, A, A, 1.0, nan, A, None) == EARG
    assert L.swiglu_fwd_mult(2, 1, 4, 4, 8, A, A, A, 1.0, 1.0, A, None) == EARG
    assert L.swiglu_fwd_mult(0, 1, 4, 4, 12, A, A, A, 0.5, 2.0, A, None) == ESHAPE
    assert L.swiglu_gemv_fwd_mult(0, 2, 16, 64, A, A, A, -inf, 1.0, A, None) == EARG
    assert L.swiglu_gemv_fwd_mult(0, 9, 16, 64, A, A, A, 0.5, 1.0, A, None) == ESHAPE
    need = L.swiglu_bwd_workspace_bytes(1, 100, 60, 64)
    assert L.swiglu_bwd_mult(1, 100, 60, 64, A, A, A, A, nan, 1.0, A, A, A, A, need, None) == EARG
    assert L.swiglu_bwd_mult(1, 100, 60, 64, A, A, A, A, 0.5, 1.0, A, A, A, A, need - 1, None) == EWS
    assert L.swiglu_bwd_act_mult(2, 1, 100, 60, 64, A, A, A, A, 1.0, 1.0, A, A, A, A, need, None) == EARG
    assert L.swiglu_bwd_act_mult(1, 1, 100, 60, 64, A, A, A, A, 1.0, 1.0, A, A, A, A, need - 1, None) == EWS


def test_act_fwd_validation(L):
    f = L.swiglu_act_fwd
    assert f(2, 0, 4, 64, A, A, 7.0, A, None, None) == EARG           # unknown activation
    assert f(0, 5, 4, 64, A, A, 7.0, A, None, None) == EDTYPE         # unknown output type
    assert f(0, 1, 4, 60, A, A, 7.0, A, None, None) == ESHAPE         # cols % 8
    assert f(0, 0, 4, 64, A, A, 0.0, A, None, None) == EARG
    assert f(0, 0, 4, 64, A, A, math.nan, A, None, None) == EARG
    assert f(0, 0, 4, 64, None, A, 7.0, A, None, None) == ENULL
    assert f(1, 1, 4, 64, A, A, 7.0, None, None, None) == ENULL
    assert f(0, 0, 4, 64, A, A, 7.0, MIS, None, None) == EALIGN
    assert f(0, 0, 4, 64, A, A, 7.0, A, 0x10004, None) == EALIGN       # count: 8-byte aligned


def test_fwd_fp8_validation(L):
    f = L.swiglu_fwd_fp8
    assert f(2, 4, 64, 8, A, A, A, A, A, None, None) == EARG           # unknown activation
    assert f(0, 4, 48, 8, A, A, A, A, A, None, None) == ESHAPE         # N % 32
    assert f(0, 4, 64, 12, A, A, A, A, A, None, None) == ESHAPE        # bf16: K % 8
    assert f(0, -1, 64, 8, A, A, A, A, A, None, None) == ESHAPE
    assert f(0, 4, 64, (1 << 22), A, A, A, A, A, None, None) == EUNSUP
    assert f(1, 4, 64, 8, A, A, A, None, A, None, None) == ENULL       # q
    assert f(1, 4, 64, 8, A, A, A, A, None, None, None) == ENULL       # scale
    assert f(1, 4, 64, 8, A, A, A, MIS, A, None, None) == EALIGN       # q: 16-byte rows
    assert f(1, 4, 64, 8, A, A, A, A, A, MIS, None) == EALIGN          # h_out
    assert f(0, 4, 64, 8, A, MIS, A, A, A, None, None) == EALIGN
    assert f(0, 0, 64, 8, None, None, None, None, None, None, None) == OK
    assert f(0, 4, 0, 8, None, None, None, None, None, None, None) == OK


def test_act_bwd_validation(L):
    f = L.swiglu_act_bwd
    assert f(4, 62, A, A, A, None, 7.0, A, A, None, None) == ESHAPE    # cols % 4
    assert f(-1, 64, A, A, A, None, 7.0, A, A, None, None) == ESHAPE
    assert f(4, 64, A, A, A, None, 0.0, A, A, None, None) == EARG
    assert f(4, 64, A, A, A, None, math.nan, A, A, None, None) == EARG
    assert f(4, 64, A, None, A, None, 7.0, A, A, None, None) == ENULL
    assert f(4, 64, A, A, A, None, 7.0, A, None, None, None) == ENULL
    assert f(4, 64, A, A, MIS, None, math.inf, A, A, None, None) == EALIGN
    assert f(4, 64, A, A, A, 0x10002, math.inf, A, A, None, None) == EALIGN   # weights: 4-byte aligned
    assert f(0, 64, None, None, None, None, 7.0, None, None, None, None) == OK


def test_act_bwd_format_validation(L):
    f = L.swiglu_act_bwd_dt
    assert f(5, 4, 64, A, A, A, None, 7.0, A, A, None, None) == EDTYPE
    assert f(1, 4, 60, A, A, A, None, 7.0, A, A, None, None) == ESHAPE     # bf16: cols % 8
    assert f(0, 4, 60, A, A, A, None, 7.0, A, None, None, None) == ENULL   # fp32: cols % 4 suffices
    assert f(1, 4, 64, A, A, MIS, None, 7.0, A, A, None, None) == EALIGN
    assert f(1, 4, 64, A, A, A, None, 7.0, A, None, None, None) == ENULL


def test_probe_mfma_validation(L):
    assert L.swiglu_probe_mfma(-1, 4, A, None) == ESHAPE
    assert L.swiglu_probe_mfma(4, 4, None, None) == ENULL
    assert L.swiglu_probe_mfma(0, 4, None, None) == OK


def test_probe_validation(L):
    assert L.swiglu_probe_read2(A, A, 17, A, None) == ESHAPE
    assert L.swiglu_probe_read2(None, A, 32, A, None) == ENULL
    assert L.swiglu_probe_read2(A, A, 0, A, None) == OK


def test_probe_read2_cfg_validation(L):
    assert L.swiglu_probe_read2_cfg(A, A, 32, 128, 4, 4096, A, None) == EARG
    assert L.swiglu_probe_read2_cfg(A, A, 32, 256, 3, 4096, A, None) == EARG
    assert L.swiglu_probe_read2_cfg(A, A, 32, 512, 1, 0, A, None) == EARG
    assert L.swiglu_probe_read2_cfg(A, A, 32, 512, 1, 65536, A, None) == EARG
    assert L.swiglu_probe_read2_cfg(A, A, 17, 256, 8, 4096, A, None) == ESHAPE
    assert L.swiglu_probe_read2_cfg(None, A, 32, 256, 8, 4096, A, None) == ENULL
    assert L.swiglu_probe_read2_cfg(A, A, 0, 512, 2, 16384, A, None) == OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_product_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "swiglu_mlp_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "synth" not in text, fn


def test_bwd_noalloc_validation(L):
    # Errors as swiglu_bwd_act_mult's, then the static-scratch bound; every
    # case returns before any HIP call.
    f = L.swiglu_bwd_noalloc
    ESCRATCH = 9
    assert f(2, 1, 4, 64, 8, A, A, A, A, 1.0, 1.0, A, A, A, None) == EARG          # unknown activation
    assert f(0, 1, 4, 64, 8, A, A, A, A, math.nan, 1.0, A, A, A, None) == EARG     # multiplier
    assert f(0, 5, 4, 64, 8, A, A, A, A, 1.0, 1.0, A, A, A, None) == EDTYPE
    assert f(0, 1, 4, 64, 12, A, A, A, A, 1.0, 1.0, A, A, A, None) == ESHAPE       # bf16: K % 8
    assert f(0, 1, 4, 64, 8, None, A, A, A, 1.0, 1.0, A, A, A, None) == ENULL
    assert f(0, 1, 4, 64, 8, A, A, A, A, 1.0, 1.0, MIS, A, A, None) == EALIGN
    assert f(0, 1, 4, 64, (1 << 22), A, A, A, A, 1.0, 1.0, A, A, A, None) == EUNSUP
    assert f(0, 1, 4, 64, 0, None, None, None, None, 1.0, 1.0, None, None, None, None) == OK   # K == 0: nothing to do
    big = (4096, 8192, 4096)
    assert L.swiglu_bwd_workspace_bytes(1, *big) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(0, 1, *big, A, A, A, A, 1.0, 1.0, A, A, A, None) == ESCRATCH
    assert f(1, 0, *big, A, A, A, A, 1.0, 1.0, A, A, A, None) == ESCRATCH
    assert L.swiglu_status_str(ESCRATCH) == b"problem needs more scratch than the static buffer holds"


def test_library_is_built_from_the_tree(L):
    # The loaded library carries the hash of the sources it was built from.
    from swiglu_mlp_fwd_amd.build import source_hash
    assert L.swiglu_source_hash().decode() == source_hash()


def test_a_stale_library_is_refused(monkeypatch):
    # Sources that hash differently from the library's embedded hash: the
    # loader raises instead of handing out the library.
    import swiglu_mlp_fwd_amd.build as B
    monkeypatch.setattr(B, "source_hash", lambda: "0000000000000000")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="stale"):
        _lib.lib()
    monkeypatch.undo()
    _lib._lib = None
    assert _lib.lib() is not None
