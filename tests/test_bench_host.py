"""Host-side checks of bench.py's contract pieces (no GPU needed)."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    """A copy of the forward kernel's sources under a temporary root."""
    csrc = tmp_path / "swiglu_mlp_fwd_amd" / "csrc"
    csrc.mkdir(parents=True)
    for fn in bench.FWD_KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "swiglu_mlp_fwd_amd", "csrc", fn), csrc / fn)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_source_hash_ignores_comments_but_not_code(fake_root):
    h0 = bench.kernel_source_hash()
    gemm = fake_root / "swiglu_mlp_fwd_amd" / "csrc" / "gemm.hip"
    text = gemm.read_text()
    gemm.write_text("// a new comment line\n/* and a block\n   comment */\n" + text + "\n\n")
    assert bench.kernel_source_hash() == h0
    gemm.write_text(text + "\nconstexpr int kOneMoreConstant = 1;\n")     # a line of code
    assert bench.kernel_source_hash() != h0


def test_traffic_is_reported_only_for_the_measured_sources(fake_root):
    name = "fwd_dual_gemm_bf16_8192x14336x4096"
    entry = {"source_hash": bench.kernel_source_hash(), "bytes_per_launch": 123456789}
    (fake_root / "profiles" / "traffic.json").write_text(json.dumps({name: entry}))
    assert bench.load_traffic(name) == 123456789
    entry["source_hash"] = "0" * 16
    (fake_root / "profiles" / "traffic.json").write_text(json.dumps({name: entry}))
    assert bench.load_traffic(name) is None
    (fake_root / "profiles" / "traffic.json").unlink()
    assert bench.load_traffic(name) is None


def test_clock_adjusted_roofline_needs_cycles_counted_on_the_current_sources(fake_root):
    name = "fwd_dual_gemm_bf16_8192x14336x4096"
    entry = {"source_hash": bench.kernel_source_hash(), "cycles_per_launch": 2_400_000,
             "mfma_busy_cycles_per_simd": 1_800_000}
    (fake_root / "profiles" / "cycles.json").write_text(json.dumps({name: entry}))
    r = bench.clock_adjusted(name, 1000.0, 1.5e-3)     # 2.4 M cycles in 1.5 ms: 1.6 GHz
    assert r["sclk_GHz"] == 1.6
    assert abs(r["peak"] - bench.PEAK_BF16_TFLOPS * 1.6 / 2.4) < 0.1
    assert abs(r["frac"] - 1000.0 / (bench.PEAK_BF16_TFLOPS * 1.6 / 2.4)) < 1e-4
    assert r["mfma_busy_frac"] == 0.75
    entry["source_hash"] = "0" * 16
    (fake_root / "profiles" / "cycles.json").write_text(json.dumps({name: entry}))
    assert bench.clock_adjusted(name, 1000.0, 1.5e-3) is None
    (fake_root / "profiles" / "cycles.json").unlink()
    assert bench.clock_adjusted(name, 1000.0, 1.5e-3) is None
