"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts the roofline divides by, the traffic entry's source check, and the
benchmark workloads' shapes."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_are_the_hand_count():
    b = _bench()
    from workloads import WORKLOADS
    # decode: every expert's W1 (2F x H) and W2 (H x F) in bf16, each live
    # token's x row, its k ids and probabilities (4 + 4 bytes), its fp32 output
    w = WORKLOADS["decode"]
    ab = b.alg_bytes(w, "bf16", touched=64)
    weights = 64 * (2 * 1024 * 2048 + 2048 * 1024) * 2
    assert ab["step"] == weights + 256 * 2048 * 2 + 256 * 6 * 8 + 256 * 2048 * 4
    # the FC1 stage: W1, x rows, the SwiGLU rows written (bf16 [R][F])
    assert ab["fc1"] == 64 * 2 * 1024 * 2048 * 2 + 256 * 2048 * 2 + 256 * 6 * 1024 * 2
    # bounded decode counts the live tokens only, never the 65,536-row capacity
    w = WORKLOADS["bounded_decode"]
    ab = b.alg_bytes(w, "bf16", touched=128)
    assert ab["step"] == (128 * 3 * 2688 * 1856 * 2 + 512 * 2688 * 2 + 512 * 6 * 8
                          + 512 * 2688 * 4)
    # MXFP8: one byte per weight plus one E8M0 byte per 32; MXFP4: half a byte
    w = WORKLOADS["mxfp8_16k"]
    assert b.alg_bytes(w, "mxfp8", 128)["step"] == pytest.approx(
        128 * 3 * 2048 * 1024 * (1 + 1 / 32) + 16384 * 2048 * 2 + 16384 * 8 * 8 + 16384 * 2048 * 4)
    assert b.alg_bytes(w, "mxfp4", 128)["step"] == pytest.approx(
        128 * 3 * 2048 * 1024 * (0.5 + 1 / 32) + 16384 * 2048 * 2 + 16384 * 8 * 8 + 16384 * 2048 * 4)
    # the other combines change only the output term
    w = WORKLOADS["decode"]
    d = b.alg_bytes(w, "bf16", 64, "fp32")["step"]
    assert b.alg_bytes(w, "bf16", 64, "bf16")["step"] == d - 256 * 2048 * 2
    assert b.alg_bytes(w, "bf16", 64, "rows")["step"] == d - 256 * 2048 * 4 + 256 * 6 * 2048 * 4


def test_traffic_entry_is_dropped_once_a_gemm_source_changes(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "kernel.h"
    src.write_text("// a kernel\n")
    (tmp_path / "profiles").mkdir()
    entry = dict(gemm_source_sha256=hashlib.sha256(src.read_bytes()).hexdigest(),
                 fetch_bytes_per_launch=1000.0, write_bytes_per_launch=24.0)
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"decode": entry}))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "GEMM_SOURCES", ["kernel.h"])
    assert b.measured_traffic("decode") == 1024.0
    assert b.measured_traffic("bf16_16k") is None          # no entry
    src.write_text("// a changed kernel\n")
    assert b.measured_traffic("decode") is None


def test_every_gemm_source_in_the_traffic_check_exists():
    b = _bench()
    for s in b.GEMM_SOURCES:
        assert os.path.exists(os.path.join(ROOT, s)), s


def test_workload_shapes():
    from workloads import WORKLOADS
    shapes = {n: (w.T, w.T_cap, w.H, w.F, w.E, w.k, w.precision) for n, w in WORKLOADS.items()}
    assert shapes["tiny"] == (64, 64, 128, 256, 8, 2, "bf16")
    assert shapes["decode"] == (256, 256, 2048, 1024, 64, 6, "bf16")
    assert shapes["logprob"] == (4096, 4096, 2048, 1024, 128, 8, "bf16") and WORKLOADS["logprob"].bias
    assert shapes["mxfp8_16k"] == (16384, 16384, 2048, 1024, 128, 8, "mxfp8")
    assert shapes["bf16_16k"] == (16384, 16384, 2048, 1024, 128, 8, "bf16")
    assert shapes["bounded_decode"] == (512, 65536, 2688, 1856, 128, 6, "bf16")


def test_default_run_covers_every_workload_and_picks_the_roofline():
    """The default run measures every benchmark workload with decode as the
    headline; the FC1 roofline is the one whose floor is higher (MFMA for the
    16K-token workloads, HBM for the decode-sized ones)."""
    b = _bench()
    from workloads import WORKLOADS
    assert set(b.ALL_WORKLOADS) == set(WORKLOADS) and b.ALL_WORKLOADS[0] == b.HEADLINE == "decode"
    w = WORKLOADS["bf16_16k"]
    ab = b.alg_bytes(w, "bf16", 128)
    r = b.roofline_of(w, ab, 1000.0)
    assert r["bound"] == "mfma" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(4 * 2048 * 1024 * 131072 / 1e-3 / 1e12)
    assert r["other_bound"]["bound"] == "hbm"
    w = WORKLOADS["decode"]
    r = b.roofline_of(w, b.alg_bytes(w, "bf16", 64), 100.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(b.alg_bytes(w, "bf16", 64)["fc1"] / 100e-6 / 1e9 / 8000.0)
