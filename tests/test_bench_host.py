"""Host-side logic of bench.py (CPU only): the work formulas behind the
roofline, the traffic-record lookup, the CPU oracle baseline and the one-GPU
guard."""

import hashlib
import json
import os
import subprocess
import sys
from itertools import product

import numpy as np
import pytest

import bench
import workloads as wlm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _count_flops(r, c):
    """Multiply-add count of one iteration by brute force over the outputs each
    stage computes (upper triangles of the symmetric ones), two flops each."""
    a = sum(2 * c for i, j in product(range(r), range(r)) if i <= j)
    b = sum(2 * r for i, j in product(range(r), range(r)) if i <= j)
    x = sum(2 * r for i, j in product(range(r), range(c)))
    return {"a": a, "b": b, "x": x}


@pytest.mark.parametrize("r,c", [(1, 1), (1, 5), (2, 3), (4, 4), (3, 7)])
def test_ns_flops_match_a_direct_count(r, c):
    assert bench.ns_flops(r, c) == _count_flops(r, c)


def test_stage_flops_take_the_shorter_side():
    wl = wlm._contiguous("t", [(3, 7), (7, 3)], ["w", "t"], "bf16", 0.02, 1e-3)
    want = {k: 2 * v for k, v in _count_flops(3, 7).items()}
    assert bench.stage_flops(wl, 5) == want


def test_dense_flops_count_full_products():
    wl = wlm._contiguous("t", [(3, 7), (7, 3), (5, 5)], ["w", "t", "s"], "bf16", 0.02, 1e-3)
    # full A = X X^T (2 r^2 c), full A A (2 r^3), full B X (2 r^2 c)
    want = sum(2 * r * r * c + 2 * r ** 3 + 2 * r * r * c for r, c in [(3, 7), (3, 7), (5, 5)])
    assert bench.dense_flops(wl) == want


def test_elementwise_bytes_per_element():
    wl = wlm._contiguous("t", [(8, 16)], ["w"], "bf16", 0.02, 1e-3)
    n = 8 * 16
    got = bench.elementwise_bytes(wl, "bf16")
    assert got["front_cast"] == 14 * n   # G, M read; M written; bf16 iterate written
    assert got["front"] == 16 * n
    assert got["apply"] == 8 * n         # O read, bf16 W read and written
    wl32 = wlm._contiguous("t", [(8, 16)], ["w"], "f32", 0.02, 1e-3)
    assert bench.elementwise_bytes(wl32, "f32")["apply"] == 12 * n
    assert bench.elementwise_bytes(wl32, "f32")["front_cast"] == 16 * n


def test_kernel_sources_exist():
    for k in ("ns_x_t256_bf16", "ns_a_t128+64_f32", "front", "apply", "front_cast", "norm"):
        assert os.path.exists(os.path.join(ROOT, "newton_schulz_flat_amd", "csrc",
                                           bench.kernel_source(k))), k


def test_recorded_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    csrc = tmp_path / "newton_schulz_flat_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k_ns_gemm.hip").write_bytes(b"kernel source, version 1")
    rec = {"sources_sha256": {"k_ns_gemm.hip": hashlib.sha256(b"kernel source, version 1").hexdigest()},
           "per_launch_bytes": {"ns_x_t256_bf16": {"read": 3.0e9, "written": 0.5e9}}}
    (tmp_path / "profiles" / "w_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("ns_x_t256_bf16", "w") == pytest.approx(3.5e9)
    assert bench.recorded_traffic("ns_a_t256_bf16", "w") is None  # not profiled
    assert bench.recorded_traffic("ns_x_t256_bf16", "other") is None  # no record
    (csrc / "k_ns_gemm.hip").write_bytes(b"kernel source, version 2")
    assert bench.recorded_traffic("ns_x_t256_bf16", "w") is None  # source changed


def test_committed_traffic_records_are_well_formed():
    for name in ("owner_share", "llama_layer", "moe_set"):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"{name}_traffic.json")))
        assert set(rec["sources_sha256"]) >= {"k_ns_gemm.hip", "k_norm_cast.hip"}
        for k, b in rec["per_launch_bytes"].items():
            assert b["read"] >= 0 and b["written"] >= 0, (name, k)
        assert "ns_x_t256_bf16" in rec["per_launch_bytes"], name


def test_cpu_baseline_fields_on_a_small_workload():
    wl = wlm.make_workload("single")
    out = bench.cpu_baseline(wl, budget_s=0.01)
    assert out["kind"] == "oracle" and out["unit"] == "matrices/s"
    assert out["value"] > 0 and np.isfinite(out["value"])
    assert out["cores"] >= 1 and out["nproc"] >= 1
    assert isinstance(out["cpu_model"], str) and isinstance(out["blas"], str)
    assert "256x512" in out["sample"]
    assert out["seconds_per_step"] == pytest.approx(wl.n / out["value"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
