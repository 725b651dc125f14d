"""Host-side checks of bench.py that need no GPU: the one-GPU refusal, the
algorithmic bytes of the decode step, and the guard on the recorded HBM
traffic figure."""
import os
import shutil
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ternary_weight_i2_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_stack(layers, N):
    """Objects with the shapes step_bytes reads: (x, xq, xs, xsum, mats) per
    dependency group, mats = (P, alpha, dot, y, M, K)."""
    out = []
    for _ in range(layers):
        groups = []
        for _, projs in bench.GROUPS:
            K = synth.SHAPES["b2"][projs[0]][1]
            mats = [(None, 0.0, None, None, synth.SHAPES["b2"][p][0], K) for p in projs]
            groups.append((SimpleNamespace(shape=(N, K)), None, None, None, mats))
        out.append({"groups": groups})
    return out


def test_step_bytes_of_the_2b_stack():
    # 30 layers; per layer the packed weights of q, o (2560x2560), k, v
    # (640x2560), gate, up (6912x2560) and down (2560x6912) at 2 bits; one bf16
    # token per dependency group (K = 2560 three times, 6912 once); 4 + 4
    # bytes per output row.
    packed = 30 * (2 * 2560 * 2560 + 2 * 640 * 2560 + 3 * 6912 * 2560) // 4
    tokens = 30 * 2 * (3 * 2560 + 6912)
    outputs = 30 * 8 * (2560 + 640 + 640 + 2560 + 6912 + 6912 + 2560)
    assert packed == 521_011_200
    assert bench.step_bytes(_fake_stack(30, 1)) == packed + tokens + outputs == 527_354_880


def test_recorded_traffic_belongs_to_the_committed_kernel(tmp_path, monkeypatch):
    # the committed GEMV sources are the ones the counters were taken on
    assert bench.measured_traffic() == bench.TRAFFIC["bytes_per_launch"]
    # any edit to them drops the figure
    for f in bench.TRAFFIC["sources"]:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)
    with open(tmp_path / bench.TRAFFIC["sources"][0], "a") as fh:
        fh.write("\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("argv", [[], ["--steps", "3", "--warmup", "1"]])
def test_defaults_are_one_gpu(monkeypatch, argv):
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    a = bench.parse()
    assert a.gpus == 1 and a.steps >= 1 and a.warmup >= 0


def test_recorded_mfma_busy_belongs_to_the_committed_gemm(tmp_path, monkeypatch):
    for n in (128, 4096):
        assert bench.measured_mfma_busy(n) == bench.GEMM_COUNTERS["mfma_busy"][n]
    for f in bench.GEMM_COUNTERS["sources"]:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)
    with open(tmp_path / bench.GEMM_COUNTERS["sources"][0], "a") as fh:
        fh.write("\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_mfma_busy() is None
