"""Host logic of bench.py (CPU): the one-GPU refusal, the lookup of
committed counter summaries and the algorithmic byte accounting."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def _summary(tmp, kernel, workload, sha, traffic="123456"):
    d = tmp / "profiles"
    d.mkdir(exist_ok=True)
    (d / f"{kernel}_{workload}_traffic.txt").write_text(
        "# comment = ignored\n"
        f"kernel = {kernel}\nworkload = {workload}\nsource_sha256 = {sha}\n"
        f"traffic_bytes_per_launch = {traffic}\n")


def test_measured_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: sha)
    assert bench.measured_traffic("k_gateup", "w") is None          # no summary
    _summary(tmp_path, "k_gateup", "w", sha)
    assert bench.measured_traffic("k_gateup", "w") == 123456.0
    _summary(tmp_path, "k_gateup", "w", "0" * 64)                     # sources changed
    assert bench.measured_traffic("k_gateup", "w") is None
    _summary(tmp_path, "k_gateup", "w", sha, traffic="not a number")
    assert bench.measured_traffic("k_gateup", "w") is None


def test_source_hash_covers_every_kernel_source():
    csrc = os.path.join(ROOT, "block_quantized_expert_amd", "csrc")
    # codec.hip (one-time packing and image build) and measure.hip (the plain
    # read the kernels are compared with) hold no kernel a traffic summary covers
    kernels = {f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp"))
               and f not in ("codec.hip", "measure.hip")}
    assert kernels <= set(bench.KERNEL_SOURCES)
    assert len(bench.kernel_source_hash()) == 64


def test_expert_bytes_are_the_packed_matrices():
    lay = synth.gen_layer(synth.WORKLOADS[synth.TINY], 0, threads=2)
    for e in (0, lay.E):
        tot, gu = bench.expert_bytes(lay, e)
        sizes = []
        for m in range(3):
            rows, cols = lay.matrix_shape(m)
            sizes.append(rows * cols // 32 * {2: 10, 3: 14, 4: 17}[int(lay.fmts[e][m])])
        assert gu == sizes[0] + sizes[1] and tot == sum(sizes)
