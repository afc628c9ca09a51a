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
    sha = bench.kernel_source_hash("k_gateup")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel: sha)
    assert bench.measured_traffic("k_gateup", "w") is None          # no summary
    _summary(tmp_path, "k_gateup", "w", sha)
    assert bench.measured_traffic("k_gateup", "w") == 123456.0
    _summary(tmp_path, "k_gateup", "w", "0" * 64)                     # sources changed
    assert bench.measured_traffic("k_gateup", "w") is None
    _summary(tmp_path, "k_gateup", "w", sha, traffic="not a number")
    assert bench.measured_traffic("k_gateup", "w") is None
    _summary(tmp_path, "k_other", "w", sha)                           # no source set
    assert bench.measured_traffic("k_other", "w") is None


def test_source_hash_covers_every_kernel_source():
    csrc = os.path.join(ROOT, "block_quantized_expert_amd", "csrc")
    # codec.hip (one-time packing and image build), measure.hip (the plain
    # read the kernels are compared with) and dense.hip (dense projections)
    # hold no kernel a traffic summary covers
    kernels = {f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp"))
               and f not in ("codec.hip", "measure.hip", "dense.hip")}
    covered = set()
    for k, names in bench.KERNEL_SOURCES.items():
        assert {"abi.hip", "rfpx_impl.hpp"} <= set(names), k
        covered |= set(names)
        assert len(bench.kernel_source_hash(k)) == 64
    assert kernels <= covered


def test_source_hash_is_per_kernel_family(tmp_path):
    """A change to the prefill source leaves the decode kernels' summaries
    valid, and the other way round."""
    import shutil
    src = os.path.join(ROOT, "block_quantized_expert_amd", "csrc")
    dst = tmp_path / "block_quantized_expert_amd" / "csrc"
    shutil.copytree(src, dst)
    base = {k: bench.kernel_source_hash(k, str(tmp_path)) for k in bench.KERNEL_SOURCES}
    with open(dst / "prefill.hip", "a") as fh:
        fh.write("\n// changed\n")
    after = {k: bench.kernel_source_hash(k, str(tmp_path)) for k in bench.KERNEL_SOURCES}
    assert after["k_gateup"] == base["k_gateup"] and after["k_down"] == base["k_down"]
    assert after["k_pf_gateup"] != base["k_pf_gateup"]
    with open(dst / "expert.hip", "a") as fh:
        fh.write("\n// changed\n")
    again = {k: bench.kernel_source_hash(k, str(tmp_path)) for k in bench.KERNEL_SOURCES}
    assert again["k_gateup"] != after["k_gateup"] and again["k_pf_down"] == after["k_pf_down"]


def test_expert_bytes_are_the_packed_matrices():
    lay = synth.gen_layer(synth.WORKLOADS[synth.TINY], 0, threads=2)
    for e in (0, lay.E):
        tot, gu = bench.expert_bytes(lay, e)
        sizes = []
        for m in range(3):
            rows, cols = lay.matrix_shape(m)
            sizes.append(rows * cols // 32 * {2: 10, 3: 14, 4: 17}[int(lay.fmts[e][m])])
        assert gu == sizes[0] + sizes[1] and tot == sum(sizes)
