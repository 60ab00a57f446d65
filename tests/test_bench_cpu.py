"""bench.py's host-side contract, without a GPU: it refuses more than one
GPU, fails loudly when no GPU is visible, and reports HBM traffic from a
committed counter summary only while that summary's kernel-source hash
matches the sources."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "no GPU" in r.stderr and r.stdout == ""


def test_traffic_is_read_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    src = bench.kernel_source_hash(["zr_rs.hip", "zr_fold.hpp", "zr_device.hpp"])
    (tmp_path / "k.counters.txt").write_text(
        "# a summary\nkernel_source_sha256_16 = %s\nhbm_bytes_per_launch = 12345.0\n"
        "algorithmic_bytes_per_launch = 12000\n" % src)
    assert bench.read_traffic("k.counters.txt", src, 12000) == 12345
    assert bench.read_traffic("k.counters.txt", "0" * 16, 12000) is None   # kernel changed since
    assert bench.read_traffic("k.counters.txt", src, 14400) is None   # another workload's bytes
    assert bench.read_traffic("missing.txt", src, 12000) is None
    (tmp_path / "bad.counters.txt").write_text("kernel_source_sha256_16 = %s\n" % src)
    assert bench.read_traffic("bad.counters.txt", src, 12000) is None      # no byte count
    (tmp_path / "old.counters.txt").write_text(
        "kernel_source_sha256_16 = %s\nhbm_bytes_per_launch = 12345.0\n" % src)
    assert bench.read_traffic("old.counters.txt", src, 12000) is None      # no byte model


def test_committed_counter_summaries_carry_what_the_bench_reads():
    names = [n for n in os.listdir(bench.PROFILES) if n.endswith(".counters.txt")]
    assert len(names) >= 4
    for n in names:
        kv = {}
        for line in open(os.path.join(bench.PROFILES, n)):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        assert len(kv.get("kernel_source_sha256_16", "")) == 16, n
        assert any(k.startswith("hbm_bytes_per_") for k in kv), n
        assert any(k.startswith("algorithmic_bytes_per_") for k in kv), n
        assert "rocprofv3" in open(os.path.join(bench.PROFILES, n)).read(), n  # the command that made it
