"""bench.py's host-side contract, on the CPU: one GPU only, a clear refusal
without a GPU, and the command line of the per-workload child processes."""

import argparse
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and
                    os.path.exists("/dev/kfd"), reason="a GPU may be present")
def test_no_gpu_is_refused_without_spawning():
    r = run_bench()
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_child_command_line(monkeypatch):
    import bench
    seen = {}

    class Done:
        returncode = 0
        stdout = '# noise\n{"x": 1}\n'

    def fake_run(cmd, **kw):
        seen["cmd"] = cmd
        return Done()

    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    a = argparse.Namespace(workload="opt13b", steps=7, warmup=2, cpu_seconds=3.0,
                           partition_size=512, no_fuse=True, no_cpu_baseline=False,
                           no_translation=True)
    assert bench.run_child(a, "long_gqa") == {"x": 1}
    cmd = seen["cmd"]
    assert cmd[0] == sys.executable and cmd[1].endswith("bench.py")
    i = cmd.index("--child")
    assert cmd[i + 1] == "long_gqa"
    for flag, val in (("--workload", "opt13b"), ("--steps", "7"), ("--warmup", "2"),
                      ("--partition-size", "512")):
        assert cmd[cmd.index(flag) + 1] == val
    assert "--no-fuse" in cmd and "--no-translation" in cmd
    assert "--no-cpu-baseline" not in cmd


def test_cpu_baseline_legs_on_the_host():
    """The CPU baseline's two legs (one thread; one process per core of the
    host share) run the oracle on a sample of a batch built on the CPU."""
    import dataclasses
    import types
    import torch
    import bench
    from paged_kv_cache_311_amd import workloads as wl
    w = dataclasses.replace(wl.WORKLOADS["opt13b"], num_seqs=6, num_heads=4, num_kv_heads=4,
                            lengths=("uniform", 1, 200), max_len=200)
    b = wl.make_batch(w, 5, "cpu")
    st = types.SimpleNamespace(w=w, b=b, torch=torch)
    r = bench.cpu_baseline(st, 0.3)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16 and r["cores"] == min(len(os.sched_getaffinity(0)), 16)
    assert r["single_thread"]["cores"] == 1 and r["single_thread"]["value"] > 0


def test_unique_bytes_count_shared_blocks_once():
    import dataclasses
    import numpy as np
    import bench
    from paged_kv_cache_311_amd import workloads as wl
    w = dataclasses.replace(wl.WORKLOADS["opt13b"], num_kv_heads=2, head_size=64)
    per_token = 2 * 2 * 64 * 2
    # two sequences share block 7 (full); each has a private last block
    tables = np.array([[7, 3, -1], [7, 5, 9]], np.int32)
    lens = np.array([20, 40])
    assert bench.kv_unique_bytes(w, tables, lens) == (16 + 4 + 16 + 8) * per_token
    assert bench.kv_bytes(w, lens) == 60 * per_token
