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
