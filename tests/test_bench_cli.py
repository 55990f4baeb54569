"""bench.py's command line on the CPU: the one-GPU contract.

The library runs on one GPU; rows are independent, so a run on several GPUs
would be the one-GPU throughput per shard.  bench.py therefore refuses
--gpus N for N != 1 with a message and exit status 2, before it touches a
GPU, and the same holds under a multi-process launcher's environment.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120,
                          env=dict(os.environ, **(env or {})))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run(["--gpus", n])
        assert r.returncode == 2, r.stderr
        assert "one GPU only" in r.stderr
        assert r.stdout == ""


def test_refused_under_a_launcher_environment_too():
    r = _run(["--gpus", "4"], env={"RANK": "1", "LOCAL_RANK": "1", "WORLD_SIZE": "4",
                                   "MASTER_ADDR": "127.0.0.1", "MASTER_PORT": "29511"})
    assert r.returncode == 2, r.stderr
    assert r.stdout == ""
