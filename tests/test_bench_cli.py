"""bench.py's contract on the command line, without a GPU: it measures one
GPU only and says so for any other count (before touching torch)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_a_multi_rank_launch_is_refused():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
