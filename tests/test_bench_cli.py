"""bench.py's command-line contract that holds without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode != 0
    assert "--gpus 2" in r.stdout + r.stderr and "only --gpus 1 runs" in r.stdout + r.stderr


def test_multi_rank_launch_is_refused_too():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _bench(env=env)
    assert r.returncode != 0
    assert "only --gpus 1 runs" in r.stdout + r.stderr


def test_unknown_workload_is_rejected():
    r = _bench("--workload", "no_such_workload")
    assert r.returncode != 0
