"""bench.py's command-line contract on the CPU: it measures one GPU, and
asking for more exits before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = run(env=env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_lists_the_workloads():
    r = run("--help")
    assert r.returncode == 0
    for w in ("block", "batched", "stack", "sweep", "qpass", "tree"):
        assert w in r.stdout
