"""The benchmark's command-line contract on a machine without a GPU: it
measures one GPU and says so, with a nonzero exit, when asked for more."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr, r.stderr
    assert r.stdout.strip() == "", r.stdout


def test_a_multi_rank_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr, r.stderr
