"""bench.py's command-line contract on the host: it measures one GPU only, so a request for more
GPUs (flag or torchrun environment) exits with status 2 and a message, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
