"""bench.py's command line, without a GPU: more than one GPU is refused with a message, and a
host with no visible GPU is refused too (no CPU fallback is ever timed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_visible_gpu_is_refused():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible here")
    r = _run(["--steps", "1", "--warmup", "0"])
    assert r.returncode == 1
    assert "no GPU" in r.stderr
    assert r.stdout == ""
