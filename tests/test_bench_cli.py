"""bench.py's command line on the CPU: it measures one GPU only, so more than one
GPU (by flag or by a launcher's WORLD_SIZE) ends with status 2 and says so, and
without a GPU it ends with status 2 before timing anything."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    p = _run(args, env)
    assert p.returncode == 2, (p.returncode, p.stderr)
    assert "one MI355X only" in p.stderr
    assert p.stdout.strip() == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the exit without a GPU")
def test_no_gpu_exits_before_timing():
    p = _run(["--gpus", "1"])
    assert p.returncode == 2, (p.returncode, p.stderr)
    assert "needs a GPU" in p.stderr
    assert p.stdout.strip() == ""
