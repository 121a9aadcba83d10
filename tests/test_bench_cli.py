"""bench.py's command line, on the CPU: it measures one GPU only, so a request
for more (by flag or by a launcher's WORLD_SIZE) ends at once with a message
and a non-zero status, before torch is imported or a device is touched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=60)


@pytest.mark.parametrize("args,env", [
    (["--gpus", "2"], None),
    (["--gpus", "8", "--steps", "3"], None),
    (["--gpus", "1"], {"WORLD_SIZE": "2"}),
])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
    assert not r.stdout.lstrip().startswith("{")   # no result line


def test_help_lists_the_contract_flags():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--mode"):
        assert flag in r.stdout
