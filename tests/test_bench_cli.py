"""CPU: bench.py measures one GPU.  Asked for more (--gpus N > 1, or launched
as one rank of several), it prints one JSON line saying so and exits with
status 2 before touching a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_one_rank_of_several_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])
