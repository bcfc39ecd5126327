"""bench.py's command line on the host: a request for more than one GPU,
by flag or by the launcher's WORLD_SIZE, exits with status 2 and says why,
before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_bench_refuses_several_gpus_by_flag():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "asked for 2" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_several_ranks_by_world_size():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "asked for 4" in r.stderr
