"""bench.py's command line on the CPU: more than one GPU is refused with a
message (this build runs on one GPU; the sharded path is design only), and
unknown workloads are refused before any GPU work."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, env=e, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in msg and "one GPU" in msg["error"]


def test_world_size_above_one_is_refused():
    r = _run(env={"WORLD_SIZE": "2"})
    assert r.returncode != 0 and "error" in json.loads(r.stdout.strip().splitlines()[-1])


def test_unknown_workload_is_refused():
    r = _run("--workload", "c9")
    assert r.returncode != 0 and "unknown workload" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
