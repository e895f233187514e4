"""bench.py's contract on the host: a run on more than one GPU exits with a
message before any device work (the bench measures one GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=e, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None),
                      ([], {"WORLD_SIZE": "4"})):
        r = _run(args, env)
        assert r.returncode == 2, (args, r.returncode, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""
