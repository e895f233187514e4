"""bench.py's contract on the host: a run on more than one GPU exits with a
message before any device work (the bench measures one GPU); the sweep's
workload list is checked; the stored counter traffic belongs to the AdamW
sources in the tree."""
import json
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


def test_sweep_rejects_unknown_workloads():
    r = _run(["--configs", "1"])
    assert r.returncode == 2 and "--configs takes workloads 2 3 4 5" in r.stderr, r.stderr
    assert r.stdout == ""


def test_traffic_record_matches_the_kernel_sources():
    """The stored counter traffic of the headline workload belongs to the
    AdamW sources in the tree: the bench reports it only while their hash
    matches, so a stale record would silently turn roofline.traffic null."""
    sys.path.insert(0, ROOT)
    import bench
    path = bench.traffic_file("gpt-13b-nd1-rank0")
    with open(path) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
    assert bench.load_traffic("gpt-13b-nd1-rank0", 12_848_143_360) is not None
