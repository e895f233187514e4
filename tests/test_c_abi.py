"""The C ABI from a plain C caller: tests/c_client.c is compiled with gcc as
strict C99 against include/zero.h, linked to the built library, and run with
no Python or torch in the process.  Its planner results must equal the
oracle's, its memory figures must round to the pages' table, and the device
entry points must reject bad arguments on the host with ZERO_EINVAL."""
import json
import os
import shutil
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_sharded_mixed_grads_amd")
LIB = os.path.join(PKG, "libzero_mi355x.so")


@pytest.fixture(scope="module")
def client_output(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    if not os.path.exists(LIB):
        pytest.skip("the library has not been built")
    exe = str(tmp_path_factory.mktemp("c_abi") / "c_client")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_client.c"),
                    f"-L{PKG}", "-l:libzero_mi355x.so", f"-Wl,-rpath,{PKG}", "-o", exe],
                   check=True)
    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env,
                         timeout=60).stdout
    lines = {}
    for line in out.splitlines():
        key, *rest = line.split()
        lines.setdefault(key, []).append(rest)
    return lines


def test_partition_matches_oracle(client_output):
    st, b, e = client_output["partition"][0]
    assert int(st) == 0
    assert (int(b), int(e)) == oracle.partition(100291305472, 400, 399)


def test_mem_bytes_match_oracle_and_page_table(client_output):
    table = json.load(open(os.path.join(ROOT, "tests", "golden", "zero_dp_memory_table.json")))
    printed = table["rows"]["64"]
    for stage_s, st, nbytes in client_output["mem_bytes"]:
        stage = int(stage_s)
        assert int(st) == 0
        assert int(nbytes) == oracle.mem_bytes(stage, 7_500_000_000, 64, 12)
        gb = int(nbytes) / table["unit_bytes"]
        digits = len(printed[stage].split(".")[1]) if "." in printed[stage] else 0
        assert f"{gb:.{digits}f}" == printed[stage], (stage, gb)


def test_bucket_plan_matches_oracle(client_output):
    st, count, *segs = client_output["plan"][0]
    assert int(st) == 0
    got = [tuple(int(x) for x in s.split(":")) for s in segs]
    want = [(s.bucket, s.tensor, s.src_off, s.dst_off, s.len)
            for s in oracle.bucket_plan([1000, 37, 4096, 3, 2500], 1024, 500, 7000)]
    assert int(count) == len(want) and got == want


def test_state_layout_contract(client_output):
    st, *offs = client_output["layout"][0]
    assert int(st) == 0
    n, pool = 1_000_000, 1 << 30
    offs = [int(x) for x in offs]
    step = offs[1]
    assert offs == [i * step for i in range(5)]
    assert step % (2 << 20) == 0 and step >= 4 * n + 16 and 4 * step + 2 * n + 16 <= pool


def test_errors_are_reported_on_the_host(client_output):
    st, name, has_detail = client_output["error_partition"][0]
    assert (int(st), name, int(has_detail)) == (1, "ZERO_EINVAL", 1)
    assert client_output["error_adam"][0] == ["1", "ZERO_EINVAL"]
    assert client_output["error_flatten"][0] == ["1", "ZERO_EINVAL"]
