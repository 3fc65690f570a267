"""Host logic of the benchmark's counter records: the code hash ignores comments and white space
and follows any change of code."""
import json
import os
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hash_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    rel = os.path.relpath(p, ROOT)
    return bench.code_sha256([rel])


def test_code_hash_ignores_comments_and_space(tmp_path):
    a = _hash_of(tmp_path, "int f(int x) {\n  return x + 1;  // add one\n}\n")
    b = _hash_of(tmp_path, "/* header */\nint f(int x)\n{\n    return x + 1;\n}\n// trailing\n")
    assert a == b


def test_code_hash_follows_code(tmp_path):
    a = _hash_of(tmp_path, "int f(int x) { return x + 1; }")
    b = _hash_of(tmp_path, "int f(int x) { return x + 2; }")
    assert a != b


@pytest.mark.parametrize("record", ["sparse_decode_traffic.json", "prefill_attention_traffic.json"])
def test_traffic_records_are_well_formed(record):
    rec = json.load(open(os.path.join(ROOT, "profiles", record)))
    for key in ("kernel", "workload", "sources", "code_sha256", "read_bytes_per_launch",
                "write_bytes_per_launch", "scale", "traffic_bytes_per_launch"):
        assert key in rec
    assert rec["traffic_bytes_per_launch"] == pytest.approx(
        rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"], abs=2)
    for f in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, f)), f


def test_more_than_one_gpu_exits_with_a_message():
    """The benchmark measures one GPU: --gpus above 1 exits with status 2 and says so."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
