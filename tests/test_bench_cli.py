"""bench.py's command-line contract that needs no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_recorded_traffic_matches_the_gemm_sources():
    """The committed per-launch traffic record names the GEMM sources it was
    measured on; bench.py reports it only while they are unchanged."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "gemm_i8_traffic.json")) as f:
        rec = json.load(f)
    # each field is rounded on its own
    assert abs(rec["traffic_bytes_per_launch"] - rec["fetch_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 1
    if rec["source_hash"] == bench.gemm_source_hash():
        assert bench.recorded_traffic(rec["workload"], rec["path"]) == rec["traffic_bytes_per_launch"]
    else:
        assert bench.recorded_traffic(rec["workload"], rec["path"]) is None
    assert bench.recorded_traffic("no such workload", rec["path"]) is None


def test_source_hash_ignores_comments_only():
    """The traffic record stays valid across comment and layout edits of the
    GEMM sources, and not across code edits."""
    sys.path.insert(0, ROOT)
    import bench
    src = "int f(int a) { // sum\n  return a + 1; /* one */ }\nconst char* s = \"// kept\";\n"
    base = bench._code_only(src)
    assert bench._code_only(src.replace("// sum", "// total").replace("/* one */", "")) == base
    assert bench._code_only(src.replace("a + 1", "a + 2")) != base
    assert bench._code_only(src.replace("\"// kept\"", "\"// gone\"")) != base
    assert "// kept" in base and "sum" not in base

