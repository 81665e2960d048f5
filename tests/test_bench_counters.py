"""CPU tests of bench.py's counter arithmetic on small rocprofv3-shaped SQLite files:
the per-launch HBM traffic it records (each counter divided by what the same
counter reads for a plain copy of known size) and the kernel-time summary."""
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counters_db(path, rows):
    """rows: (dispatch_id, kernel_name, counter_name, value, duration_ns)"""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (dispatch_id integer, kernel_name text, "
              "counter_name text, value real, duration integer)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    c.commit()
    c.close()


def test_record_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    gemm = "void tabit::(anonymous namespace)::gemm_i8_kernel<256, 256, 4, 4, 128, 2, 1, false>(...)"
    # a warm-up dispatch first; the record takes the last two gemm dispatches only
    _counters_db(str(tmp_path / "f" / "a.db"),
                 [(1, gemm, "FETCH_SIZE", 99999.0, 1000), (2, "quant_int8_kernel", "FETCH_SIZE", 7.0, 10),
                  (3, gemm, "FETCH_SIZE", 1000.0, 1000), (4, gemm, "FETCH_SIZE", 3000.0, 1000)])
    _counters_db(str(tmp_path / "w" / "a.db"),
                 [(1, gemm, "WRITE_SIZE", 5.0, 1000), (3, gemm, "WRITE_SIZE", 400.0, 1000),
                  (4, gemm, "WRITE_SIZE", 600.0, 1000)])
    cal = 1 << 20   # a 1 MiB copy that FETCH_SIZE reads as half its bytes, WRITE_SIZE as all
    _counters_db(str(tmp_path / "cf" / "a.db"),
                 [(1, "fill", "FETCH_SIZE", 3.0, 10), (2, "copy", "FETCH_SIZE", 512.0, 10)])
    _counters_db(str(tmp_path / "cw" / "a.db"),
                 [(1, "fill", "WRITE_SIZE", 64.0, 10), (2, "copy", "WRITE_SIZE", 1024.0, 10)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                         str(tmp_path / "cw"), cal, 2, "wl", "masked")
    rec = json.loads(out.read_text())
    assert rec["fetch_factor"] == 0.5 and rec["write_factor"] == 1.0
    assert rec["dispatches"] == 2
    # mean of 1000 and 3000 KiB, divided by 0.5; mean of 400 and 600 KiB
    assert rec["fetch_bytes_per_launch"] == 4000 * 1024
    assert rec["write_bytes_per_launch"] == 500 * 1024
    assert rec["traffic_bytes_per_launch"] == 4500 * 1024
    assert rec["source_hash"] == bench.gemm_source_hash()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.recorded_traffic("wl", "masked") == 4500 * 1024
    assert bench.recorded_traffic("wl", "bitserial") is None


def test_summarize_rocpd_kernel_table(tmp_path, capsys):
    p = tmp_path / "t" / "x.db"
    os.makedirs(p.parent)
    c = sqlite3.connect(str(p))
    c.execute("create table kernels (name text, duration integer)")
    c.executemany("insert into kernels values (?, ?)",
                  [("void tabit::(anonymous namespace)::gemm_i8_kernel<1>(int)", 30000),
                   ("void tabit::(anonymous namespace)::gemm_i8_kernel<1>(int)", 10000),
                   ("quant_int8_kernel<0>(float)", 20000)])
    c.commit()
    c.close()
    bench.summarize_rocpd(str(tmp_path / "t"))
    lines = capsys.readouterr().out.splitlines()
    assert lines[0].split() == ["kernel", "calls", "avg_us", "total_ms", "pct"]
    g = lines[1].split()
    assert g[0] == "gemm_i8_kernel<1>" and g[1:] == ["2", "20.00", "0.04", "66.7"]
    q = lines[2].split()
    assert q[0] == "quant_int8_kernel<0>" and q[1:] == ["1", "20.00", "0.02", "33.3"]
