"""Host-side checks of bench.py's bookkeeping (no GPU):
* an HBM-traffic record in profiles/traffic.json is used only for the kernel
  code it was measured on (comments and layout aside);
* the rocprofv3 summary sums a counter's rows (one per hardware instance)
  within a dispatch and averages over dispatches;
* a request for several GPUs is refused.
"""
import json
import os
import shutil
import sqlite3
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _sources(tmp_path, monkeypatch):
    d = str(tmp_path / "csrc")
    shutil.copytree(bench.CSRC, d)
    monkeypatch.setattr(bench, "CSRC", d)
    return d


def test_source_hash_ignores_comments_and_layout_not_code(tmp_path, monkeypatch):
    d = _sources(tmp_path, monkeypatch)
    h_norm, h_core = bench.kernel_source_hash("prefill_norm"), bench.kernel_source_hash("prefill_core")
    p = os.path.join(d, "norm.hip")
    text = open(p).read()
    open(p, "w").write("// a comment\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n") + "\n")
    assert bench.kernel_source_hash("prefill_norm") == h_norm
    open(p, "w").write(text + "\nint gdn_one_more_symbol;\n")
    assert bench.kernel_source_hash("prefill_norm") != h_norm
    assert bench.kernel_source_hash("prefill_core") == h_core        # another kernel's record
    h = os.path.join(d, "gdn_device.h")
    open(h, "a").write("\nconstexpr int gdn_one_more_constant = 1;\n")
    assert bench.kernel_source_hash("prefill_core") != h_core        # a shared header: every record


def test_traffic_record_used_only_for_matching_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("prefill_norm") is None            # no file
    (tmp_path / "traffic.json").write_text("{not json")
    assert bench.measured_traffic("prefill_norm") is None            # unreadable
    rec = {"kernels": {
        "prefill_norm": {"fetch_bytes": 100.0, "write_bytes": 50.0,
                         "source_sha256": bench.kernel_source_hash("prefill_norm")},
        "prefill_prep": {"fetch_bytes": 7.0, "write_bytes": 7.0, "source_sha256": "0" * 64},
    }}
    (tmp_path / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("prefill_norm") == 150
    assert bench.measured_traffic("prefill_prep") is None            # measured on other code
    assert bench.measured_traffic("decode_b1") is None               # never measured


def test_committed_traffic_records_name_known_kernels():
    with open(os.path.join(bench.PROFILES, "traffic.json")) as f:
        rec = json.load(f)["kernels"]
    assert set(rec) <= set(bench.TRAFFIC_SOURCES)
    for k, v in rec.items():
        assert v["fetch_bytes"] > 0 and v["write_bytes"] > 0, k
        assert len(v["source_sha256"]) == 64, k


def test_summary_sums_instances_within_a_dispatch(tmp_path):
    db = str(tmp_path / "pmc.db")
    c = sqlite3.connect(db)
    c.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text, value real)")
    name = "void gdn::(anonymous namespace)::norm_kernel<gdn::bf16_t, true>(gdn::NormParams, int)"
    rows = [(name, 1, "FETCH_SIZE", 10.0), (name, 1, "FETCH_SIZE", 20.0), (name, 2, "FETCH_SIZE", 40.0),
            (name, 1, "WRITE_SIZE", 5.0)]
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    c.commit()
    c.close()
    lines = bench.summarize_rocprof(db).splitlines()
    fetch = [l for l in lines if "FETCH_SIZE" in l]
    assert len(fetch) == 1 and fetch[0].startswith("gdn::norm_kernel<gdn::bf16_t, true>")
    assert fetch[0].split()[-2:] == ["2", "35.0"]                   # (10 + 20 + 40) / 2 dispatches
    assert [l for l in lines if "WRITE_SIZE" in l][0].split()[-2:] == ["1", "5.0"]


def test_summary_of_a_kernel_trace(tmp_path):
    db = str(tmp_path / "trace.db")
    c = sqlite3.connect(db)
    c.execute("create table kernels (name text, grid_x int, grid_y int, workgroup_x int, duration int)")
    name = "void gdn::(anonymous namespace)::chunk_state_kernel<(gdn::Prec)1, gdn::bf16_t, true, false>(gdn::PrefillParams, long)"
    c.executemany("insert into kernels values (?, ?, ?, ?, ?)", [(name, 98304, 1, 512, 2000), (name, 98304, 1, 512, 4000)])
    c.commit()
    c.close()
    row = [l for l in bench.summarize_rocprof(db).splitlines() if "chunk_state" in l][0]
    assert row.startswith("gdn::chunk_state_kernel<BF16X3, gdn::bf16_t, true, false>")
    assert row.split()[-4:] == ["512", "2", "3.00", "2.00"]          # wg, calls, avg and min in us


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
