"""bench.py host logic (no GPU): the refusal of multi-GPU runs, the traffic
figure taken from a committed rocprofv3 summary only while the summary's
source digest matches the source, and the summary writer on a small
hand-made rocprofv3 output."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_traffic_follows_the_source_digest(monkeypatch):
    path = os.path.join(ROOT, "profiles", "attention_sink_decode.md")
    text = open(path).read()
    digest = text.split("`")[1]  # the first code span is the source digest
    want = float([l for l in text.splitlines() if l.startswith("traffic_bytes_per_attention_call:")][0]
                 .split(":")[1])
    monkeypatch.setattr(bench, "source_digest", lambda src=bench.ATTN_SOURCE: digest)
    assert bench.committed_traffic("sink_decode") == want
    # a source that changed since the counters were taken: no traffic figure
    monkeypatch.setattr(bench, "source_digest", lambda src=bench.ATTN_SOURCE: "0" * 16)
    assert bench.committed_traffic("sink_decode") is None
    # no summary for the workload
    assert bench.committed_traffic("no_such_workload") is None


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_summary_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    """A split kernel (two dispatches), an appending split and a fold: the
    summary's traffic per call is each counter's mean per dispatch, scaled by
    what the same counter reads for a copy of known size, summed over the
    plain call's kernels (the appending split is the step's, not the call's).
    The summary goes to a temporary tree, not to the committed one."""
    d = tmp_path / "wl"
    for sub in ("stats", "fetch", "write", "copy_fetch", "copy_write"):
        (d / sub).mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    split = "void pkv::attn_parallel<64, 1, false, false, 0, false, false, false>(pkv::AttnParams)"
    append = "void pkv::attn_parallel<64, 1, false, true, 0, false, false, false>(pkv::AttnParams)"
    fold = "void pkv::attn_fold<64, 1, false>(pkv::AttnParams)"
    copy = "__amd_rocclr_copyBuffer"
    _write_csv(d / "stats" / "s_kernel_stats.csv",
               [{"Name": split, "Calls": 2, "TotalDurationNs": 90000, "AverageNs": 45000, "Percentage": 90.0,
                 "MinNs": 44000, "MaxNs": 46000},
                {"Name": fold, "Calls": 2, "TotalDurationNs": 10000, "AverageNs": 5000, "Percentage": 10.0,
                 "MinNs": 4900, "MaxNs": 5100}])

    def counter_rows(name, counter, values):
        return [{"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v} for v in values]
    # KiB per dispatch; the 2 MiB copy counts 1024 KiB of FETCH_SIZE (so x 2.0)
    # and 2048 KiB of WRITE_SIZE (x 1.0)
    _write_csv(d / "fetch" / "f_counter_collection.csv",
               counter_rows(split, "FETCH_SIZE", [1000.0, 1200.0]) + counter_rows(append, "FETCH_SIZE", [999.0])
               + counter_rows(fold, "FETCH_SIZE", [50.0]))
    _write_csv(d / "write" / "w_counter_collection.csv",
               counter_rows(split, "WRITE_SIZE", [10.0, 30.0]) + counter_rows(append, "WRITE_SIZE", [99.0])
               + counter_rows(fold, "WRITE_SIZE", [4.0]))
    _write_csv(d / "copy_fetch" / "c_counter_collection.csv", counter_rows(copy, "FETCH_SIZE", [1024.0]))
    _write_csv(d / "copy_write" / "c_counter_collection.csv", counter_rows(copy, "WRITE_SIZE", [2048.0]))
    (d / "copy.json").write_text('{"copy_bytes": 2097152}')
    assert bench.summarize_profile(str(d), "unit_case", ["cmd one", "cmd two"]) == 0
    text = (tmp_path / "profiles" / "attention_unit_case.md").read_text()
    want = (1100 * 2.0 + 20 * 1.0) * 1024 + (50 * 2.0 + 4 * 1.0) * 1024
    line = [l for l in text.splitlines() if l.startswith("traffic_bytes_per_attention_call:")][0]
    assert float(line.split(":")[1]) == pytest.approx(want)
    assert f"`{bench.source_digest()}`" in text
    assert "    cmd one" in text and "| attn_parallel<64, 1, false, false, 0, false, false, false> | 2 | 45.00 |" in text
    assert not os.path.exists(os.path.join(ROOT, "profiles", "attention_unit_case.md"))
