"""Host logic of the bench's counter summary: dispatches are attributed to
stages by the marker kernels around each call, averaged over calls, scaled by
the calibration copy, and recorded with the hash of the stage's sources (a
record whose sources no longer hash the same is ignored)."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
MARK = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<long>, std::array<char*, 1ul> >"


def write_csv(path, dispatches, counter):
    rows = [{"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
             "Counter_Value": val} for i, (name, val) in enumerate(dispatches, start=1)]
    rows = rows[1::2] + rows[0::2]   # the summary orders dispatches by id, not by file position
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        w.writerows(rows)


def dispatches(scale):
    """setup work, two calls of gemm_wgrad (one kernel each), two calls of the
    permute (two kernels each), then the calibration copy, as the counter pass
    brackets them.  The copy reads 2 x its size / scale in the counter's KiB."""
    d = [("setup_kernel", 999.0)]
    for v in (100.0, 120.0):
        d += [(MARK, 0.0), ("mx::k_gemm<false, true, false>", v * scale), (MARK, 0.0), ("randn", 5.0)]
    for v in (10.0, 30.0):
        d += [(MARK, 0.0), ("mx::k_route_hist", 1.0 * scale), ("mx::k_permute_tokens", v * scale), (MARK, 0.0)]
    d += [(MARK, 0.0), ("__amd_rocclr_copyBuffer", 2.0 * bench.CALIB_BYTES / 1024 / scale), (MARK, 0.0)]
    return d


LABELS = ["gemm_wgrad", "other", "gemm_wgrad", "other", "permute", "other", "permute", "other",
          "calibration", "other"]


def test_summary_attributes_by_marker(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fetch, dispatches(1.0), "FETCH_SIZE")
    write_csv(write, dispatches(2.0), "WRITE_SIZE")
    log = tmp_path / "pass.log"
    log.write_text("counter pass: progress\n" + json.dumps(
        {"counter_pass": {"labels": LABELS, "reps": 2,
                          "algorithmic_bytes": {"gemm_wgrad": 1.0e6, "permute": 5.0e4}}}) + "\n")
    out = tmp_path / "traffic.txt"
    bench.summarize_counters(str(fetch), str(write), str(log), out_path=str(out))
    rec = {}
    for line in out.read_text().splitlines():
        if line.startswith("stage="):
            kv = dict(f.split("=", 1) for f in line.split())
            rec[kv["stage"]] = kv
    assert set(rec) == {"gemm_wgrad", "permute"}
    # factors: copy size / the copy's reading (fetch 2x its size: 0.5; write 2x / 2 = 1x: 1.0)
    ff, fw = 0.5, 1.0
    assert float(rec["gemm_wgrad"]["fetch_bytes"]) == pytest.approx(110.0 * 1024 * ff, abs=1)
    assert float(rec["gemm_wgrad"]["write_bytes"]) == pytest.approx(220.0 * 1024 * fw, abs=1)
    assert float(rec["permute"]["fetch_bytes"]) == pytest.approx(21.0 * 1024 * ff, abs=1)
    assert rec["gemm_wgrad"]["source"] == "mxfp8_block_scaled_07_amd/csrc/gemm.hip"
    assert rec["permute"]["source"] == "mxfp8_block_scaled_07_amd/csrc/permute.hip"


def test_summary_rejects_a_marker_count_mismatch(tmp_path):
    fetch = tmp_path / "f.csv"
    write_csv(fetch, dispatches(1.0), "FETCH_SIZE")
    log = tmp_path / "pass.log"
    log.write_text(json.dumps({"counter_pass": {"labels": LABELS[:-1], "reps": 2, "algorithmic_bytes": {}}}) + "\n")
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(fetch), str(fetch), str(log), out_path=str(tmp_path / "t.txt"))


def test_traffic_record_ignored_when_sources_change(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    import hashlib
    digest = hashlib.sha256(b"kernel v1").hexdigest()
    tf = tmp_path / "traffic.txt"
    tf.write_text(f"stage=gemm_fwd source=k.hip sha256={digest} fetch_bytes=10 write_bytes=5 "
                  f"algorithmic_bytes=10 ratio=1.5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gemm_fwd")["bytes"] == 15.0
    src.write_text("kernel v2")
    assert bench.measured_traffic("gemm_fwd") is None


def test_stage_entry_fractions():
    """A stage's throughput against the spec peak (frac), the measured copy or
    MFMA-loop ceiling (frac_ceiling) and, for the row+col quantizes of plain
    tensors, the tile quantizer's access pattern (frac_pattern)."""
    work = {"gemm_flops": {"gemm_fwd": 2e12}, "bytes": {"quant_w": 4e9, "permute": 1e8}}
    ceil = {"hbm_copy_gbps": 5000.0, "quant_pattern_gbps": 4000.0, "mfma_mxfp8_tflops": 2500.0}
    e = bench.stage_entry("gemm_fwd", 1.0, work, ceil)           # 2e12 FLOP in 1 ms
    assert e == {"ms": 1.0, "tflops": 2000.0, "frac": 0.4, "frac_ceiling": 0.8}
    e = bench.stage_entry("quant_w", 1.0, work, ceil)            # 4e9 bytes in 1 ms
    assert e == {"ms": 1.0, "gbps": 4000.0, "frac": 0.5, "frac_ceiling": 0.8, "frac_pattern": 1.0}
    e = bench.stage_entry("permute", 2.0, work, ceil)
    assert e == {"ms": 2.0, "gbps": 50.0, "frac": 0.0063, "frac_ceiling": 0.01}
