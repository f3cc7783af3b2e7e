"""Host logic of bench.py, without a GPU: the counter-record ingestion (scaling by the
calibration copy, per-launch and whole-call sums, utilisation fractions), the stale
record check, the roofline object of the JSON line, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

KERNELS = {  # launch -> a kernel symbol it matches
    "segment_summary": "void gtr::(anonymous namespace)::k_sum<1, 64, false, false>(gtr::GlaArgs)",
    "state_scan": "void gtr::(anonymous namespace)::k_scan_rows<16, 4>(float*)",
    "chunk_output": "void gtr::(anonymous namespace)::k_rows<1, 64, false, false>(gtr::GlaArgs)",
}
COPY = "__amd_rocclr_copyBuffer"


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kn, cn, v in rows:
            w.writerow({"Kernel_Name": kn, "Counter_Name": cn, "Counter_Value": v})


def _fixture(tmp_path):
    """Counter CSVs where FETCH_SIZE reads half of every byte and WRITE_SIZE all of
    them (KiB), two dispatches per kernel, and an SQ pass with known totals."""
    copy_kib = bench.COPY_BYTES / 1024
    fetch = [(COPY, "FETCH_SIZE", copy_kib / 2), (COPY, "FETCH_SIZE", 10.0)]
    write = [(COPY, "WRITE_SIZE", copy_kib), (COPY, "WRITE_SIZE", 5.0)]
    sq = []
    true_bytes = {"segment_summary": (100e6, 8e6), "state_scan": (9e6, 9e6),
                  "chunk_output": (160e6, 25e6)}
    for name, kn in KERNELS.items():
        fb, wb = true_bytes[name]
        for _ in range(2):  # two dispatches, the same counts
            fetch.append((kn, "FETCH_SIZE", fb / 2 / 1024))
            write.append((kn, "WRITE_SIZE", wb / 1024))
        c = {"SQ_WAVES": 2000, "SQ_INSTS_VALU": 4000 * 2000, "SQ_INSTS_MFMA": 100 * 2000,
             "SQ_INSTS_VALU_TRANS_F32": 50 * 2000, "SQ_INSTS_LDS": 300 * 2000,
             # busy 1000 cycles per XCD; MFMA busy a quarter of 1024 SIMDs' cycles,
             # VALU active half of 256 CUs' cycles
             "GRBM_GUI_ACTIVE": 1000 * bench.XCD_COUNT,
             "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1000 * bench.CU_COUNT * bench.SIMDS_PER_CU,
             "SQ_ACTIVE_INST_VALU": 0.5 * 1000 * bench.CU_COUNT, "SQ_BUSY_CYCLES": 1234}
        for cn, v in c.items():
            sq.append((kn, cn, v))
    paths = [str(tmp_path / n) for n in ("fetch.csv", "write.csv", "sq.csv")]
    for p, rows in zip(paths, (fetch, write, sq)):
        _csv(p, rows)
    return paths, true_bytes


def test_ingest_counters_scales_by_the_calibration_copy(tmp_path):
    paths, true_bytes = _fixture(tmp_path)
    out = bench.ingest_counters(*paths, "mixer_2048", "mfma", bench.LAUNCH_NAMES["mfma"],
                                out_dir=str(tmp_path))
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    for name, (fb, wb) in true_bytes.items():
        rec = out["launches"][name]
        assert rec["fetch_bytes"] == pytest.approx(fb, rel=1e-6)
        assert rec["write_bytes"] == pytest.approx(wb, rel=1e-6)
        assert rec["valu_insts_per_wave"] == 4000 and rec["mfma_insts_per_wave"] == 100
        assert rec["mfma_busy_frac"] == pytest.approx(0.25)
        assert rec["valu_busy_frac"] == pytest.approx(0.5)
    assert out["call_fetch_bytes"] == pytest.approx(sum(f for f, _ in true_bytes.values()), rel=1e-6)
    assert out["call_write_bytes"] == pytest.approx(sum(w for _, w in true_bytes.values()), rel=1e-6)
    # written where asked, with the sources hash of this tree
    rec = json.load(open(tmp_path / "counters_mfma_mixer_2048.json"))
    assert rec["sources_hash"] == bench.kernel_sources_hash()
    assert bench.counters_record("mfma", "mixer_2048", out_dir=str(tmp_path)) is not None


def test_stale_counter_record_is_ignored(tmp_path):
    paths, _ = _fixture(tmp_path)
    bench.ingest_counters(*paths, "mixer_2048", "mfma", bench.LAUNCH_NAMES["mfma"],
                          out_dir=str(tmp_path))
    p = tmp_path / "counters_mfma_mixer_2048.json"
    rec = json.load(open(p))
    rec["sources_hash"] = "0" * 16  # taken from other kernels
    json.dump(rec, open(p, "w"))
    assert bench.counters_record("mfma", "mixer_2048", out_dir=str(tmp_path)) is None


def test_ingest_needs_one_kernel_per_launch(tmp_path):
    paths, _ = _fixture(tmp_path)
    with pytest.raises(SystemExit, match="expected one kernel"):
        bench.ingest_counters(*paths, "mixer_2048", "fast", bench.LAUNCH_NAMES["fast"],
                              out_dir=str(tmp_path))


def test_roofline_record():
    names = bench.LAUNCH_NAMES["mfma"]
    comp, us, launch = 176_161_024, 80.0, [27.0, 10.0, 44.0]
    cr = {"launches": {"segment_summary": {"bytes": 1, "mfma_busy_frac": 0.1},
                       "state_scan": {"bytes": 2, "mfma_busy_frac": 0.0},
                       "chunk_output": {"bytes": 190_000_000, "mfma_busy_frac": 0.2,
                                        "valu_busy_frac": 0.4}},
          "call_bytes": 330_000_000}
    r = bench.roofline_record(comp, us, launch, names, cr, 1e12)
    assert r["kernel"] == "chunk_output" and r["kernel_us"] == 44.0
    assert r["achieved"] == pytest.approx(comp / 44e-6 / 1e9, abs=0.1)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS, abs=1e-4)
    assert r["whole_call_frac"] == pytest.approx(comp / 80e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=1e-4)
    assert r["traffic"] == 190_000_000 and r["whole_call"]["traffic"] == 330_000_000
    assert r["mfma_util"]["measured_kernel"] == 0.2 and r["valu_busy_kernel"] == 0.4
    # busy-cycle weighted over the launches
    assert r["mfma_util"]["measured_call"] == pytest.approx((0.1 * 27 + 0.2 * 44) / 81, abs=1e-4)
    assert r["mfma_util"]["algorithmic_call"] == pytest.approx(1e12 / 80e-6 / 1e12 / 2500, abs=1e-5)
    # no counter record: measured fields are null, never invented
    r = bench.roofline_record(comp, us, launch, names, None, 1e12)
    assert r["traffic"] is None and r["whole_call"]["traffic"] is None
    assert r["mfma_util"]["measured_kernel"] is None and r["mfma_util"]["measured_call"] is None


def test_bench_runs_on_one_gpu_only():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_launch_names_follow_the_launch_count():
    assert bench.launch_names("mfma", 3) == ["segment_summary", "state_scan", "chunk_output"]
    # the output kernel folds the incoming states itself: no scan launch
    assert bench.launch_names("mfma", 2) == ["segment_summary", "chunk_output"]
    assert bench.launch_names("fast", 1) == ["fast_single_launch"]
    with pytest.raises(SystemExit, match="launches"):
        bench.launch_names("mfma", 1)
    with pytest.raises(SystemExit, match="launches"):
        bench.launch_names("serial", 2)  # the token-serial path always scans


def test_ingest_without_the_scan_launch(tmp_path):
    paths, true_bytes = _fixture(tmp_path)
    for p in paths:  # the same record with the scan kernel's rows taken out
        rows = [r for r in csv.DictReader(open(p)) if "scan" not in r["Kernel_Name"]]
        _csv(p, [(r["Kernel_Name"], r["Counter_Name"], r["Counter_Value"]) for r in rows])
    names = bench.present_launches(paths[0], "mfma")
    assert names == ["segment_summary", "chunk_output"]
    out = bench.ingest_counters(*paths, "mixer_2048", "mfma", names, out_dir=str(tmp_path))
    assert set(out["launches"]) == {"segment_summary", "chunk_output"}
    assert out["call_fetch_bytes"] == pytest.approx(
        true_bytes["segment_summary"][0] + true_bytes["chunk_output"][0], rel=1e-6)
    # a required launch that is missing is still an error
    assert bench.present_launches(paths[0], "fast") == ["fast_single_launch"]
    with pytest.raises(SystemExit, match="expected one kernel"):
        bench.ingest_counters(*paths, "mixer_2048", "fast", ["fast_single_launch"],
                              out_dir=str(tmp_path))
