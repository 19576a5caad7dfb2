"""Host checks of the profile-record helpers (entropic_ot_attention_amd/profiling.py) on small
synthetic rocprofv3 CSV files: the traffic record scales each counter by its calibration copy,
the counter summary derives the busy fractions it documents, and the source hash follows the
step kernel's sources."""

import csv
import json
import os

import pytest

from entropic_ot_attention_amd import profiling as P

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, counter, value in rows:
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter, Counter_Value=value)
            w.writerow(r)


def test_traffic_record_scales_by_the_calibration_copy(tmp_path):
    calib = 1 << 20                    # the copy moves 1 MiB each way
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # the fetch counter reads half the true bytes, the write counter all of them; counters are
    # summed over the rows of one dispatch (one row per XCD here)
    _write(f, [(1, "neg_kernel", "FETCH_SIZE", 256.0), (1, "neg_kernel", "FETCH_SIZE", 256.0),
               (2, "sinkhorn_step_kernel<17>", "FETCH_SIZE", 100.0),
               (3, "sinkhorn_step_kernel<17>", "FETCH_SIZE", 300.0)])
    _write(w, [(1, "neg_kernel", "WRITE_SIZE", 1024.0),
               (2, "sinkhorn_step_kernel<17>", "WRITE_SIZE", 10.0),
               (3, "sinkhorn_step_kernel<17>", "WRITE_SIZE", 30.0)])
    rec = P.traffic_record(str(f), str(w), "sinkhorn_step_kernel", "neg_kernel", calib, "cmd", "wl")
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2.0)
    assert rec["write_bytes_per_launch"] == pytest.approx(20.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(rec["fetch_bytes_per_launch"] +
                                                   rec["write_bytes_per_launch"])
    assert rec["fetch_launches"] == 2 and rec["source_sha256"] == P.source_sha()
    json.dumps(rec)


def test_traffic_record_needs_both_kernels(tmp_path):
    f = tmp_path / "f.csv"
    _write(f, [(1, "neg_kernel", "FETCH_SIZE", 1.0)])
    with pytest.raises(RuntimeError):
        P.traffic_record(str(f), str(f), "sinkhorn_step_kernel", "neg_kernel", 1, "cmd", "wl")


def test_counter_summary_fractions(tmp_path):
    cyc = 240000.0                      # kernel cycles per XCD
    simd = 1024
    rows = [(1, "k", "GRBM_GUI_ACTIVE", cyc * 8), (1, "k", "SQ_WAVES", 1000.0),
            (1, "k", "SQ_INSTS_VALU", 5e6),
            (1, "k", "SQ_ACTIVE_INST_VALU", 0.5 * simd * cyc / 4),       # quad-cycle units
            (1, "k", "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * simd * cyc)]
    c = tmp_path / "c.csv"
    _write(c, rows)
    out = tmp_path / "c.md"
    P.counters_markdown([str(c)], str(out), "rocprofv3 --pmc ...")
    text = out.read_text()
    assert "| VALU busy | 0.500 |" in text
    assert "| MFMA busy | 0.250 |" in text
    assert "| SQ_INSTS_VALU per wave | 5000 |" in text
    assert "kernel cycles 240000 (100.0 us at 2.4 GHz)" in text


def test_memory_counter_summary(tmp_path):
    cyc = 100000.0                      # kernel cycles per XCD
    # two passes over two dispatches each; counters summed over the rows of one dispatch
    p1 = [(d, "k", c, v) for d in (1, 2) for c, v in
          (("GRBM_GUI_ACTIVE", cyc * 8), ("TCC_REQ_sum", 0.25 * 128 * cyc),
           ("TCC_HIT_sum", 0.9 * 0.25 * 128 * cyc), ("TCC_MISS_sum", 0.1 * 0.25 * 128 * cyc))]
    p2 = [(d, "k", c, v) for d in (1, 2) for c, v in
          (("GRBM_GUI_ACTIVE", cyc * 8), ("TCP_TOTAL_CACHE_ACCESSES_sum", 4e6),
           ("TCP_TCC_READ_REQ_sum", 1e6), ("TA_BUSY_avr", 0.4 * cyc), ("TA_BUSY_max", 0.6 * cyc),
           ("TCP_PENDING_STALL_CYCLES_sum", 0.2 * 256 * cyc))]
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    _write(a, p1)
    _write(b, p2)
    out = tmp_path / "m.md"
    P.memory_counters_markdown([str(a), str(b)], str(out), "rocprofv3 --pmc ...")
    text = out.read_text()
    assert "dispatches averaged per pass: 2; kernel cycles 100000" in text
    assert "| L2 requests per cycle | 32.0 (0.250 of the channels' rate) |" in text
    assert "| L2 requests per launch | 3.2e+06 (0.410 GB) |" in text
    assert "| L2 hit rate | 0.900 |" in text
    assert "| L1 hit rate (reads sent on to L2) | 0.750 |" in text
    assert "| address unit busy (mean CU) | 0.400 |" in text
    assert "| address unit busy (busiest CU) | 0.600 |" in text
    assert "| L1 pending-request stall per CU | 0.200 |" in text


def test_source_hash_follows_the_step_kernel_sources(tmp_path):
    paths = []
    for name in ("a.hip", "b.h"):
        p = tmp_path / name
        p.write_text(name)
        paths.append(str(p))
    h0 = P.source_sha(paths)
    (tmp_path / "a.hip").write_text("a.hip changed")
    assert P.source_sha(paths) != h0
    assert all(os.path.exists(p) for p in P.STEP_KERNEL_SOURCES)


def test_bench_band_entries_and_roofline_constants():
    """bench.py's per-launch work counts: the band size by brute force, the VALU ceiling (the fp32
    vector peak, 256 CUs x 4 SIMDs x 32 fma lanes x 2.4 GHz) with 7 issue slots per band entry, and
    the SIMD issue floor of the long workload's step launch (about 37.7 us)."""
    import bench
    for L in (0, 1, 2, 7, 64, 100):
        for h in (0, 1, 3, 50, 200):
            brute = sum(1 for i in range(L) for j in range(L) if abs(i - j) <= h)
            assert bench.band_entries(L, h) == brute
    assert bench.VALU_LANE_OPS_PER_S == pytest.approx(78.6432e12)     # 157.3 TFLOP/s / 2
    assert bench.SLOTS_PER_ENTRY_STEP == 7
    assert bench.tail_pass_flops_per_entry(2, 64) == 22 * 64
    assert bench.VJP_R2_FLOPS_PER_ENTRY_D == 4 + 2 + 8 + 6
    nnz = bench.band_entries(262144, 128) * 4
    cyc = nnz * (2 * bench.BF16_MFMA_CYCLES / 256 + bench.SLOTS_PER_ENTRY_STEP * bench.VALU_SLOT_CYCLES / 64)
    assert cyc / (bench.N_SIMD * bench.CLOCK_HZ) == pytest.approx(37.69e-6, rel=1e-3)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_kernel_busy_record(tmp_path):
    """The step-kernel counter record averages every dispatch of the named kernel over the
    passes and derives the busy fractions as the markdown summary does."""
    cyc = 240000.0
    p1, p2 = tmp_path / "p1.csv", tmp_path / "p2.csv"
    k = "sinkhorn_step_kernel<17>"
    _write(p1, [(1, k, "GRBM_GUI_ACTIVE", 8 * cyc), (1, k, "SQ_WAVES", 100.0),
                (1, k, "SQ_INSTS_VALU", 1000.0), (2, "other", "GRBM_GUI_ACTIVE", 1.0)])
    _write(p2, [(5, k, "GRBM_GUI_ACTIVE", 8 * cyc),
                (5, k, "SQ_ACTIVE_INST_VALU", 0.25 * 1024 * cyc / 4),
                (5, k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc)])
    rec = P.kernel_busy([str(p1), str(p2)], "sinkhorn_step_kernel")
    assert rec["cycles"] == pytest.approx(cyc)
    assert rec["valu_busy"] == pytest.approx(0.25)
    assert rec["mfma_busy"] == pytest.approx(0.5)
    assert rec["lds_busy"] is None and rec["waves"] == 100 and rec["valu_insts_per_wave"] == 10
