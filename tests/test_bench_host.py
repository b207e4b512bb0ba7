"""bench.py's host-side logic, on the CPU: the one-GPU refusal, the HBM
traffic summary (counters scaled by the copy probe, tied to the sources'
hash), the SQ-counter summary (VALU issue, shader clock, MFMA busy) and the
roofline of the dominant kernel family, on synthetic counter files and timings."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counters(d, rows):
    """rows: (dispatch id, kernel name, counter, value, start ns, end ns)"""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, cnt, val, t0, t1 in rows:
            w.writerow(dict(Correlation_Id=disp, Dispatch_Id=disp, Agent_Id="Agent 1", Queue_Id=1, Process_Id=1,
                            Thread_Id=1, Grid_Size=256, Kernel_Id=1, Kernel_Name=name, Workgroup_Size=256,
                            LDS_Block_Size=0, Scratch_Size=0, VGPR_Count=64, Accum_VGPR_Count=0, SGPR_Count=32,
                            Counter_Name=cnt, Counter_Value=val, Start_Timestamp=t0, End_Timestamp=t1))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_summary_scales_each_counter_by_the_copy_probe(tmp_path, monkeypatch):
    out = tmp_path / "traffic_wl.txt"
    monkeypatch.setattr(bench, "traffic_path", lambda wl: str(out))
    copy_mib = 64
    agg = "void egnn::(anonymous namespace)::aggregate_kernel<4, 2, float>(int const*)"
    probe = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    # the probe moves 64 MiB each way; FETCH_SIZE reads half of it, WRITE_SIZE all
    _counters(tmp_path / "f", [(1, probe, "FETCH_SIZE", copy_mib * 1024 / 2, 0, 1),
                               (2, agg, "FETCH_SIZE", 1000.0, 0, 1), (3, agg, "FETCH_SIZE", 3000.0, 0, 1)])
    _counters(tmp_path / "w", [(1, probe, "WRITE_SIZE", copy_mib * 1024, 0, 1),
                               (2, agg, "WRITE_SIZE", 500.0, 0, 1), (3, agg, "WRITE_SIZE", 700.0, 0, 1)])
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "wl", copy_mib, ["bench.py"])
    kv = dict(l.split(": ", 1) for l in out.read_text().splitlines() if ": " in l and not l.startswith("#"))
    assert float(kv["copy_scale_fetch"]) == pytest.approx(2.0)
    assert float(kv["copy_scale_write"]) == pytest.approx(1.0)
    # mean per dispatch: fetch 2000 KiB x 2, write 600 KiB x 1
    assert float(kv["traffic_bytes_per_launch[aggregate]"]) == pytest.approx((2000 * 2 + 600) * 1024)
    assert kv["source_sha256"] == bench.kernel_source_hash()
    assert bench.read_traffic("wl", "aggregate") == pytest.approx((2000 * 2 + 600) * 1024)
    assert bench.read_traffic("wl", "rotate_in") is None
    # a figure measured on other sources is not reported
    out.write_text(out.read_text().replace(bench.kernel_source_hash(), "0" * 64))
    assert bench.read_traffic("wl", "aggregate") is None


def test_traffic_summary_needs_the_copy_probe(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda wl: str(tmp_path / "t.txt"))
    name = "void egnn::(anonymous namespace)::hblocks_kernel<16, 4, float>()"
    _counters(tmp_path / "f", [(1, name, "FETCH_SIZE", 1.0, 0, 1)])
    _counters(tmp_path / "w", [(1, name, "WRITE_SIZE", 1.0, 0, 1)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "wl", 64, ["bench.py"])


def test_sq_summary_issue_clock_and_mfma_busy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    k = "void egnn::(anonymous namespace)::wrad_grad_kernel<4, 2, 8, float, 0, 4>(int const*)"
    gui = 8 * 2_000_000              # 2e6 cycles per XCD
    ns = 1_000_000                   # 1 ms -> 2.0 GHz
    p1 = [(1, k, c, v, 0, ns) for c, v in [("SQ_WAVES", 100), ("SQ_WAVE_CYCLES", 1e6), ("SQ_BUSY_CYCLES", 1e6),
                                            ("SQ_WAIT_ANY", 4e5), ("SQ_WAIT_INST_ANY", 1e5),
                                            ("SQ_ACTIVE_INST_VALU", 3e5), ("SQ_INSTS_VALU", 256_000_000),
                                            ("SQ_ACTIVE_INST_ANY", 5e5)]]
    p2 = [(1, k, c, v, 0, ns) for c, v in [("GRBM_GUI_ACTIVE", gui), ("SQ_INSTS_VMEM_RD", 100),
                                            ("SQ_INSTS_VMEM_WR", 10), ("SQ_INSTS_LDS", 50), ("SQ_INSTS_SALU", 20),
                                            ("SQ_ACTIVE_INST_LDS", 1e4), ("SQ_INST_CYCLES_VMEM", 1e4),
                                            ("SQ_WAIT_INST_LDS", 1e3)]]
    p3 = [(1, k, c, v, 0, ns) for c, v in [("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 2e6 * 0.25)]]
    for name, rows in (("p1", p1), ("p2", p2), ("p3", p3)):
        _counters(tmp_path / name, rows)
    bench.summarize_sq(str(tmp_path / "p1"), str(tmp_path / "p2"), "wl", ["bench.py"], str(tmp_path / "p3"))
    text = (tmp_path / "profiles" / "sq_wl.txt").read_text()
    # VALU issue: 256e6 instructions x 4 cycles over 1024 SIMDs x 2e6 cycles = 0.5
    assert "valu_issue 0.500" in text
    assert "clock 2.00 GHz" in text
    assert "mfma_busy 0.250" in text
    assert "VALU 2560000," in text          # per wave


def test_roofline_takes_the_family_with_the_most_time():
    timing = {"cgemm_fwd_f32": dict(total_ms=20.0, launches=4, flops=4 * 0.5e12, bytes=0.0),
              "aggregate": dict(total_ms=5.0, launches=2, flops=0.0, bytes=2 * 20e9)}
    fam, r = bench.roofline(timing, "f32", "no_such_workload")
    assert fam == "cgemm_fwd_f32" and r["bound"] == "mfma"
    # 0.5 TFLOP per 5 ms launch = 100 TFLOP/s against the fp32 peak
    assert r["achieved"] == pytest.approx(100.0)
    assert r["frac"] == pytest.approx(100.0 / bench.MFMA_PEAK_TFLOPS["f32"], abs=1e-4)
    assert r["executed_frac"] == pytest.approx(0.75 * r["frac"], abs=1e-4)
    assert r["traffic"] is None
    timing["aggregate"]["total_ms"] = 50.0
    fam, r = bench.roofline(timing, "f32", "no_such_workload")
    # 20 GB per 25 ms launch = 800 GB/s
    assert fam == "aggregate" and r["bound"] == "hbm" and r["achieved"] == pytest.approx(800.0)
    assert r["frac"] == pytest.approx(800.0 / bench.HBM_PEAK_GBS, abs=1e-4)


def test_every_timing_family_names_a_kernel_of_the_library():
    """The families' kernel-name pieces must match kernels that exist in the sources."""
    src = ""
    for f in os.listdir(bench.CSRC):
        if f.endswith(".hip"):
            src += open(os.path.join(bench.CSRC, f)).read()
    for fam, tag in bench.FAMILY_KERNELS.items():
        pieces = (tag,) if isinstance(tag, str) else tag
        head = pieces[0].lstrip(":").split("<")[0]
        assert head in src, (fam, head)
