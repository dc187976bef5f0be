"""Host logic of bench.py on the CPU: the refusal of runs on several GPUs, the counter summaries it
derives from rocprofv3 CSVs (shader clock and MFMA busy, wave states, per-dispatch kernel tables), the traffic
record's staleness check, and the algorithmic byte counts. Synthetic CSVs stand in for rocprofv3
output; nothing here touches a GPU or the committed profiles."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture
def scratch_root(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "profiles" / "traffic.json"))
    return tmp_path


def _write_csv(path, header, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def test_runs_on_several_gpus_are_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in out and out["n_gpus"] == 2


def test_gemm_clock_from_counters(tmp_path):
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    # dispatch 5: 18e6 cycles per XCD in 10 ms -> 1.8 GHz; MFMA busy 70% of every SIMD's cycles
    for name, val in [("GRBM_GUI_ACTIVE", 8 * 18e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 256 * 4 * 18e6 * 0.7),
                      ("SQ_BUSY_CYCLES", 1.0)]:
        rows.append([5, "void sq::k_gemm_tile<1>(...)", name, val, 1_000_000, 11_000_000])
    rows.append([6, "void sq::k_norm_quant<...>(...)", "GRBM_GUI_ACTIVE", 1.0, 0, 10])
    _write_csv(tmp_path / "clk" / "run_counter_collection.csv", header, rows)
    clk = bench.gemm_clock(str(tmp_path / "clk"))
    assert len(clk) == 1
    assert clk[0]["ms"] == pytest.approx(10.0)
    assert clk[0]["sclk_GHz"] == pytest.approx(1.8)
    assert clk[0]["mfma_busy"] == pytest.approx(0.7)


def test_fp8_table_splits_a_kernel_serving_two_row_counts(scratch_root):
    header = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows, t = [], 0
    for ms in [0.35] * 7 + [0.88] * 7:                                   # activations, then fold weights
        rows.append(["void sq::k_norm_quant<sq::f16_t, 0, 20, 512, 0>(...)", 131072, 512, t, t + int(ms * 1e6)])
        t += 2_000_000
    for ms in [0.0047] + [0.0021] * 13:                                  # one slow first launch: not split
        rows.append(["void sq::k_fill_zero(...)", 81920, 256, t, t + int(ms * 1e6)])
        t += 10_000
    rows.append(["void at::native::other(...)", 1, 1, 0, 5])
    _write_csv(scratch_root / "tr" / "run_kernel_trace.csv", header, rows)
    bench.summarize_fp8(str(scratch_root / "tr"))
    text = (scratch_root / "profiles" / "kernel_trace_fp8_mtnlg530b.md").read_text()
    nq = [ln for ln in text.splitlines() if ln.startswith("| `sq::k_norm_quant")]
    assert len(nq) == 2 and all("| 7 |" in ln for ln in nq)
    assert "0.8800" in nq[0] and "0.3500" in nq[1]                       # slower group first
    fz = [ln for ln in text.splitlines() if ln.startswith("| `sq::k_fill_zero")]
    assert len(fz) == 1 and "| 14 |" in fz[0]
    assert "at::native" not in text


def test_traffic_record_goes_stale_with_the_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    rec = {"source_sha256": bench.gemm_source_hash(), "traffic_bytes_per_launch": 1.0}
    with open(bench.TRAFFIC_JSON, "w") as f:
        json.dump(rec, f)
    assert bench.recorded_traffic()["traffic_bytes_per_launch"] == 1.0
    rec["source_sha256"] = "0" * 64
    with open(bench.TRAFFIC_JSON, "w") as f:
        json.dump(rec, f)
    assert bench.recorded_traffic() is None
    os.remove(bench.TRAFFIC_JSON)
    assert bench.recorded_traffic() is None


def test_decode_bytes_counts_weights_tokens_scales_and_output():
    # N*K weight codes + M*K token codes + 4 (M + N) scale bytes + 2 M N fp16 outputs
    assert bench.decode_bytes(1, 9216) == 9216 * 9216 + 9216 + 4 * (1 + 9216) + 2 * 9216
    assert bench.decode_bytes(64, 36864, 9216) == 36864 * 9216 + 64 * 9216 + 4 * (64 + 36864) + 2 * 64 * 36864


def test_prefill_summary_splits_runs_by_launch_count(scratch_root, monkeypatch):
    # 1 warm-up and 2 timed rounds of 1 launch per shape: each shape's 3 dispatches, in start order,
    # whatever else (another library's kernels) runs between them
    monkeypatch.setattr(bench, "PREFILL_WARM", 1)
    monkeypatch.setattr(bench, "PREFILL_TIMES", 2)
    monkeypatch.setattr(bench, "prefill_reps", lambda m, n, k: 1)
    header = ["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows, t = [], 0
    shapes = bench.prefill_shapes()
    for i, _ in enumerate(shapes):
        for ms in (0.3, 0.1, 0.2):                                 # median 0.2 ms (+ i)
            rows.append(["void sq::k_gemm_tile<1>(...)", 256, t, t + int((ms + i) * 1e6)])
            t += 20_000_000
        rows.append(["void at::native::elementwise_kernel(...)", 1024, t, t + 1_000_000])
        t += 20_000_000
    _write_csv(scratch_root / "pf" / "run_kernel_trace.csv", header, rows[::-1])    # any file order
    bench.summarize_prefill(str(scratch_root / "pf"))
    text = (scratch_root / "profiles" / "prefill_gemm_all_workloads.md").read_text()
    body = [ln for ln in text.splitlines() if ln.startswith("| ") and "`sq::" in ln]
    assert len(body) == len(shapes)
    for i, ln in enumerate(body):
        assert f"| 3 | {0.2 + i:.4f} | {0.1 + i:.4f} |" in ln
    assert "elementwise" not in text
    rows.append(["void sq::k_gemm_tile<1>(...)", 256, t, t + 1])     # one dispatch too many
    _write_csv(scratch_root / "pf2" / "run_kernel_trace.csv", header, rows)
    with pytest.raises(SystemExit):
        bench.summarize_prefill(str(scratch_root / "pf2"))


def test_clock_sampler_reads_the_current_dpm_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1788Mhz *\n2: 2400Mhz\n")
    assert bench.ClockSampler(str(f)).read_mhz() == 1788.0
    f.write_text("0: 500Mhz\n1: 573Mhz\n2: 2400Mhz\n")
    with pytest.raises(RuntimeError):
        bench.ClockSampler(str(f)).read_mhz()


def test_clock_sampler_reads_board_power_and_cap(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1788Mhz *\n")
    hw = tmp_path / "hwmon" / "hwmon3"
    hw.mkdir(parents=True)
    (hw / "power1_input").write_text("1350000000\n")
    (hw / "power1_cap").write_text("1400000000\n")
    s = bench.ClockSampler(str(f))
    assert s.power_path == str(hw / "power1_input")
    assert s.read_watts() == 1350.0 and s.cap_watts() == 1400.0
    (hw / "power1_input").unlink()
    (hw / "power1_average").write_text("900000000\n")
    assert bench.ClockSampler(str(f)).read_watts() == 900.0
    assert bench.ClockSampler(str(tmp_path / "pp_dpm_sclk"), hwmon=str(tmp_path / "none")).power_path is None


def test_ln_wave_states_from_counters(scratch_root):
    # one dispatch of 4096 waves over 200,000 cycles per XCD (0.1 ms): each wave lives 200 quad-cycles
    # of which 50 on an instruction, 40 ready but not issued and 110 waiting; the SIMDs' VALU holds
    # 0.6 of the dispatch's quad-cycles
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    quads = 200_000 / 4
    vals = {"SQ_WAVE_CYCLES": 4096 * 200, "SQ_ACTIVE_INST_ANY": 4096 * 50, "SQ_WAIT_INST_ANY": 4096 * 40,
            "SQ_WAIT_ANY": 4096 * 110, "SQ_ACTIVE_INST_VALU": 0.6 * 1024 * quads, "SQ_WAVES": 4096,
            "GRBM_GUI_ACTIVE": 8 * 200_000, "SQ_INSTS_VALU": 1.0, "SQ_BUSY_CYCLES": 1.0}
    rows = [[9, "void sq::k_norm_quant<sq::f16_t, 1, 5, 512, 0>(...)", k, v, 0, 100_000] for k, v in vals.items()]
    rows.append([3, "void sq::k_gemm_tile<1, 4>(...)", "SQ_WAVES", 1, 0, 10])
    _write_csv(scratch_root / "w" / "run_counter_collection.csv", header, rows)
    bench.summarize_ln_waits(str(scratch_root / "w"))
    text = (scratch_root / "profiles" / "norm_quant_layernorm_waits_mtnlg530b.md").read_text()
    body = [ln for ln in text.splitlines() if ln.startswith("| timed")]
    assert body == ["| timed | 0.1000 | 4096 | 0.25 | 0.20 | 0.55 | 0.60 |"]
