"""Benchmark of the SmoothQuant W8A8 linear layer on one MI355X.

One step = the whole path over one batch of the workload, for every site of it:
calibration absmax -> smoothing fold (s, folded norm, INT8 weights) -> fused
norm + per-token INT8 quantisation -> INT8 GEMM with dequant epilogue.
Default workload: the MT-NLG-530B-width layer (hidden 20480: LayerNorm -> fc1
20480 -> 81920 and fc2 81920 -> 20480 at 8192 tokens, fp16), the largest
single-GPU prefill configuration.

Prints one JSON line. `value` is the step's GEMM work (2*M*N*K summed over the
sites) divided by the step time, in TOPS; `roofline` reports the GEMM kernel
against the INT8 dense MFMA peak from HIP events around each launch (with the
HBM traffic, shader clock and MFMA-busy fraction of the committed rocprofv3
counter record while the GEMM sources are unchanged since it was taken); `kernels`
gives every stage's average duration and its achieved rate; `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0        # MI355X dense INT8 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
EPS = 1e-5


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=5)
    p.add_argument("--m", type=int, default=None, help="token count (workloads with several)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true", help="leave out the decode GEMM block")
    p.add_argument("--no-clock", action="store_true", help="leave out the shader-clock sampling")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one plain device copy of this size (counter calibration runs)")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="turn rocprofv3 CSV output of this benchmark into profiles/ summaries and exit")
    p.add_argument("--decode-sweep", action="store_true",
                   help="time the decode GEMMs (K=9216, N in {9216, 36864}, 1..64 tokens) with rotating weight "
                        "copies and exit")
    p.add_argument("--summarize-decode", metavar="TRACE_DIR",
                   help="turn a rocprofv3 --kernel-trace of --decode-sweep into a profiles/ table and exit")
    p.add_argument("--granularities", action="store_true",
                   help="time per-token, per-tensor dynamic and static activation steps and both weight-step "
                        "folds on the default workload's sites, and exit")
    p.add_argument("--accuracy", action="store_true",
                   help="synthetic accuracy study: plain INT8 vs SmoothQuant over alpha, on every workload, and exit")
    p.add_argument("--accuracy-tokens", type=int, default=256, help="token rows per site in the accuracy study")
    p.add_argument("--summarize-granularities", metavar="TRACE_DIR",
                   help="turn a rocprofv3 --kernel-trace --stats of --granularities into a profiles/ table and exit")
    p.add_argument("--fp8", action="store_true",
                   help="INT8 against FP8 (E4M3) per stage on the MT-NLG-530B-width sites (HIP-event medians) and "
                        "exit; with --decode-sweep / --summarize-decode, the FP8 decode GEMMs instead")
    p.add_argument("--summarize-fp8", metavar="TRACE_DIR",
                   help="turn a rocprofv3 --kernel-trace --stats of --fp8 into a profiles/ table and exit")
    p.add_argument("--llm-int8", action="store_true",
                   help="time LLM.int8()'s decomposition beside the SmoothQuant run-time path on the OPT-6.7B and "
                        "MT-NLG-530B-width sites, and exit")
    p.add_argument("--summarize-llm-int8", nargs="+", metavar="PATH",
                   help="TRACE_DIR [SWEEP_STDOUT]: turn a rocprofv3 --kernel-trace --stats of --llm-int8 (and the "
                        "run's stdout) into a profiles/ table and exit")
    p.add_argument("--prefill-sweep", action="store_true",
                   help="time the prefill GEMMs of every workload (fp16 out) and exit")
    p.add_argument("--summarize-decode-counters", metavar="PMC_DIR",
                   help="turn a rocprofv3 --pmc SQ_WAVE_CYCLES SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
                        "SQ_LDS_BANK_CONFLICT run of --decode-sweep into a profiles/ table and exit")
    p.add_argument("--summarize-ln-counters", metavar="PMC_DIR",
                   help="turn a rocprofv3 --pmc SQ_INSTS_VALU GRBM_GUI_ACTIVE run of this benchmark into a "
                        "profiles/ table of the LayerNorm quantiser's vector-ALU issue and exit")
    p.add_argument("--summarize-ln-waits", metavar="PMC_DIR",
                   help="turn a rocprofv3 --pmc run of the LayerNorm wave-state counters into a profiles/ table "
                        "and exit")
    p.add_argument("--summarize-prefill", metavar="TRACE_DIR",
                   help="turn a rocprofv3 --kernel-trace of --prefill-sweep into a profiles/ table and exit")
    return p.parse_args()


# ----------------------------------------------------------------------------- counter summaries

GEMM_SOURCES = ["w8a8_int8_linear_amd/csrc/k_gemm.hip", "w8a8_int8_linear_amd/csrc/sq_device.h",
                "w8a8_int8_linear_amd/csrc/sq_launch.h"]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "k_gemm_tile_traffic.json")


def build_flags():
    """The compile flags of the library (the COMMON list of its build script, loaded by path)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_sq_build_flags", os.path.join(ROOT, "w8a8_int8_linear_amd",
                                                                                "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [f for f in mod.COMMON if not f.startswith(("-I", "/"))]


def gemm_source_hash() -> str:
    """Hash of everything that shapes the GEMM kernel's code: its sources and the compile flags."""
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(json.dumps(build_flags()).encode())
    return h.hexdigest()


class ClockSampler:
    """The GPU's current shader clock, read from the driver's sysfs DPM table (pp_dpm_sclk: the line
    marked '*' holds the current clock, which the driver updates continuously) from a host thread
    every ~2 ms while a workload runs: a same-run measure of the clock the GEMM holds. (The
    gpu-metrics table behind amdsmi refreshes only every few hundred ms on this driver, so it is
    not used.) Where the card's hwmon directory has them, the board power (power1_input, or
    power1_average; microwatts) is sampled in the same loop and the power cap (power1_cap) read once."""

    def __init__(self, path=None, hwmon=None):
        import glob
        paths = [path] if path else sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(paths) != 1:
            raise RuntimeError(f"expected one pp_dpm_sclk, found {paths}")
        self.path = paths[0]
        self.samples = []
        self.watts = []
        dirs = [hwmon] if hwmon else sorted(glob.glob(os.path.join(os.path.dirname(self.path), "hwmon", "hwmon*")))
        self.power_path = self.cap_path = None
        for d in dirs[:1]:
            for name in ("power1_input", "power1_average"):
                if os.path.exists(os.path.join(d, name)):
                    self.power_path = os.path.join(d, name)
                    break
            if os.path.exists(os.path.join(d, "power1_cap")):
                self.cap_path = os.path.join(d, "power1_cap")

    def read_watts(self):
        with open(self.power_path) as f:
            return int(f.read().strip()) / 1e6

    def cap_watts(self):
        if not self.cap_path:
            return None
        with open(self.cap_path) as f:
            return int(f.read().strip()) / 1e6

    def read_mhz(self):
        with open(self.path) as f:
            for line in f:
                if "*" in line:
                    return float(line.split(":", 1)[1].split("Mhz")[0].strip())
        raise RuntimeError("no current level in pp_dpm_sclk")

    def run_while(self, torch, fn, seconds):
        """Call fn() repeatedly for about `seconds` (each call drained before the next) while sampling."""
        import threading
        stop = threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    self.samples.append(self.read_mhz())
                except Exception:          # a failed read is skipped, not invented
                    pass
                if self.power_path:
                    try:
                        self.watts.append(self.read_watts())
                    except Exception:
                        pass
                time.sleep(0.002)
        th = threading.Thread(target=loop, daemon=True)
        fn()
        torch.cuda.synchronize()
        self.samples.clear()
        self.watts.clear()
        th.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            fn()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        return self.samples


def recorded_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None when the
    kernel has changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != gemm_source_hash():
        return None
    return rec


N_XCD, N_CU, SIMD_PER_CU, PEAK_SCLK_GHZ = 8, 256, 4, 2.4     # MI355X; the dense peaks are quoted at 2.4 GHz


def _read_csv(path):
    """Rows of a rocprofv3 CSV as dicts, the file closed on return."""
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def gemm_clock(clock_dir):
    """Shader clock and MFMA-busy fraction of each GEMM dispatch of a --pmc GRBM_GUI_ACTIVE
    SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES run: GRBM_GUI_ACTIVE sums the busy cycles of the
    XCDs, so cycles per XCD over the dispatch's duration is the clock; the MFMA busy cycles,
    summed over the CUs, are divided by the cycles of every SIMD."""
    import glob
    from collections import defaultdict
    hits = glob.glob(os.path.join(clock_dir, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no counter collection under {clock_dir}")
    per = defaultdict(dict)
    for r in _read_csv(hits[0]):
        if "k_gemm_tile" in r["Kernel_Name"]:
            d = per[int(r["Dispatch_Id"])]
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = []
    for _, d in sorted(per.items()):
        cyc = d["GRBM_GUI_ACTIVE"] / N_XCD
        out.append({"ms": d["ns"] / 1e6, "sclk_GHz": cyc / d["ns"],
                    "mfma_busy": d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_CU * SIMD_PER_CU) / cyc})
    return out


def summarize_counters(trace_dir, fetch_dir, write_dir, clock_dir=None):
    """rocprofv3 CSVs of `bench.py` runs -> profiles/*.md and the GEMM traffic record.

    FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what it reads for
    the plain device copy of --copy-probe-mib MiB that the counter runs add at the end.
    With clock_dir (a GRBM_GUI_ACTIVE / MFMA-busy run), the record also carries each GEMM
    dispatch's shader clock and MFMA-busy fraction.
    """
    import glob
    from collections import defaultdict

    def one(d, pat):
        hits = glob.glob(os.path.join(d, "**", pat), recursive=True)
        if not hits:
            raise SystemExit(f"no {pat} under {d}")
        return hits[0]

    stats = list(_read_csv(one(trace_dir, "*kernel_stats.csv")))
    counters = {}
    for name, d in [("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)]:
        rows = [r for r in _read_csv(one(d, "*counter_collection.csv")) if r["Counter_Name"] == name]
        copy = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        copy = max(copy, key=lambda r: float(r["Counter_Value"]))
        per = defaultdict(list)
        for r in rows:
            if "sq::" in r["Kernel_Name"]:
                per[(int(r["Dispatch_Id"]), r["Kernel_Name"])] = float(r["Counter_Value"])
        counters[name] = {"copy_kib": float(copy["Counter_Value"]), "per": per}
    copy_kib = 1024.0 * max(1, int(os.environ.get("COPY_PROBE_MIB", "1024")))
    scale = {k: copy_kib / v["copy_kib"] for k, v in counters.items()}
    gemm = sorted(k for k in counters["FETCH_SIZE"]["per"] if "k_gemm" in k[1])
    gemm_w = sorted(k for k in counters["WRITE_SIZE"]["per"] if "k_gemm" in k[1])
    launches = []
    for (fd, _), (wd, _) in zip(gemm, gemm_w):
        fb = counters["FETCH_SIZE"]["per"][(fd, _)] * scale["FETCH_SIZE"] * 1024
        wb = counters["WRITE_SIZE"]["per"][(wd, _)] * scale["WRITE_SIZE"] * 1024
        launches.append({"fetch_bytes": fb, "write_bytes": wb})
    cmd_trace = ("rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
                 "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-decode --no-clock")
    cmd_pmc = ("rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} -d <dir> -o run --output-format csv -- "
               "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-decode --no-clock --copy-probe-mib 1024")
    cmd_clock = ("rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES -d <dir> -o run "
                 "--output-format csv -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-decode --no-clock")
    rec = {"kernel": "k_gemm_tile", "workload": "mtnlg530b_width_m8192_h20480 (fc1 then fc2)",
           "source_sha256": gemm_source_hash(), "fetch_scale": scale["FETCH_SIZE"],
           "write_scale": scale["WRITE_SIZE"], "launches": launches,
           "traffic_bytes_per_launch": sum(l["fetch_bytes"] + l["write_bytes"] for l in launches) / len(launches),
           "commands": [cmd_trace, cmd_pmc]}
    if clock_dir:
        clk = gemm_clock(clock_dir)
        timed = clk[-2:]                                 # the timed step's fc1 and fc2; the rest warm up
        rec["clock"] = clk
        rec["sclk_GHz"] = sum(c["sclk_GHz"] for c in timed) / len(timed)
        rec["mfma_busy"] = sum(c["mfma_busy"] for c in timed) / len(timed)
        rec["commands"].append(cmd_clock)
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# rocprofv3 kernel statistics: bench.py, MT-NLG-530B-width layer (M=8192, hidden 20480)", "",
             f"Command: `{cmd_trace}`", "",
             "| kernel | calls | average ms | min ms | max ms |", "|---|---|---|---|---|"]
    for r in stats:
        if "sq::" in r["Name"]:
            short = r["Name"].split("(")[0].replace("void ", "")
            lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                         f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} |")
    lines += ["", "Each step launches every kernel of both sites (fc1 behind LayerNorm, fc2 without a norm); "
              "k_gemm_tile's average covers both GEMM shapes (8192x81920x20480 and 8192x20480x81920)."]
    with open(os.path.join(ROOT, "profiles", "kernel_stats_mtnlg530b_width.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE, WRITE_SIZE): MT-NLG-530B-width layer", "",
             f"Commands: `{cmd_pmc}` (one run per counter).", "",
             f"Scale: the 1 GiB device copy reads FETCH_SIZE = {counters['FETCH_SIZE']['copy_kib']:.0f} KiB "
             f"and WRITE_SIZE = {counters['WRITE_SIZE']['copy_kib']:.0f} KiB, so FETCH_SIZE is multiplied by "
             f"{scale['FETCH_SIZE']:.3f} and WRITE_SIZE by {scale['WRITE_SIZE']:.3f}.", "",
             "| dispatch | kernel | fetched GB | written GB |", "|---|---|---|---|"]
    for (fd, name), (wd, _) in zip(sorted(counters["FETCH_SIZE"]["per"]), sorted(counters["WRITE_SIZE"]["per"])):
        fb = counters["FETCH_SIZE"]["per"][(fd, name)] * scale["FETCH_SIZE"] * 1024 / 1e9
        wb = counters["WRITE_SIZE"]["per"][(wd, name)] * scale["WRITE_SIZE"] * 1024 / 1e9
        lines.append(f"| {fd} | `{name.split('(')[0].replace('void ', '')}` | {fb:.3f} | {wb:.3f} |")
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_mtnlg530b_width.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if clock_dir:
        lines = ["# Shader clock and MFMA busy of the GEMM (rocprofv3 counters): MT-NLG-530B-width layer", "",
                 f"Command: `{cmd_clock}`.", "",
                 "One warm-up step, then the timed step; the bench reports the timed step's averages "
                 f"(clock {rec['sclk_GHz']:.3f} GHz, MFMA busy {rec['mfma_busy']:.3f}).", "",
                 f"Clock = GRBM_GUI_ACTIVE / {N_XCD} XCDs / dispatch duration; MFMA busy = "
                 f"SQ_VALU_MFMA_BUSY_CYCLES / ({N_CU} CUs x {SIMD_PER_CU} SIMDs) / cycles per XCD. The dense INT8 "
                 f"peak of 5.0 POPS is quoted at {PEAK_SCLK_GHZ} GHz and scales with the clock.", "",
                 "| dispatch | ms | shader clock GHz | MFMA busy | TOPS | peak at this clock | fraction of it |",
                 "|---|---|---|---|---|---|---|"]
        n_clk = len(rec["clock"])
        for i, c in enumerate(rec["clock"]):
            tops = 2.0 * 8192 * 81920 * 20480 / (c["ms"] * 1e-3) / 1e12
            pk = PEAK_INT8_TOPS * c["sclk_GHz"] / PEAK_SCLK_GHZ
            tag = ("fc1" if i % 2 == 0 else "fc2") + (" (warm-up)" if i < n_clk - 2 else "")
            lines.append(f"| {tag} | {c['ms']:.3f} | {c['sclk_GHz']:.3f} | "
                         f"{c['mfma_busy']:.3f} | {tops:.0f} | {pk:.0f} | {tops / pk:.3f} |")
        with open(os.path.join(ROOT, "profiles", "gemm_clock_mtnlg530b_width.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))


# ----------------------------------------------------------------------------- decode sweep

DEC_K = 9216                                  # OPT-66B hidden size
DEC_NS = [9216, 36864]                        # the square projection and fc1
DEC_MS = [1, 2, 4, 8, 16, 32, 48, 64]
DEC_WARM, DEC_ITERS = 2, 12
DEC_CMD = "rocprofv3 --kernel-trace -d <dir> -o run --output-format csv -- python3 bench.py --decode-sweep"


def decode_bytes(m, n, k=DEC_K):
    """Algorithmic bytes of one decode GEMM: Wq, Xq, both scale vectors and the fp16 output."""
    return n * k + m * k + 4 * (m + n) + 2 * m * n


def decode_sweep(fp8=False):
    """Decode GEMMs at the OPT-66B width with enough weight copies (>= 600 MB) rotating that no
    launch finds its weights in the 256 MB MALL; HIP-event medians per shape (the launch gap
    included; the rocprofv3 trace of this run gives the kernel durations). fp8: E4M3 codes of
    N(0, 1) values through sq_fp8_gemm instead of INT8 codes through sq_w8a8_gemm."""
    import torch
    import w8a8_int8_linear_amd as sq
    gen = torch.Generator(device="cpu").manual_seed(3)

    def codes(rows):
        if fp8:
            return torch.randn(rows, DEC_K, generator=gen).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
        return torch.randint(-127, 128, (rows, DEC_K), dtype=torch.int8, generator=gen).cuda()

    gemm = sq.sq_fp8_gemm if fp8 else sq.sq_w8a8_gemm
    for n in DEC_NS:
        copies = max(2, -(-600_000_000 // (n * DEC_K)))
        ws = [codes(n) for _ in range(copies)]
        wsc = (torch.rand(n, generator=gen) * 0.01).cuda()
        for m in DEC_MS:
            xq = codes(m)
            xs = (torch.rand(m, generator=gen) * 0.01).cuda()
            y = torch.empty(m, n, dtype=torch.float16, device="cuda")
            for i in range(DEC_WARM):
                gemm(xq, xs, ws[i % copies], wsc, y=y, out_dtype=torch.float16)
            torch.cuda.synchronize()
            ts = []
            for i in range(DEC_ITERS):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                gemm(xq, xs, ws[i % copies], wsc, y=y, out_dtype=torch.float16)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            ts.sort()
            med = ts[len(ts) // 2]
            print(json.dumps({"decode": [m, n, DEC_K], "format": "fp8" if fp8 else "int8", "us_event_median": round(med, 2),
                              "GBps": round(decode_bytes(m, n) / med / 1e3, 1)}), flush=True)
            del xq, y
        del ws
        torch.cuda.empty_cache()


DEC_BLOCK_MS = [1, 8, 32, 64]                 # the OPT-66B decode token counts


def decode_block(torch, sq, replays=5):
    """Decode GEMMs (K = 9216, N in {9216, 36864}, 1/8/32/64 tokens, fp16 out) for the default JSON
    line. Per shape, one HIP graph launches the GEMM once per weight copy (copies totalling >= 600 MB
    rotate, so no launch finds its weights in the 256 MB MALL); the graph is replayed between two HIP
    events on the stream the library launches on, and the per-launch time is the replay's time over
    the number of launches (kernel time plus the graph's dispatch gap)."""
    gen = torch.Generator(device="cuda").manual_seed(3)
    out = []
    for n in DEC_NS:
        copies = max(2, -(-600_000_000 // (n * DEC_K)))
        ws = [torch.randint(-127, 128, (n, DEC_K), dtype=torch.int8, device="cuda", generator=gen)
              for _ in range(copies)]
        wsc = torch.rand(n, device="cuda", generator=gen) * 0.01
        for m in DEC_BLOCK_MS:
            xq = torch.randint(-127, 128, (m, DEC_K), dtype=torch.int8, device="cuda", generator=gen)
            xs = torch.rand(m, device="cuda", generator=gen) * 0.01
            y = torch.empty(m, n, dtype=torch.float16, device="cuda")

            def launches():
                for w in ws:
                    sq.sq_w8a8_gemm(xq, xs, w, wsc, y=y, out_dtype=torch.float16)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                launches()                                     # warm-up outside the capture
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                launches()
            graph.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(replays):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                graph.replay()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / copies)
            ts.sort()
            us = ts[len(ts) // 2]
            gbs = decode_bytes(m, n) / us / 1e3
            out.append({"tokens": m, "N": n, "K": DEC_K, "us": round(us, 2), "GBps": round(gbs, 1),
                        "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
            del graph, xq, y
        del ws
        torch.cuda.empty_cache()
    return out


DEC_PMC = ("SQ_WAVE_CYCLES", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT")


def summarize_decode_counters(pmc_dir):
    """LDS counters of the decode kernels in a --pmc run of --decode-sweep: per kernel instance, the
    shares of wave cycles spent waiting on LDS instructions and issuing them, summed over the
    instance's dispatches (SQ_LDS_BANK_CONFLICT counts the LDS unit's stall cycles, not wave
    cycles, so it is not turned into a share)."""
    import glob
    from collections import defaultdict
    hits = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no counter collection under {pmc_dir}")
    tot = defaultdict(lambda: defaultdict(float))
    calls = defaultdict(set)
    for r in _read_csv(hits[0]):
        name = r["Kernel_Name"]
        if "sq::k_gemm_decode" not in name and "sq::k_gemv" not in name:
            continue
        grid = int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)
        wg = int(r.get("Workgroup_Size") or r.get("Workgroup_Size_X") or 1)
        key = (name.split("(")[0].replace("void ", ""), grid // wg)
        tot[key][r["Counter_Name"]] += float(r["Counter_Value"])
        calls[key].add(r["Dispatch_Id"])
    cmd = ("rocprofv3 --pmc " + " ".join(DEC_PMC) + " -d <dir> -o run --output-format csv -- "
           "python3 bench.py --decode-sweep")
    lines = ["# Decode GEMM LDS counters (rocprofv3 --pmc): OPT-66B width, K = 9216, INT8", "",
             f"Command: `{cmd}`, then `python bench.py --summarize-decode-counters <dir>`.", "",
             "Summed over each kernel instance's dispatches (every token count it serves, warm-up included). "
             "Both columns are shares of all wave cycles (SQ_WAVE_CYCLES). SQ_LDS_BANK_CONFLICT, collected "
             "in the same run, counts the LDS unit's stall cycles rather than wave cycles and is not shown.",
             "", "| kernel | workgroups | dispatches | LDS wait / wave cycles | LDS active / wave cycles |"
             "", "|---|---|---|---|---|"]
    for key in sorted(tot, key=lambda k: (k[1], k[0])):
        c = tot[key]
        wc = max(c["SQ_WAVE_CYCLES"], 1.0)
        lines.append(f"| `{key[0]}` | {key[1]} | {len(calls[key])} | {c['SQ_WAIT_INST_LDS'] / wc:.3f} | "
                     f"{c['SQ_ACTIVE_INST_LDS'] / wc:.3f} |")
    with open(os.path.join(ROOT, "profiles", "decode_gemm_lds_counters_opt66b_k9216.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_ln_counters(pmc_dir, m=8192, k=20480):
    """Vector-ALU issue of the LayerNorm quantiser (MT-NLG width, 8192 x 20480 fp16) per dispatch:
    SQ_INSTS_VALU counts wave instructions over the device, GRBM_GUI_ACTIVE the busy cycles summed over
    the XCDs. Lane instructions per element = 64 x instructions / (M K); a CU issues at most one VALU
    wave instruction per cycle (four SIMDs, four cycles each), so the issue share is instructions over
    CU cycles."""
    import glob
    from collections import defaultdict
    hits = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no counter collection under {pmc_dir}")
    per = defaultdict(dict)
    for r in _read_csv(hits[0]):
        if "sq::k_norm_quant<sq::f16_t, 1," in r["Kernel_Name"]:
            d = per[int(r["Dispatch_Id"])]
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        raise SystemExit("no LayerNorm quantiser dispatch in the run")
    cmd = ("rocprofv3 --pmc SQ_INSTS_VALU GRBM_GUI_ACTIVE -d <dir> -o run --output-format csv -- "
           "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-decode --no-clock")
    lines = ["# LayerNorm quantiser vector-ALU issue (rocprofv3 --pmc): MT-NLG width, 8192 x 20480 fp16", "",
             f"Command: `{cmd}`, then `python bench.py --summarize-ln-counters <dir>`.", "",
             "Kernel `sq::k_norm_quant<sq::f16_t, 1, 5, 512, 0>` (LayerNorm, per-token INT8 steps). Clock = "
             "GRBM_GUI_ACTIVE / 8 XCDs / duration; issue share = SQ_INSTS_VALU / (256 CUs x cycles).", "",
             "| dispatch | ms | clock GHz | VALU lane instructions per element | VALU issue share |",
             "|---|---|---|---|---|"]
    for i, (_, d) in enumerate(sorted(per.items())):
        cyc = d["GRBM_GUI_ACTIVE"] / N_XCD
        lines.append(f"| {'warm-up' if i == 0 and len(per) > 1 else 'timed'} | {d['ns'] / 1e6:.4f} | "
                     f"{cyc / d['ns']:.2f} | {64.0 * d['SQ_INSTS_VALU'] / (m * k):.1f} | "
                     f"{d['SQ_INSTS_VALU'] / (N_CU * cyc):.2f} |")
    with open(os.path.join(ROOT, "profiles", "norm_quant_layernorm_valu_mtnlg530b.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


LN_WAIT_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_BUSY_CYCLES "
                    "SQ_INSTS_VALU SQ_WAVES GRBM_GUI_ACTIVE")


def summarize_ln_waits(pmc_dir):
    """Where the LayerNorm quantiser's waves spend their time (MT-NLG width, 8192 x 20480 fp16). The SQ
    wave-state counters count quad-cycles summed over every wave: working on an instruction
    (SQ_ACTIVE_INST_ANY), ready but not yet issued because other waves hold the unit
    (SQ_WAIT_INST_ANY), and waiting on a counter or barrier (SQ_WAIT_ANY), each over the waves' lifetime
    (SQ_WAVE_CYCLES). One wave64 VALU instruction holds its SIMD for one quad-cycle, so the SIMDs'
    VALU share is SQ_ACTIVE_INST_VALU over (SIMDs x quad-cycles of the dispatch)."""
    import glob
    from collections import defaultdict
    hits = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no counter collection under {pmc_dir}")
    per = defaultdict(lambda: defaultdict(float))
    for r in _read_csv(hits[0]):
        if "sq::k_norm_quant<sq::f16_t, 1," in r["Kernel_Name"]:
            d = per[int(r["Dispatch_Id"])]
            d[r["Counter_Name"]] += float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        raise SystemExit("no LayerNorm quantiser dispatch in the run")
    cmd = (f"rocprofv3 --pmc {LN_WAIT_COUNTERS} -d <dir> -o run --output-format csv -- "
           "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-decode --no-clock")
    lines = ["# LayerNorm quantiser wave states (rocprofv3 --pmc): MT-NLG width, 8192 x 20480 fp16", "",
             f"Command: `{cmd}`, then `python bench.py --summarize-ln-waits <dir>`.", "",
             "Kernel `sq::k_norm_quant<sq::f16_t, 1, 5, 512, 0>`: 512 threads (8 waves) per workgroup, two "
             "workgroups per CU (116 VGPRs and 64 KiB of LDS each: four waves per SIMD). Shares of the waves' lifetime "
             "(SQ_WAVE_CYCLES); SIMD VALU busy = SQ_ACTIVE_INST_VALU / (1024 SIMDs x dispatch cycles / 4).", "",
             "| dispatch | ms | waves | instruction in progress | ready, waiting for issue | waiting on a counter "
             "or barrier | SIMD VALU busy |",
             "|---|---|---|---|---|---|---|"]
    for i, (_, d) in enumerate(sorted(per.items())):
        wc = d["SQ_WAVE_CYCLES"]
        quads = d["GRBM_GUI_ACTIVE"] / N_XCD / 4
        lines.append(f"| {'warm-up' if i == 0 and len(per) > 1 else 'timed'} | {d['ns'] / 1e6:.4f} | "
                     f"{int(d['SQ_WAVES'])} | {d['SQ_ACTIVE_INST_ANY'] / wc:.2f} | {d['SQ_WAIT_INST_ANY'] / wc:.2f} | "
                     f"{d['SQ_WAIT_ANY'] / wc:.2f} | {d['SQ_ACTIVE_INST_VALU'] / (4 * N_CU * quads):.2f} |")
    with open(os.path.join(ROOT, "profiles", "norm_quant_layernorm_waits_mtnlg530b.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_decode(trace_dir, fp8=False):
    """Kernel durations of a --decode-sweep trace (with --fp8: of --decode-sweep --fp8), matched to
    its shapes by dispatch order."""
    import glob
    hits = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    rows = [r for r in _read_csv(hits[0]) if "sq::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = DEC_WARM + DEC_ITERS
    shapes = [(m, n) for n in DEC_NS for m in DEC_MS]
    if len(rows) != per * len(shapes):
        raise SystemExit(f"expected {per * len(shapes)} dispatches, found {len(rows)}")
    fmt, flag = ("FP8 (E4M3)", " --fp8") if fp8 else ("INT8", "")
    lines = [f"# {fmt} decode GEMM kernel durations (rocprofv3 kernel trace): OPT-66B width, K = 9216, fp16 out", "",
             f"Command: `{DEC_CMD}{flag}`, then `python bench.py --summarize-decode <dir>{flag}`.", "",
             "Each shape: 2 warm-up and 12 timed launches, rotating weight copies totalling >= 600 MB so that "
             "no launch finds its weights in the MALL. Bytes = Wq + Xq + scales + fp16 output; "
             "the bar is 75% of 8 TB/s.", "",
             "| tokens | N | kernel | median us | min us | TB/s | 75% bar us |", "|---|---|---|---|---|---|---|"]
    for i, (m, n) in enumerate(shapes):
        rs = rows[i * per + DEC_WARM:(i + 1) * per]
        du = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs)
        med = du[len(du) // 2]
        name = rs[0]["Kernel_Name"].split("(")[0].replace("void ", "")
        b = decode_bytes(m, n)
        lines.append(f"| {m} | {n} | `{name}` | {med:.2f} | {du[0]:.2f} | {b / med / 1e6:.2f} | {b / 6e6:.2f} |")
    out = "decode_gemm_fp8_opt66b_k9216.md" if fp8 else "decode_gemm_opt66b_k9216.md"
    with open(os.path.join(ROOT, "profiles", out), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ----------------------------------------------------------------------------- granularities

GRAN_CMD = ("rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
            "python3 bench.py --granularities")


PREFILL_WARM, PREFILL_TIMES = 3, 3


def prefill_reps(m, n, k):
    return 5 if m * n * k > 1e12 else 30


def prefill_sweep():
    """Prefill GEMMs of every workload's sites (fp16 out, with the dequantising epilogue): the best of
    three means of back-to-back launches, after PREFILL_WARM untimed launches."""
    import torch
    import w8a8_int8_linear_amd as sq

    def best_ms(fn, n):
        for _ in range(PREFILL_WARM):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(PREFILL_TIMES):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) / n)
        return best

    g = torch.Generator(device="cpu").manual_seed(1)
    for wl_name, site_name, m, n, k in prefill_shapes():       # decode shapes: --decode-sweep
        xq = torch.randint(-127, 128, (m, k), dtype=torch.int8, generator=g).cuda()
        wq = torch.randint(-127, 128, (n, k), dtype=torch.int8, generator=g).cuda()
        xs = torch.rand(m, generator=g).cuda()
        ws = torch.rand(n, generator=g).cuda()
        y = torch.empty(m, n, dtype=torch.float16, device="cuda")
        t = best_ms(lambda: sq.sq_w8a8_gemm(xq, xs, wq, ws, y=y, out_dtype=torch.float16), prefill_reps(m, n, k))
        ops = 2.0 * m * n * k
        print(json.dumps({"workload": wl_name, "site": site_name, "mnk": [m, n, k],
                          "tiles": -(-m // 256) * -(-n // 256), "ms": round(t, 4),
                          "TOPS": round(ops / t / 1e9, 1)}), flush=True)
        del xq, wq, y
        torch.cuda.empty_cache()


PREFILL_CMD = "rocprofv3 --kernel-trace -d <dir> -o run --output-format csv -- python3 bench.py --prefill-sweep"


def prefill_shapes():
    """(workload, site, m, n, k) of every prefill GEMM, in --prefill-sweep order."""
    from synth import WORKLOADS
    out = []
    for wl_id in sorted(WORKLOADS):
        wl = WORKLOADS[wl_id]
        m = max(wl.m)
        if m > 64:
            out += [(wl.name, site.name, m, site.n, site.k) for site in wl.sites]
    return out


def summarize_prefill(trace_dir):
    """Per-shape durations of this library's GEMM in a --prefill-sweep kernel trace. Dispatches are
    taken in start order; each shape's launches are the next PREFILL_WARM + PREFILL_TIMES * reps
    GEMM dispatches."""
    import glob
    import statistics
    hits = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    rows = sorted((r for r in _read_csv(hits[0]) if "sq::k_gemm" in r["Kernel_Name"]),
                  key=lambda r: int(r["Start_Timestamp"]))
    shapes = prefill_shapes()
    counts = [PREFILL_WARM + PREFILL_TIMES * prefill_reps(m, n, k) for _, _, m, n, k in shapes]
    if len(rows) != sum(counts):
        raise SystemExit(f"{len(rows)} GEMM dispatches, expected {sum(counts)}")
    runs, at = [], 0
    for c in counts:
        rs = rows[at:at + c]
        at += c
        wg = int(rs[0].get("Workgroup_Size_X") or 1)
        runs.append({"name": rs[0]["Kernel_Name"].split("(")[0].replace("void ", ""),
                     "grid": int(rs[0]["Grid_Size_X"]) // wg, "wg": wg,
                     "ns": [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs]})
    lines = ["# Prefill GEMM kernel durations (rocprofv3 kernel trace): every workload's prefill sites, fp16 out",
             "", f"Command: `{PREFILL_CMD}`, then `python bench.py --summarize-prefill <dir>`.", "",
             "Random int8 operands; every launch of the sweep (warm-up included), back to back. The grid is "
             "one workgroup per 256x256 tile, or (up to 16 tiles per resident workgroup) one per CU looping "
             "over the tiles.", "",
             "| workload | site | M x N x K | kernel | workgroups x threads | launches | median ms | min ms | "
             "TOPS (median) |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (wl, site, m, n, k), run in zip(shapes, runs):
        med = statistics.median(run["ns"]) / 1e6
        lines.append(f"| {wl} | {site} | {m} x {n} x {k} | `{run['name']}` | {run['grid']} x {run['wg']} | "
                     f"{len(run['ns'])} | {med:.4f} | {min(run['ns']) / 1e6:.4f} | "
                     f"{2.0 * m * n * k / med / 1e9:.1f} |")
    with open(os.path.join(ROOT, "profiles", "prefill_gemm_all_workloads.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def median_ms(torch, fn, n):
    """Median of n launches of fn, each between a pair of HIP events, after one untimed launch."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2]


def granularity_sweep(args):
    """Per-token vs per-tensor dynamic vs static activation steps, INT8 and FP8 (and per-channel vs
    per-tensor weight steps in the fold) on the MT-NLG-width sites, HIP-event medians over 20 launches
    (fold: 5)."""
    import torch
    import w8a8_int8_linear_amd as sq
    from synth import WORKLOADS
    wl = WORKLOADS[5]
    sites = build_sites(torch, sq, wl, wl.m[0])

    def med(fn, n):
        return median_ms(torch, fn, n)

    for d in sites:
        m, k, n, norm = d["m"], d["k"], d["n"], d["norm"]
        amax = sq.smoothquant_calibrate(d["x_cal"], norm, d["gamma"], d["beta"], EPS)
        fo = sq.smoothquant_fold(amax, d["w"], wl.alpha, EPS, norm, d["gamma"], d["beta"])
        stp = sq.sq_static_step(amax, fo["s"])
        g, b = fo["gamma_f"], fo["beta_f"]
        e = d["x"].element_size()
        nq_bytes = m * k * e + m * k + 4 * m + 4 * k * (2 if b is not None else 1)
        stp8 = sq.sq_static_step_fp8(amax, fo["s"])
        xq8 = torch.empty(m, k, dtype=torch.uint8, device="cuda")
        runs = [("per-token", lambda: sq.sq_norm_quant(d["x"], norm, g, b, EPS, d["xq"], d["xs"])),
                ("per-tensor dynamic (2 passes)",
                 lambda: sq.sq_norm_quant_per_tensor(d["x"], norm, g, b, EPS, d["xq"], d["xs"])),
                ("per-tensor static", lambda: sq.sq_norm_quant_static(d["x"], stp, norm, g, b, EPS, d["xq"], d["xs"])),
                ("FP8 per-token", lambda: sq.sq_norm_quant_fp8(d["x"], norm, g, b, EPS, xq8, d["xs"])),
                ("FP8 per-tensor dynamic (2 passes)",
                 lambda: sq.sq_norm_quant_fp8_per_tensor(d["x"], norm, g, b, EPS, xq8, d["xs"])),
                ("FP8 per-tensor static",
                 lambda: sq.sq_norm_quant_fp8_static(d["x"], stp8, norm, g, b, EPS, xq8, d["xs"]))]
        for name, fn in runs:
            ms = med(fn, 20)
            print(json.dumps({"stage": "norm_quant", "granularity": name, "site": d["site"].name, "shape": [m, k],
                              "ms": round(ms, 4), "GBps": round(nq_bytes / ms / 1e6, 1)}), flush=True)
        fold_bytes = 2 * n * k * e + n * k + 4 * n + 16 * k
        f8 = {key: (torch.empty_like(v, dtype=torch.uint8) if key == "wq" else torch.empty_like(v))
              for key, v in d["fold"].items()}
        for name, fn in [("per-channel", lambda: sq.smoothquant_fold(amax, d["w"], wl.alpha, EPS, norm, d["gamma"],
                                                                      d["beta"], out=d["fold"])),
                         ("per-tensor (3 weight passes)",
                          lambda: sq.smoothquant_fold_per_tensor(amax, d["w"], wl.alpha, EPS, norm, d["gamma"],
                                                                 d["beta"], out=d["fold"])),
                         ("FP8 per-tensor (3 weight passes)",
                          lambda: sq.smoothquant_fold_fp8_per_tensor(amax, d["w"], wl.alpha, EPS, norm, d["gamma"],
                                                                     d["beta"], out=f8))]:
            ms = med(fn, 5)
            print(json.dumps({"stage": "fold", "granularity": name, "site": d["site"].name, "shape": [n, k],
                              "ms": round(ms, 4), "GBps": round(fold_bytes / ms / 1e6, 1)}), flush=True)


def kernel_stats_table(trace_dir, title, cmd, flag, note, out_name):
    """A rocprofv3 --kernel-trace --stats run's per-kernel statistics as a profiles/ table."""
    import glob
    hits = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no kernel stats under {trace_dir}")
    lines = [f"# rocprofv3 kernel statistics: {title}", "",
             f"Command: `{cmd}`, then `python bench.py {flag} <dir>`.", "", note, "",
             "| kernel | calls | average ms | min ms | max ms |", "|---|---|---|---|---|"]
    for r in _read_csv(hits[0]):
        if "sq::" in r["Name"]:
            short = r["Name"].split("(")[0].replace("void ", "")
            lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                         f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} |")
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_granularities(trace_dir):
    """Kernel statistics of a --granularities run as a profiles/ table."""
    kernel_stats_table(
        trace_dir, "activation and weight step granularities, MT-NLG-530B-width sites", GRAN_CMD,
        "--summarize-granularities",
        "Sites: LayerNorm 8192x20480 -> fc1 and NONE 8192x81920 -> fc2 (fp16), folds of their weights "
        "(81920x20480, 20480x81920). The last template argument of `k_norm_quant` is its mode: 0 one INT8 step "
        "per row, 1 the rows' maxima (first per-tensor pass), 2 INT8 codes with a step given for the whole "
        "tensor (second per-tensor pass, or a static step), 3 one FP8 step per row, 4 FP8 codes with a given "
        "step (saturated to +-448); `k_tensor_step` reduces the rows' maxima to the tensor step (/127 or /448). "
        "Each kernel's rows mix the activation passes and the fold's weight passes.",
        "kernel_stats_granularities_mtnlg530b.md")


# ----------------------------------------------------------------------------- FP8 (E4M3) against INT8

FP8_CMD = ("rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
           "python3 bench.py --fp8")


def fp8_sweep(args):
    """INT8 against FP8 (OCP E4M3) for each stage of the MT-NLG-width sites, HIP-event medians over
    20 launches (fold: 5). Both GEMMs are priced against the same 5.0 POP/s dense peak."""
    import torch
    import w8a8_int8_linear_amd as sq
    from synth import WORKLOADS
    wl = WORKLOADS[5]
    sites = build_sites(torch, sq, wl, wl.m[0])
    for d in sites:
        m, k, n, norm = d["m"], d["k"], d["n"], d["norm"]
        amax = sq.smoothquant_calibrate(d["x_cal"], norm, d["gamma"], d["beta"], EPS)
        f8 = {key: (torch.empty_like(v, dtype=torch.uint8) if key == "wq" else torch.empty_like(v))
              for key, v in d["fold"].items()}
        fo = sq.smoothquant_fold(amax, d["w"], wl.alpha, EPS, norm, d["gamma"], d["beta"], out=d["fold"])
        sq.smoothquant_fold_fp8(amax, d["w"], wl.alpha, EPS, norm, d["gamma"], d["beta"], out=f8)
        g, b = fo["gamma_f"], fo["beta_f"]
        xq8 = torch.empty(m, k, dtype=torch.uint8, device="cuda")
        xs8 = torch.empty(m, dtype=torch.float32, device="cuda")
        e = d["x"].element_size()
        o = d["y"].element_size()
        sizes = {"norm_quant": m * k * e + m * k + 4 * m + 4 * k * (2 if b is not None else 1),
                 "fold": 2 * n * k * e + n * k + 4 * n + 16 * k,
                 "gemm": n * k + 4 * n + m * k + 4 * m + o * m * n}
        stages = [
            ("norm_quant", "int8", 20, lambda: sq.sq_norm_quant(d["x"], norm, g, b, EPS, d["xq"], d["xs"])),
            ("norm_quant", "fp8", 20, lambda: sq.sq_norm_quant_fp8(d["x"], norm, g, b, EPS, xq8, xs8)),
            ("fold", "int8", 5, lambda: sq.smoothquant_fold(amax, d["w"], wl.alpha, EPS, norm, d["gamma"], d["beta"],
                                                            out=d["fold"])),
            ("fold", "fp8", 5, lambda: sq.smoothquant_fold_fp8(amax, d["w"], wl.alpha, EPS, norm, d["gamma"],
                                                               d["beta"], out=f8)),
            ("gemm", "int8", 20, lambda: sq.sq_w8a8_gemm(d["xq"], d["xs"], fo["wq"], fo["w_scale"], y=d["y"],
                                                         out_dtype=d["y"].dtype)),
            ("gemm", "fp8", 20, lambda: sq.sq_fp8_gemm(xq8, xs8, f8["wq"], f8["w_scale"], y=d["y"],
                                                       out_dtype=d["y"].dtype)),
        ]
        for stage, fmt, reps, fn in stages:
            ms = median_ms(torch, fn, reps)
            rec = {"stage": stage, "format": fmt, "site": d["site"].name, "ms": round(ms, 4),
                   "GBps": round(sizes[stage] / ms / 1e6, 1)}
            if stage == "gemm":
                tops = 2.0 * m * n * k / ms / 1e9
                rec.update(shape=[m, n, k], TOPS=round(tops, 1), frac=round(tops / 5000.0, 4))
            else:
                rec["shape"] = [m, k] if stage == "norm_quant" else [n, k]
            print(json.dumps(rec), flush=True)
        del f8, xq8, xs8
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- LLM.int8() against SmoothQuant

LLM_TAU = 6.0          # the outlier threshold on the LLM.int8() page ("going deeper", tau = 6)
LLM_CMD = ("rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
           "python3 bench.py --llm-int8")


def llm_int8_sweep(args):
    """The run-time path of SmoothQuant (fused norm + per-token INT8 quantiser, then the INT8 GEMM with
    its epilogue, on the folded parameters) beside LLM.int8()'s decomposition of the same linear (its
    whole run-time call: per-channel maxima of the batch, outlier selection, quantiser, 16-bit gather,
    INT8 GEMM into binary32, 16-bit product and merge), on every site of the OPT-6.7B and MT-NLG-530B-
    width workloads. Offline work (calibration and fold; LLM.int8()'s weight quantisation) is done first
    and not timed. HIP-event medians of whole calls (MT-NLG: 5 launches, OPT: 20)."""
    import torch
    import w8a8_int8_linear_amd as sq
    from synth import WORKLOADS
    for wl_id in (2, 5):
        wl = WORKLOADS[wl_id]
        sites = build_sites(torch, sq, wl, wl.m[0])
        reps = 5 if wl_id == 5 else 20
        for d in sites:
            m, k, n, norm = d["m"], d["k"], d["n"], d["norm"]
            amax = sq.smoothquant_calibrate(d["x_cal"], norm, d["gamma"], d["beta"], EPS)
            fo = sq.smoothquant_fold(amax, d["w"], wl.alpha, EPS, norm, d["gamma"], d["beta"], out=d["fold"])
            wq, ws = sq.sq_norm_quant(d["w"], "none")
            work = torch.empty(sq.sq_llm_int8_workspace(m, n, k)["total"], dtype=torch.uint8, device="cuda")
            y2 = torch.empty_like(d["y"])

            def smoothquant():
                sq.sq_norm_quant(d["x"], norm, fo["gamma_f"], fo["beta_f"], EPS, d["xq"], d["xs"])
                sq.sq_w8a8_gemm(d["xq"], d["xs"], fo["wq"], fo["w_scale"], y=d["y"], out_dtype=d["y"].dtype)

            def llm_int8():
                sq.sq_llm_int8_linear(d["x"], d["w"], wq, ws, norm, d["gamma"], d["beta"], EPS, LLM_TAU,
                                      out_dtype=y2.dtype, y=y2, workspace=work)
            t_sq = median_ms(torch, smoothquant, reps)
            t_li = median_ms(torch, llm_int8, reps)
            count = sq.llm_int8_parts(work, m, n, k, d["w"].dtype)["count"]
            print(json.dumps({"workload": wl.name, "site": d["site"].name, "mnk": [m, n, k],
                              "outlier_channels": count, "smoothquant_ms": round(t_sq, 4),
                              "llm_int8_ms": round(t_li, 4), "llm_int8_over_smoothquant": round(t_li / t_sq, 3)}),
                  flush=True)
            del work, y2, wq, ws
            torch.cuda.empty_cache()
        del sites
        torch.cuda.empty_cache()


def summarize_llm_int8(trace_dir, sweep_log=None):
    """Kernel statistics of a --llm-int8 run as a profiles/ table; with the run's stdout (sweep_log),
    also its per-site HIP-event medians."""
    kernel_stats_table(
        trace_dir, "LLM.int8() decomposition beside the SmoothQuant run-time path, OPT-6.7B and MT-NLG-530B-width "
        "sites", LLM_CMD, "--summarize-llm-int8",
        "Per site, 20 (OPT-6.7B) or 5 (MT-NLG) timed calls plus one warm-up of each path, after the untimed "
        "offline work. SmoothQuant at run time: `k_norm_quant` (mode 0) then the INT8 GEMM. LLM.int8(): "
        "`k_fill_zero_f32` + the per-channel maxima (`k_calibrate` / `k_colmax`), `k_outlier_select`, "
        "`k_norm_quant` (mode 5 with a norm: also the row statistics; mode 0 without), `k_outlier_gather`, "
        "the INT8 GEMM into binary32, `k_outlier_merge`. The offline kernels (calibration, fold, weight "
        "quantisation) appear too; each kernel's row mixes every site it ran on.",
        "llm_int8_vs_smoothquant.md")
    if sweep_log:
        with open(sweep_log) as f:
            recs = [json.loads(ln) for ln in f if ln.startswith("{")]
        lines = ["", "Per site, HIP-event medians of whole calls in the same run (the profiler's overhead included):",
                 "", "| workload | site | M x N x K | outlier channels | SmoothQuant ms | LLM.int8() ms | ratio |",
                 "|---|---|---|---|---|---|---|"]
        for r in recs:
            m, n, k = r["mnk"]
            lines.append(f"| {r['workload']} | {r['site']} | {m} x {n} x {k} | {r['outlier_channels']} | "
                         f"{r['smoothquant_ms']:.4f} | {r['llm_int8_ms']:.4f} | {r['llm_int8_over_smoothquant']:.2f} |")
        with open(os.path.join(ROOT, "profiles", "llm_int8_vs_smoothquant.md"), "a") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))


def summarize_fp8(trace_dir):
    """Per-dispatch durations of a --fp8 kernel trace, grouped by kernel and grid (one kernel name
    serves both the activation quantiser and the fold's weight quantiser), as a profiles/ table."""
    import glob
    import statistics
    hits = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    groups = {}
    for r in _read_csv(hits[0]):
        if "sq::" not in r["Kernel_Name"]:
            continue
        short = r["Kernel_Name"].split("(")[0].replace("void ", "")
        wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        ms = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        groups.setdefault((short, wgs, r["Workgroup_Size_X"]), []).append(ms)
    lines = ["# rocprofv3 kernel trace: INT8 against FP8 (OCP E4M3), MT-NLG-530B-width sites", "",
             f"Command: `{FP8_CMD}`, then `python bench.py --summarize-fp8 <dir>`.", "",
             "Sites: LayerNorm 8192x20480 -> fc1 (N 81920) and NONE 8192x81920 -> fc2 (N 20480), fp16. "
             "`k_norm_quant` mode 0 is the INT8 per-token quantiser and mode 3 the FP8 one; with no norm the same "
             "kernel quantises the fold's weights (81920x20480, 20480x81920); where one grid serves both, the "
             "dispatches are split at their widest duration gap (the 20480-row weights take about 2.5x the "
             "8192-row activations). "
             "`k_gemm_tile` is the INT8 GEMM (v_mfma_i32_16x16x64_i8), `k_gemm_tile_fp8` the FP8 one "
             "(v_mfma_scale_f32_16x16x128_f8f6f4). Durations are per dispatch, start to end.", "",
             "| kernel | workgroups x threads | calls | median ms | min ms | max ms |",
             "|---|---|---|---|---|---|"]
    rows = []
    for (name, wgs, wgsize), v in groups.items():
        v = sorted(v)
        # one kernel and grid may serve two row counts: split at the widest duration gap above 1.5x
        # that leaves at least three dispatches on each side
        ratio, cut = max(((v[i + 1] / v[i], i + 1) for i in range(2, len(v) - 3) if v[i] > 0), default=(1.0, 0))
        parts = [v[:cut], v[cut:]] if ratio > 1.5 else [v]
        rows += [(name, wgs, wgsize, p) for p in parts]
    for name, wgs, wgsize, v in sorted(rows, key=lambda r: (-statistics.median(r[3]), r[0])):
        lines.append(f"| `{name}` | {wgs} x {wgsize} | {len(v)} | {statistics.median(v):.4f} | "
                     f"{min(v):.4f} | {max(v):.4f} |")
    with open(os.path.join(ROOT, "profiles", "kernel_trace_fp8_mtnlg530b.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ----------------------------------------------------------------------------- accuracy study

ALPHAS = (0.5, 0.65, 0.8, 0.9)


def reference_linear(torch, x, norm, gamma, beta, w, eps=EPS):
    """The unquantised layer in binary64: norm(x) (unfolded gamma, beta) times W^T."""
    x = x.double()
    if norm == "layernorm":
        mu = x.mean(dim=1, keepdim=True)
        var = ((x - mu) ** 2).mean(dim=1, keepdim=True)
        y = (x - mu) / torch.sqrt(var + eps) * gamma.double() + beta.double()
    elif norm == "rmsnorm":
        y = x / torch.sqrt((x * x).mean(dim=1, keepdim=True) + eps) * gamma.double()
    else:
        y = x
    return y @ w.double().t()


def ordinary_span(xq, outliers):
    """Median over tokens of the largest |code| among the non-outlier channels: how many of the
    127 positive levels the ordinary channels of a token actually reach."""
    import torch
    keep = torch.ones(xq.shape[1], dtype=torch.bool, device=xq.device)
    keep[torch.as_tensor(outliers, dtype=torch.long, device=xq.device)] = False
    return int(xq[:, keep].abs().amax(dim=1).median().item())


def ordinary_span_fp8(xq, outliers):
    """As ordinary_span for FP8 (E4M3) codes: the median over tokens of the largest decoded |code|
    among the non-outlier channels, out of 448."""
    import torch
    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().to(xq.device)
    keep = torch.ones(xq.shape[1], dtype=torch.bool, device=xq.device)
    keep[torch.as_tensor(outliers, dtype=torch.long, device=xq.device)] = False
    return float(table[xq[:, keep].long()].abs().amax(dim=1).median().item())


def accuracy_site(torch, sq, wl, si, m_tokens):
    """One site: relative output error and ordinary-channel span for each scheme."""
    from synth import site_inputs
    inp = site_inputs(wl.id, si, m=m_tokens, device="cuda")
    site = wl.sites[si]
    x, xc, w, g, b, norm = inp["x"], inp["x_cal"], inp["w"], inp["gamma"], inp["beta"], site.norm
    y_ref = reference_linear(torch, x, norm, g, b, w)
    ref_norm = torch.linalg.norm(y_ref).item()
    amax = sq.smoothquant_calibrate(xc, norm, g, b, EPS)
    wmax = sq.smoothquant_calibrate(w, "none")          # column max of |W|: as act_absmax at alpha 0.5 it gives s = 1
    out = []

    def run(scheme, alpha, act, fold_fn, a_in):
        fo = fold_fn(a_in, w, 0.5 if alpha is None else alpha, EPS, norm, g, b)
        gf, bf = fo["gamma_f"], fo["beta_f"]
        if act.startswith("fp8"):
            if act == "fp8":
                xq, xs = sq.sq_norm_quant_fp8(x, norm, gf, bf, EPS)
            elif act == "fp8 per-tensor":
                xq, xs = sq.sq_norm_quant_fp8_per_tensor(x, norm, gf, bf, EPS)
            else:
                xq, xs = sq.sq_norm_quant_fp8_static(x, sq.sq_static_step_fp8(a_in, fo["s"]), norm, gf, bf, EPS)
            y = sq.sq_fp8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float32)
            span = ordinary_span_fp8(xq, inp["outliers"])
        else:
            if act == "per-token":
                xq, xs = sq.sq_norm_quant(x, norm, gf, bf, EPS)
            elif act == "per-tensor":
                xq, xs = sq.sq_norm_quant_per_tensor(x, norm, gf, bf, EPS)
            else:
                xq, xs = sq.sq_norm_quant_static(x, sq.sq_static_step(a_in, fo["s"]), norm, gf, bf, EPS)
            y = sq.sq_w8a8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float32)
            span = ordinary_span(xq, inp["outliers"])
        err = torch.linalg.norm(y.double() - y_ref).item() / ref_norm
        out.append({"workload": wl.name, "site": site.name, "scheme": scheme, "alpha": alpha,
                    "rel_err": float(f"{err:.4g}"), "ordinary_span": span})

    run("plain INT8, per-tensor X and W", None, "per-tensor", sq.smoothquant_fold_per_tensor, wmax)
    run("plain INT8, per-token X, per-channel W", None, "per-token", sq.smoothquant_fold, wmax)
    for alpha in ALPHAS:
        run("SmoothQuant O3: static X, per-tensor W", alpha, "static", sq.smoothquant_fold_per_tensor, amax)
        run("SmoothQuant O2: per-tensor X and W", alpha, "per-tensor", sq.smoothquant_fold_per_tensor, amax)
        run("SmoothQuant, per-token X, per-channel W", alpha, "per-token", sq.smoothquant_fold, amax)
    if site.k % 128 == 0:
        run("plain FP8 (E4M3), per-token X, per-channel W", None, "fp8", sq.smoothquant_fold_fp8, wmax)
        for alpha in ALPHAS:
            run("SmoothQuant FP8 (E4M3), per-token X, per-channel W", alpha, "fp8", sq.smoothquant_fold_fp8, amax)
        run("SmoothQuant FP8 (E4M3) O2: per-tensor X and W", 0.5, "fp8 per-tensor",
            sq.smoothquant_fold_fp8_per_tensor, amax)
        run("SmoothQuant FP8 (E4M3) O3: static X, per-tensor W", 0.5, "fp8 static",
            sq.smoothquant_fold_fp8_per_tensor, amax)
    return out


def accuracy_study(args):
    """Plain INT8 against SmoothQuant over alpha on the synthetic stand-ins of every workload."""
    import torch
    import w8a8_int8_linear_amd as sq
    from synth import WORKLOADS
    for wl_id in sorted(WORKLOADS):
        wl = WORKLOADS[wl_id]
        m = min(max(wl.m), args.accuracy_tokens)
        for si in range(len(wl.sites)):
            for rec in accuracy_site(torch, sq, wl, si, m):
                print(json.dumps(rec), flush=True)
            torch.cuda.empty_cache()


class Timer:
    """HIP events on the stream the library launches on, one pair per launch."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def run(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.ev.setdefault(name, []).append((s, e))

    def mean_ms(self, name):
        pairs = self.ev.get(name, [])
        return sum(s.elapsed_time(e) for s, e in pairs) / max(1, len(pairs))

    def reset(self):
        self.ev = {}


def build_sites(torch, sq, wl, m):
    from synth import site_inputs
    sites = []
    out_dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.out_dtype]
    for si, site in enumerate(wl.sites):
        inp = site_inputs(wl.id, si, m=m, device="cuda")
        k, n = site.k, site.n
        d = dict(inp, norm=site.norm, k=k, n=n, m=m,
                 absmax=torch.zeros(k, dtype=torch.float32, device="cuda"),
                 fold=None,
                 xq=torch.empty(m, k, dtype=torch.int8, device="cuda"),
                 xs=torch.empty(m, dtype=torch.float32, device="cuda"),
                 y=torch.empty(m, n, dtype=out_dt, device="cuda"))
        d["fold"] = {"s": torch.empty(k, dtype=torch.float32, device="cuda"),
                     "gamma_f": torch.empty(k, dtype=torch.float32, device="cuda"),
                     "wq": torch.empty(n, k, dtype=torch.int8, device="cuda"),
                     "w_scale": torch.empty(n, dtype=torch.float32, device="cuda")}
        if inp["beta"] is not None:
            d["fold"]["beta_f"] = torch.empty(k, dtype=torch.float32, device="cuda")
        sites.append(d)
    torch.cuda.synchronize()
    return sites


def step(sq, wl, sites, timer):
    for i, d in enumerate(sites):
        d["absmax"].zero_()
        timer.run(f"calibrate{i}", lambda: sq.smoothquant_calibrate(d["x_cal"], d["norm"], d["gamma"], d["beta"],
                                                                    EPS, absmax=d["absmax"]))
        timer.run(f"fold{i}", lambda: sq.smoothquant_fold(d["absmax"], d["w"], wl.alpha, EPS, d["norm"], d["gamma"],
                                                          d["beta"], out=d["fold"]))
        f = d["fold"]
        timer.run(f"norm_quant{i}", lambda: sq.sq_norm_quant(d["x"], d["norm"], f["gamma_f"], f.get("beta_f"), EPS,
                                                             xq=d["xq"], x_scale=d["xs"]))
        timer.run(f"gemm{i}", lambda: sq.sq_w8a8_gemm(d["xq"], d["xs"], f["wq"], f["w_scale"], y=d["y"],
                                                      out_dtype=d["y"].dtype))


def kernel_report(timer, wl, sites):
    esize = {"f32": 4, "f16": 2, "bf16": 2}[wl.dtype]
    osize = {"f32": 4, "f16": 2, "bf16": 2}[wl.out_dtype]
    rep = {}
    for i, d in enumerate(sites):
        m, n, k = d["m"], d["n"], d["k"]
        nparams = 0 if d["norm"] == "none" else (2 if d["norm"] == "layernorm" else 1)
        t = timer.mean_ms(f"gemm{i}")
        ops = 2.0 * m * n * k
        gbytes = n * k + 4 * n + m * k + 4 * m + osize * m * n
        rep[f"gemm{i}"] = {"shape": [m, n, k], "ms": t, "TOPS": ops / t / 1e9, "GBps": gbytes / t / 1e6}
        t = timer.mean_ms(f"norm_quant{i}")
        b = m * k * esize + m * k + 4 * m + 4 * k * (nparams if nparams else 1)
        rep[f"norm_quant{i}"] = {"shape": [m, k], "ms": t, "GBps": b / t / 1e6}
        t = timer.mean_ms(f"calibrate{i}")
        b = wl.m_cal * k * esize + 4 * k
        rep[f"calibrate{i}"] = {"shape": [wl.m_cal, k], "ms": t, "GBps": b / t / 1e6}
        t = timer.mean_ms(f"fold{i}")
        b = 2 * n * k * esize + n * k + 4 * n + 16 * k
        rep[f"fold{i}"] = {"shape": [n, k], "ms": t, "GBps": b / t / 1e6}
    return rep


def cpu_baseline(wl, budget_s):
    """The oracle on a bounded sample of the workload, stage by stage, on the host cores: calibration,
    fold, norm + quantise (GB/s of the stage's algorithmic bytes) and the INT8 GEMM with its epilogue
    (TOPS). BLAS threads are set to the cores this process may use (OMP_NUM_THREADS when set); all
    else is single-threaded numpy and Python. The sample is every site of the workload at its full K
    (the first site's norm, activations and weights), with few enough rows that the whole leg takes
    about budget_s seconds."""
    import numpy as np
    import oracle as O
    from synth import site_inputs, to_numpy
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    esize = {"f32": 4, "f16": 2, "bf16": 2}[wl.dtype]
    osize = {"f32": 4, "f16": 2, "bf16": 2}[wl.out_dtype]
    m_s, n_s, cal_s, gm_s = 8, 256, 16, 256           # rows of each stage's sample
    acc = {k: [0.0, 0.0] for k in ("calibrate", "fold", "norm_quant", "gemm")}   # seconds, work
    reps = 0
    t_start = time.perf_counter()
    with threadpool_limits(limits=threads):
        while True:
            for si, site in enumerate(wl.sites):
                k = site.k
                inp = site_inputs(wl.id, si, m=max(m_s, gm_s), device="cpu", w_rows=n_s)
                x = to_numpy(inp["x"])
                x_cal = to_numpy(inp["x_cal"][:cal_s])
                w = to_numpy(inp["w"])
                gamma = None if inp["gamma"] is None else inp["gamma"].numpy()
                beta = None if inp["beta"] is None else inp["beta"].numpy()
                nparams = {"none": 1, "layernorm": 2, "rmsnorm": 1}[site.norm]
                t0 = time.perf_counter()
                a, _ = O.calibrate(x_cal, wl.dtype, site.norm, gamma, beta, EPS)
                t1 = time.perf_counter()
                f = O.fold(a, w, wl.dtype, wl.alpha, O.EPS_FOLD, site.norm, gamma, beta)
                t2 = time.perf_counter()
                xq, xs, _ = O.norm_quant(x[:m_s], wl.dtype, site.norm, f["gamma_f"], f["beta_f"], EPS)
                t3 = time.perf_counter()
                xq_g = np.resize(xq, (gm_s, k))              # the GEMM stage on gm_s token rows
                xs_g = np.resize(xs, gm_s)
                O.dequantize(O.int_gemm(xq_g, f["wq"]), xs_g, f["w_scale"], None, wl.out_dtype)
                t4 = time.perf_counter()
                acc["calibrate"][0] += t1 - t0
                acc["calibrate"][1] += cal_s * k * esize + 4 * k
                acc["fold"][0] += t2 - t1
                acc["fold"][1] += 2 * n_s * k * esize + n_s * k + 4 * n_s + 16 * k
                acc["norm_quant"][0] += t3 - t2
                acc["norm_quant"][1] += m_s * k * esize + m_s * k + 4 * m_s + 4 * k * nparams
                acc["gemm"][0] += t4 - t3
                acc["gemm"][1] += 2.0 * gm_s * n_s * k
            reps += 1
            if time.perf_counter() - t_start >= budget_s or reps >= 50:
                break
    stages = {name: {"value": round(work / sec / (1e12 if name == "gemm" else 1e9), 6),
                     "unit": "TOPS" if name == "gemm" else "GB/s", "seconds": round(sec, 3)}
              for name, (sec, work) in acc.items()}
    sample = (f"{reps} x every site at full K: calibration on {cal_s} tokens, fold of {n_s} weight rows, "
              f"norm+quantise of {m_s} tokens, GEMM + epilogue of {gm_s} tokens x {n_s} output channels")
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": stages["gemm"]["value"], "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": sample, "stages": stages, "blas_threads": threads, "host_cpus": cores, "cpu_model": model,
            "seconds": round(sum(sec for sec, _ in acc.values()), 3),
            "note": "value is the GEMM stage; BLAS (the binary64 matrix product of the integer codes) runs on "
                    "blas_threads threads, everything else single-threaded numpy"}


def main():
    args = parse()
    if args.summarize_counters:
        if len(args.summarize_counters) not in (3, 4):
            raise SystemExit("--summarize-counters TRACE_DIR FETCH_DIR WRITE_DIR [CLOCK_DIR]")
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_decode:
        summarize_decode(args.summarize_decode, args.fp8)
        return
    if args.summarize_granularities:
        summarize_granularities(args.summarize_granularities)
        return
    if args.summarize_fp8:
        summarize_fp8(args.summarize_fp8)
        return
    if args.summarize_decode_counters:
        summarize_decode_counters(args.summarize_decode_counters)
        return
    if args.summarize_ln_counters:
        summarize_ln_counters(args.summarize_ln_counters)
        return
    if args.summarize_ln_waits:
        summarize_ln_waits(args.summarize_ln_waits)
        return
    if args.summarize_prefill:
        summarize_prefill(args.summarize_prefill)
        return
    if args.summarize_llm_int8:
        summarize_llm_int8(*args.summarize_llm_int8[:2])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark measures one GPU; runs on several GPUs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.decode_sweep:
        decode_sweep(args.fp8)
        return
    if args.prefill_sweep:
        prefill_sweep()
        return
    if args.llm_int8:
        llm_int8_sweep(args)
        return
    if args.granularities:
        granularity_sweep(args)
        return
    if args.fp8:
        fp8_sweep(args)
        return
    if args.accuracy:
        accuracy_study(args)
        return
    import torch
    import w8a8_int8_linear_amd as sq
    from synth import WORKLOADS

    wl = WORKLOADS[args.workload]
    m = args.m if args.m is not None else wl.m[0]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)
    print(f"# building inputs for {wl.name} (M={m})", file=sys.stderr, flush=True)
    sites = build_sites(torch, sq, wl, m)
    timer = Timer(torch)
    for _ in range(args.warmup):
        step(sq, wl, sites, timer)
    torch.cuda.synchronize()
    timer.reset()
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(sq, wl, sites, timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    ms = (t1 - t0) * 1e3 / args.steps
    rep = kernel_report(timer, wl, sites)
    dims = [(d["m"], d["n"], d["k"]) for d in sites]
    clock = None
    if not args.no_clock:
        # the shader clock while site 0's GEMM runs back to back for about half a second
        d0 = sites[0]
        try:
            sampler = ClockSampler()
            mhz = sampler.run_while(torch, lambda: sq.sq_w8a8_gemm(d0["xq"], d0["xs"], d0["fold"]["wq"],
                                                                   d0["fold"]["w_scale"], y=d0["y"],
                                                                   out_dtype=d0["y"].dtype), 0.6)
            mhz.sort()
            clock = {"source": "sysfs pp_dpm_sclk current level, sampled every ~2 ms during back-to-back "
                               f"launches of the {d0['m']}x{d0['n']}x{d0['k']} GEMM after the timed steps",
                     "samples": len(mhz), "median_GHz": round(mhz[len(mhz) // 2] / 1e3, 3) if mhz else None,
                     "min_GHz": round(mhz[0] / 1e3, 3) if mhz else None,
                     "max_GHz": round(mhz[-1] / 1e3, 3) if mhz else None}
            w = sorted(sampler.watts)
            if w:
                clock["board_power_W"] = {"source": f"sysfs hwmon {os.path.basename(sampler.power_path)}, same loop",
                                          "samples": len(w), "median": round(w[len(w) // 2], 1),
                                          "max": round(w[-1], 1), "cap": sampler.cap_watts()}
        except Exception as e:        # no clock reading on this host: say so
            clock = {"error": f"{type(e).__name__}: {e}"}
    del sites
    torch.cuda.empty_cache()
    decode = None if args.no_decode else decode_block(torch, sq)
    g_ops = [2.0 * dm * dn * dk for dm, dn, dk in dims]
    value = sum(g_ops) / (ms * 1e-3) / 1e12
    g_ms = [rep[f"gemm{i}"]["ms"] for i in range(len(dims))]
    achieved = sum(g_ops) / (sum(g_ms) * 1e-3) / 1e12
    osize = {"f32": 4, "f16": 2, "bf16": 2}[wl.out_dtype]
    alg_bytes = [dn * dk + 4 * dn + dm * dk + 4 * dm + osize * dm * dn for dm, dn, dk in dims]
    rec = recorded_traffic() if args.workload == 5 and m == 8192 else None
    traffic = rec["traffic_bytes_per_launch"] if rec else None
    sclk = clock.get("median_GHz") if clock else None
    peak_sclk = PEAK_INT8_TOPS * sclk / PEAK_SCLK_GHZ if sclk else None
    out = {
        "metric": "W8A8 GEMM TOPS + % INT8 MFMA peak; norm+quant kernel HBM GB/s",
        "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8xint8->int32", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": m,
                   "sites": [f"{s.name}: K={s.k} N={s.n} norm={s.norm}" for s in wl.sites],
                   "alpha": wl.alpha, "act_dtype": wl.dtype, "out_dtype": wl.out_dtype, "m_cal": wl.m_cal},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_tile", "achieved": round(achieved, 1),
                     "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": traffic, "traffic_unit": "HBM bytes per launch",
                     "sclk_GHz": round(sclk, 3) if sclk else None,
                     "sclk_measured": clock,
                     "peak_at_sclk": round(peak_sclk, 1) if sclk else None,
                     "frac_at_sclk": round(achieved / peak_sclk, 4) if sclk else None,
                     "counter_record": ({"sclk_GHz": round(rec["sclk_GHz"], 3), "mfma_busy": round(rec["mfma_busy"], 3),
                                         "file": "profiles/k_gemm_tile_traffic.json"}
                                        if rec and "mfma_busy" in rec else None),
                     "algorithmic_bytes_per_launch": sum(alg_bytes) / len(alg_bytes),
                     "ops_per_launch": sum(g_ops) / len(g_ops)},
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in rep.items()},
        "hbm_peak_GBps": PEAK_HBM_GBS,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
