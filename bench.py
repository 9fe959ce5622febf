"""Benchmark of the streamed AllGather + GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--case 4]

A step is one ag_gemm call: plan, producer (side stream) moving the remote
shards' chunks into the workspace and releasing them on the per-source
counters, the persistent MFMA consumer computing C as chunks arrive, and the
join of the two streams.  Inputs are resident in HBM before the timed
region; the workspace is caller-owned so nothing is allocated inside it.

Workload (default): fp16 x fp16 -> fp32, 8 shards of 1024 rows, M=8192,
K=4096, N=4096, A and B ~ N(0,1) from the seeded generator, automatic chunk
size (16 rows, 64 chunks per source), unpaced producer.

Order of the run: the timed steps come first (after about 0.3 s of untimed
calls that bring the clocks out of idle, then W warm-up steps), so that no
earlier measurement has heated the board; then every workload's entry
(C1-C5: pipelined steps and the four modes taken in turn), the variants,
the ring runs, the vendor-GEMM reference and, last, the same pipelined
steps again after all of that ("sustained").

Printed: ONE JSON line with the metric (TFLOPS = 2MKN/t), the roofline of the
consumer kernel (its own average duration, taken with HIP events recorded
around every fifth timed launch on the stream it runs on; also the median
and minimum), the oracle's CPU throughput on a bounded sample of the same
workload (plus one-thread rates on C1-C3), the overlap figures of every
workload and the GFX clocks that amd-smi reads while pipelined calls keep
the GPU busy.

The roofline's "traffic" (HBM bytes per consumer launch) comes from hardware
counters, which this script cannot read itself: rocprofv3 --pmc runs of
FETCH_SIZE and WRITE_SIZE over this script, scaled by what the same counters
read for a plain device copy of known size (``--copy-calibration``), are
kept in profiles/ together with a digest of the consumer's sources; the
figure is reported only while those sources are unchanged.

Helpers for those runs:
    python bench.py --copy-calibration      a 256 MiB device copy, 10 times
    python bench.py --mfma-probe            the register-only matrix-core probe
                                            (fp16 and fp8, random against
                                            constant operands): TFLOP/s, GFX
                                            clocks and board power under load
    python bench.py --load-probe            the operand-movement probe: one
                                            64 KiB K slice per CU into LDS
                                            and 192 KiB out of it, per
                                            iteration, in several patterns
    python bench.py --only KIND             only KIND's timed steps (f16 of
                                            --case, bf16, fp8 or i8) in --mode
    python bench.py --pmc-summary DIR       mean counter value per dispatch
                                            and kernel, from rocprofv3 CSVs
    python bench.py --trace-summary DIR     per-kernel durations from a
                                            rocprofv3 kernel trace, over all
                                            dispatches and over the first
                                            --steps ones after --skip
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS (2MKN/t) and % of MFMA peak for streamed AG-GEMM; overlap efficiency"
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, published
PEAK_I8_TOPS = 5000.0        # MI355X dense int8 MFMA, published
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0
# PTO-ISA AllGather+GEMM README, 8-card table, 8192x4096x4096 fp16 -> fp32 on
# Ascend 910B1 (each rank computes all of C): other hardware, context only.
PAGE_TFLOPS_8192 = 191.03

# counter-derived traffic of the consumer on the default workload
TRAFFIC_NOTE = os.path.join(ROOT, "profiles", "consumer_f16_8x1024x4096x4096_traffic.md")
CONSUMER_SOURCES = ["consumer.hip", "kernels.hpp", "schedule.hpp", "sync.hpp"]
COPY_CALIBRATION_BYTES = 256 << 20
MODES = {"pipelined": 0, "compute": 1, "sequential": 2, "copy": 3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--case", type=int, default=4, help="workload id (see synth.CASES)")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--link-gbps", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="only the timed steps (and the CPU baseline)")
    ap.add_argument("--no-int8", action="store_true", help="skip the int8 workload")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16 variant")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 variant")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip reading the GFX clocks with amd-smi under load")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip the ring-variant runs (D = 2, 4, 8)")
    ap.add_argument("--no-chunk-sweep", action="store_true",
                    help="skip the pipelined chunk-size sweep")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the producer variants (DMA engines, reserved CUs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--ramp-calls", type=int, default=1000,
                    help="untimed calls before the warm-up that bring the clocks out of idle")
    ap.add_argument("--skip", type=int, default=0,
                    help="--trace-summary: dispatches of each kernel before the timed ones")
    ap.add_argument("--mode", choices=sorted(MODES), default="pipelined",
                    help="mode of the timed calls; hardware-counter runs use 'compute' "
                         "because counter collection serializes the two kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the register-only matrix-core probe")
    ap.add_argument("--load-probe", action="store_true",
                    help="only run the operand-movement probe (loads into LDS, LDS reads)")
    ap.add_argument("--only", choices=("bf16", "fp8", "i8"),
                    help="only this variant's timed steps, in --mode (for counter runs)")
    ap.add_argument("--vendor-only", action="store_true",
                    help="only time hipBLASLt (torch.matmul) on the workload's gathered shape "
                         "(a reference for counter runs)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="summarise rocprofv3 counter CSVs under DIR and exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarise a rocprofv3 kernel trace under DIR and exit")
    return ap.parse_args()


def code_only(text):
    """C++ source without its comments and blank lines, each line stripped:
    what the compiler sees, so that an edited comment does not disown the
    counters taken on unchanged code.  (The sources quote no "//" or
    "/*" inside string literals.)"""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.strip() for ln in text.splitlines() if ln.strip())


def consumer_digest():
    h = hashlib.sha256()
    for name in CONSUMER_SOURCES:
        with open(os.path.join(ROOT, "communication_gemm_amd", "csrc", name)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()


def stored_traffic(workload, tile_id=None):
    """HBM bytes per consumer launch from the counter note, or None when the
    note is missing, is for another workload or tile, or predates the
    sources."""
    try:
        with open(TRAFFIC_NOTE) as f:
            kv = dict(line.strip()[2:].split(": ", 1) for line in f
                      if line.startswith("- ") and ": " in line)
    except OSError:
        return None
    if kv.get("consumer_sources_sha256") != consumer_digest():
        return None
    if kv.get("workload") != workload:
        return None
    if tile_id is not None and kv.get("tile_id") != str(tile_id):
        return None
    return float(kv["hbm_bytes_per_launch"])


def pmc_summary(root):
    """Mean of every counter per dispatch, by kernel, over rocprofv3's
    counter_collection CSV files under `root`."""
    acc = {}
    for path in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"),
                                 recursive=True)):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                key = (row["Kernel_Name"], row["Counter_Name"])
                s, n = acc.get(key, (0.0, 0))
                acc[key] = (s + float(row["Counter_Value"]), n + 1)
    for (kern, ctr), (s, n) in sorted(acc.items()):
        print(f"{ctr:16s} {s / n:18.1f}  dispatches={n:4d}  {kern}")


def trace_summary(root, steps, skip=0):
    """Per-kernel dispatch durations from rocprofv3's kernel_trace CSV: all
    dispatches, and the `steps` dispatches of each kernel that follow its
    first `skip` (in dispatch order; for the default run, the timed steps of
    the timed workload's consumer come after --ramp-calls + --warmup of
    its launches)."""
    rows = []
    for path in sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"),
                                 recursive=True)):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                rows.append((int(row["Dispatch_Id"]), row["Kernel_Name"],
                             int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
    rows.sort()
    by = {}
    for _, name, ns in rows:
        by.setdefault(name, []).append(ns)
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        part = d[skip:skip + steps] or d[-steps:]
        print(f"{len(d):5d} dispatches  mean {np.mean(d) / 1e3:9.1f} us  "
              f"[{skip}, {skip + len(part)}): mean {np.mean(part) / 1e3:9.1f} us  "
              f"median {np.median(part) / 1e3:8.1f}  min {min(part) / 1e3:8.1f}  "
              f"max {max(part) / 1e3:8.1f}  {name[:110]}")


def copy_calibration(torch):
    x = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(10):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_CALIBRATION_BYTES, "copies": 10,
                      "expected_fetch_KiB": COPY_CALIBRATION_BYTES / 1024,
                      "expected_write_KiB": COPY_CALIBRATION_BYTES / 1024}), flush=True)


TIMED_STRIDE = 5     # one timed call in five carries a consumer event pair


def timed(torch, make, steps, warmup, with_consumer=True, per_call=None):
    """Run `warmup` untimed calls, then time `steps` calls back to back.

    make(events) returns a zero-argument call; events is None or a pair of
    torch events that the library records around the consumer launch, on
    the stream the consumer runs on.  One timed call in TIMED_STRIDE (the
    first of every five) carries a pair: recorded around every call, the
    pairs made the pipelined C4 step about 9 us (3%) longer.  Returns (ms
    per call, mean consumer ms or None); per_call, if a list, receives the
    consumer ms of every bracketed call."""
    plain = make(None)
    for _ in range(warmup):
        plain()
    torch.cuda.synchronize()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             if with_consumer and i % TIMED_STRIDE == 0 else None for i in range(steps)]
    # torch creates an event's HIP handle at its first record; do that now so
    # the library can record the consumer pairs itself
    for pr in pairs:
        if pr is not None:
            pr[0].record()
            pr[1].record()
    calls = [plain if pr is None else make(pr) for pr in pairs]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for c in calls:
        c()
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end) / steps
    cons = None
    if with_consumer:
        each = [pr[0].elapsed_time(pr[1]) for pr in pairs if pr is not None]
        cons = float(np.mean(each))
        if per_call is not None:
            per_call.extend(each)
    return total, cons


def ramp(torch, call, calls=0, seconds=0.0):
    """Untimed calls that bring the clocks out of their idle state (after a
    pause, such as the host drawing a workload's inputs, the first tens of
    calls run at lower clocks): `calls` of them, or as many as take about
    `seconds`."""
    t0 = time.perf_counter()
    i = 0
    while i < calls or (seconds > 0 and time.perf_counter() - t0 < seconds):
        call()
        i += 1
        if i % 100 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def interleaved(torch, calls, rounds=5, n=20):
    """The four modes taken in turn: `rounds` rounds of `n` calls of each
    mode, then the medians.  Runs taken next to each other compare the
    modes more fairly than long blocks, over which the board's clocks drift
    with its load.  Hidden fraction, overlap efficiency and speedup follow
    the readings of the PTO-ISA README's benchmark output (it prints an
    "overlap eff" without a formula)."""
    inter = {"compute": [], "copy": [], "sequential": [], "pipelined": []}
    for _ in range(rounds):
        for name in inter:
            t, _ = timed(torch, lambda ev, c=calls[name]: c, n, 2, with_consumer=False)
            inter[name].append(t)
    mi = {k: float(np.median(v)) for k, v in inter.items()}
    return {**{f"{k}_ms": round(v, 5) for k, v in mi.items()},
            "hidden_fraction": round((mi["compute"] + mi["copy"] - mi["pipelined"]) / mi["copy"], 4),
            "overlap_eff": round((mi["sequential"] - mi["pipelined"])
                                 / min(mi["copy"], mi["compute"]), 4),
            "speedup_vs_sequential": round(mi["sequential"] / mi["pipelined"], 4),
            "note": f"medians of {rounds} rounds of {n} calls per mode, the modes taken in turn"}


def device_trace(torch, agg, call_with_trace, info):
    """One pipelined call with the device trace on: how long consumer tiles
    waited for chunks and when the last chunk landed."""
    trace = torch.zeros(info.trace_words, dtype=torch.int64, device="cuda")
    call_with_trace(trace)
    if agg.check():
        raise SystemExit("traced run failed")
    tr = trace.cpu().numpy().view(np.uint64).astype(np.float64)
    nc = info.total_chunks
    start, rel, cons = tr[0], tr[1:1 + nc], tr[1 + nc:].reshape(-1, 3)
    waits = cons[:, 1] - cons[:, 0]
    return {
        "tile_wait_share": round(float(waits.sum() / (cons[:, 2] - cons[:, 0]).sum()), 4),
        "mean_tile_wait_us": round(float(waits.mean()) / 100.0, 2),
        "max_tile_wait_us": round(float(waits.max()) / 100.0, 2),
        "last_release_us": round(float(rel.max() - start) / 100.0, 2) if nc else 0.0,
        "consumer_span_us": round(float(cons[:, 2].max() - start) / 100.0, 2)}


def gfx_clocks_under_load(torch, call, max_s=30.0, power=False):
    """GFX clocks (MHz, one per XCD) read with amd-smi while `call` keeps the
    GPU busy: about a second of calls is queued first (the clocks take some
    tenths of a second to rise from their idle level), and calls keep being
    queued until the tool returns.  With power, also the board's power
    readings (W).  None without the tool."""
    import shutil
    import subprocess
    import threading
    tool = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi"
                                       if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if tool is None:
        return None
    out = {}

    def sample():
        try:
            what = ["--clock", "--power"] if power else ["--clock"]
            out["text"] = subprocess.run([tool, "metric", *what, "--json"],
                                         capture_output=True, text=True, timeout=max_s).stdout
        except (OSError, subprocess.SubprocessError):
            out["text"] = ""

    th = threading.Thread(target=sample)
    t0 = time.time()
    while time.time() - t0 < 1.0:          # about a second of queued work
        for _ in range(50):
            call()
    th.start()
    while th.is_alive() and time.time() - t0 < max_s:
        for _ in range(50):
            call()
    th.join()
    torch.cuda.synchronize()
    text = out.get("text", "")
    try:
        data, _ = json.JSONDecoder().raw_decode(text[text.index("["):])
        clocks = [v["clk"]["value"] for k, v in data[0]["clock"].items() if k.startswith("gfx_")]
    except (ValueError, KeyError, IndexError, TypeError):
        return None
    if not clocks:
        return None
    res = {"mean": round(float(np.mean(clocks)), 1), "min": min(clocks), "max": max(clocks),
           "xcds": len(clocks), "tool": "amd-smi metric --clock, during pipelined calls"}
    if power:
        watts = {}
        for k, v in (data[0].get("power") or {}).items():
            if isinstance(v, dict) and isinstance(v.get("value"), (int, float)):
                watts[k] = v["value"]
            elif isinstance(v, (int, float)):
                watts[k] = v
        res["power_w"] = watts or None
        res["tool"] = "amd-smi metric --clock --power"
    return res


PROBE_LIB = os.path.join(ROOT, "communication_gemm_amd", "libaggprobe.so")


def mfma_probe(torch, seconds=1.5):
    """The register-only matrix-core probe (libaggprobe.so): one workgroup of
    eight waves per CU, each wave issuing matrix instructions on operands
    held in registers, no memory traffic in the loop.  Per kind (fp16
    32x32x16, fp8 E4M3 32x32x64) and operand pattern (random values, or one
    constant): TFLOP/s over launches of about 10 ms, and the GFX clocks and
    board power amd-smi reads while the probe runs."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: build with communication_gemm_amd/build.py")
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.agg_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                   ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {"cus": cus, "waves_per_cu": 8, "peak_tflops": {"f16": PEAK_F16_TFLOPS,
                                                          "fp8": PEAK_FP8_TFLOPS,
                                                          "i8": PEAK_I8_TOPS}}
    # flops per chain and iteration: one 2 x 32 x 32 x 16 (fp16), one
    # 2 x 32 x 32 x 64 (fp8), two 2 x 16 x 16 x 32 (fp16 16x16x32)
    for kind, name, flop in ((0, "f16", 32768), (2, "f16_16x16x32", 32768), (1, "fp8", 131072),
                             (3, "i8", 65536), (4, "i8_16x16x64", 65536)):
        for random, pattern in ((1, "random"), (0, "constant")):
            def launch(iters):
                rc = fn(kind, random, iters, cus, 1234, ctypes.c_void_p(out.data_ptr()),
                        ctypes.c_void_p(stream))
                if rc:
                    raise SystemExit(f"probe launch failed: {rc}")
            # size a launch to about 10 ms
            launch(1000)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            launch(20000)
            torch.cuda.synchronize()
            per_iter = (time.perf_counter() - t0) / 20000
            iters = max(1000, int(0.010 / per_iter))
            ramp(torch, lambda: launch(iters), seconds=0.5)
            t, _ = timed(torch, lambda ev: (lambda: launch(iters)), max(10, int(seconds / 0.010)),
                         3, with_consumer=False)
            flops = float(cus) * 8 * iters * 8 * flop
            def blocking():
                launch(iters)
                torch.cuda.synchronize()
            clocks = gfx_clocks_under_load(torch, blocking, power=True)
            res[f"{name}_{pattern}"] = {
                "ms_per_launch": round(t, 4), "iters": iters,
                "tflops": round(flops / (t * 1e-3) / 1e12, 1),
                "frac_of_peak": round(flops / (t * 1e-3) / 1e12 /
                                      (PEAK_FP8_TFLOPS if kind == 1 else PEAK_I8_TOPS
                                       if kind in (3, 4) else PEAK_F16_TFLOPS), 4),
                "under_load": clocks}
            print(json.dumps({"probe": f"{name}_{pattern}", **res[f"{name}_{pattern}"]}),
                  flush=True)
    return res


class F16Workload:
    """One fp16 workload on the device: inputs, output, a caller-owned
    workspace (nothing is allocated inside timed loops) and prepared calls
    in every mode."""

    def __init__(self, torch, agg, case, inputs, tile=0, link_gbps=None, chunk_rows=None):
        self.torch, self.agg, self.case = torch, agg, case
        shards, B = inputs
        self.ts = [torch.from_numpy(x).cuda() for x in shards]
        self.tB = torch.from_numpy(B).cuda()
        self.C = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(agg.workspace_bytes(case.n_shards, case.M, case.K, 2),
                              dtype=torch.uint8, device="cuda")
        agg.workspace_reset(self.ws)
        self.tile = tile
        self.gbps = case.link_gbps if link_gbps is None else link_gbps
        self.cr = case.chunk_rows if chunk_rows is None else chunk_rows
        self.calls = {name: self.prep(mode) for name, mode in MODES.items()}
        # the remote slots get the real rows before anything reads them (a
        # compute-only call on an unwritten workspace multiplies whatever it
        # holds, often zeros, which draws less power and runs faster)
        self.calls["copy"]()
        torch.cuda.synchronize()

    def prep(self, mode, ev=None, chunk_rows=None, **kw):
        o = dict(workspace=self.ws, mode=mode, link_gbps=self.gbps, tile=self.tile,
                 consumer_events=ev)
        o.update(kw)
        return self.agg.ag_gemm_f16(
            self.ts, self.tB, self.C, self.cr if chunk_rows is None else chunk_rows,
            opts=self.agg.options(**o), prepare=True)

    @property
    def flops(self):
        return 2.0 * self.case.M * self.case.K * self.case.N

    def plan(self):
        """The plan of the workload's pipelined calls (the same options)."""
        info, _, _ = self.agg.plan("f16", self.case.n_shards, self.case.M, self.case.K,
                                   self.case.N, self.cr,
                                   self.agg.options(tile=self.tile, link_gbps=self.gbps,
                                                    mode=MODES["pipelined"]),
                                   num_cus=self.torch.cuda.get_device_properties(
                                       self.torch.cuda.current_device()).multi_processor_count)
        return info

    def entry(self, steps, warmup=10, trace=False, timed_steps=None):
        """Pipelined steps (with the consumer's own time) and the four modes
        taken in turn.  timed_steps: (ms per step, consumer ms) measured
        already, in place of new pipelined steps."""
        torch, agg = self.torch, self.agg
        if timed_steps is None:
            ramp(torch, self.calls["pipelined"], seconds=0.3)
            t, c = timed(torch, lambda ev: self.prep(MODES["pipelined"], ev), steps, warmup)
        else:
            t, c = timed_steps
        inter = interleaved(torch, self.calls)
        info = self.plan()
        out = {"workload": self.case.name, "chunk_rows": info.chunk_rows,
               "tile": [info.tile_m, info.tile_n], "tile_id": info.tile_id,
               "link_gbps": self.gbps, "pipelined_ms": round(t, 5),
               "tflops": round(self.flops / (t * 1e-3) / 1e12, 2),
               "consumer_ms": round(c, 5),
               "consumer_tflops": round(self.flops / (c * 1e-3) / 1e12, 2),
               "consumer_frac_of_peak": round(self.flops / (c * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
               "interleaved": inter}
        if trace:
            out["trace"] = device_trace(torch, agg, lambda tr: self.prep(
                MODES["pipelined"], trace=tr)(), info)
        if agg.check():
            raise SystemExit(f"{self.case.name} runs failed")
        return out


class I8Workload:
    """The int8 + dequant workload, as F16Workload."""

    def __init__(self, torch, agg, case, inputs):
        self.torch, self.agg, self.case = torch, agg, case
        shards, B, bias, scale = inputs
        self.ts = [torch.from_numpy(x).cuda() for x in shards]
        self.tB = torch.from_numpy(B).cuda()
        self.tb = torch.from_numpy(bias).cuda()
        self.tsc = torch.from_numpy(scale).cuda()
        self.C = torch.empty((case.M, case.N), dtype=torch.float16, device="cuda")
        self.ws = torch.empty(agg.workspace_bytes(case.n_shards, case.M, case.K, 1),
                              dtype=torch.uint8, device="cuda")
        agg.workspace_reset(self.ws)
        self.calls = {name: self.prep(mode) for name, mode in MODES.items()}
        self.calls["copy"]()
        torch.cuda.synchronize()

    def prep(self, mode, ev=None):
        return self.agg.ag_gemm_i8_dequant(
            self.ts, self.tB, self.tb, self.tsc, self.C, 0,
            opts=self.agg.options(workspace=self.ws, mode=mode, consumer_events=ev), prepare=True)

    def entry(self, steps, warmup=10):
        torch, agg, case = self.torch, self.agg, self.case
        ops = 2.0 * case.M * case.K * case.N
        ramp(torch, self.calls["pipelined"], seconds=0.3)
        t, c = timed(torch, lambda ev: self.prep(MODES["pipelined"], ev), steps, warmup)
        tc, cc = timed(torch, lambda ev: self.prep(MODES["compute"], ev), steps, warmup)
        inter = interleaved(torch, self.calls, rounds=3, n=10)
        if agg.check():
            raise SystemExit("int8 runs failed")
        info, _, _ = agg.plan("i8", case.n_shards, case.M, case.K, case.N, 0)
        return {"workload": case.name, "chunk_rows": info.chunk_rows,
                "tile": [info.tile_m, info.tile_n], "tile_id": info.tile_id,
                "pipelined_ms": round(t, 5), "tops": round(ops / (t * 1e-3) / 1e12, 2),
                "consumer_ms": round(c, 5),
                "consumer_tops": round(ops / (c * 1e-3) / 1e12, 2),
                "consumer_frac_of_peak": round(ops / (c * 1e-3) / 1e12 / PEAK_I8_TOPS, 4),
                "compute_only_consumer_ms": round(cc, 5),
                "compute_only_consumer_frac_of_peak":
                    round(ops / (cc * 1e-3) / 1e12 / PEAK_I8_TOPS, 4),
                "interleaved": inter}


# Pallas:MGPU collective matmul page: per-device (1024 D) x 4096 x 4096 fp16
# with the LHS all-gathered around a ring, on H100s (other hardware, context
# only): the ring kernel, its model lower bound and the all-gather + matmul
# reference, in microseconds for D = 2, 4, 8.
PAGE_RING_US = {2: (102, 92, 147), 4: (212, 190, 290), 8: (436, 386, 565)}
XGMI_LINK_GBPS = 153.0   # one MI355X xGMI link, per direction


def run_ring(args, torch, agg, synth):
    """The ring variant on one GPU: device 0's view of a D-device ring, the
    shards arriving one after the other over one emulated link in ring order
    (own shard, then d+1, d+2, ...), each consumed as its chunks land; beside
    it the copy-then-GEMM reference (sequential mode), the same ring paced
    at one xGMI link's rate, and the full mesh (one link per source) at that
    rate."""
    out = {}
    n = max(20, args.steps // 2)
    for D in (2, 4, 8):
        M, K, N = 1024 * D, 4096, 4096
        case = synth.Case(90 + D, "f16", D, M, K, N)
        w = F16Workload(torch, agg, case, synth.make_f16(M, K, N, D, "normal", 90000 + D))

        ramp(torch, w.calls["pipelined"], seconds=0.2)

        def us(**kw):
            mode = kw.pop("mode", MODES["pipelined"])
            return round(timed(torch, lambda ev: w.prep(mode, **kw), n, 10,
                               with_consumer=False)[0] * 1e3, 1)

        r = {"workload": f"f16 {D}x1024 rows M={M} K={K} N={N}, ring order, one serial link",
             "ring_us": us(link_model=agg.LINKS_SERIAL),
             "copy_then_gemm_us": us(link_model=agg.LINKS_SERIAL, mode=MODES["sequential"]),
             "compute_only_us": us(mode=MODES["compute"]),
             "ring_xgmi_paced_us": us(link_model=agg.LINKS_SERIAL, link_gbps=XGMI_LINK_GBPS),
             "mesh_xgmi_paced_us": us(link_model=agg.LINKS_PARALLEL, link_gbps=XGMI_LINK_GBPS)}
        if agg.check():
            raise SystemExit("ring runs failed")
        r["tflops"] = round(2.0 * M * K * N / (r["ring_us"] * 1e-6) / 1e12, 1)
        page = PAGE_RING_US[D]
        r["page_h100_us"] = {"ring": page[0], "model_bound": page[1], "allgather_then_matmul": page[2]}
        out[str(D)] = r
        del w
    return out


def run_variant(args, torch, agg, synth, kind, mode="pipelined"):
    """The bf16 or fp8 (E4M3) variant on the 8 x 1024-row fp16 workload's
    shape, pipelined (or in `mode`)."""
    case = synth.CASES[args.case]
    if kind == "bf16":
        shards, B = synth.make_bf16(case.M, case.K, case.N, case.n_shards, "normal",
                                    1000 * case.case_id)

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(
                torch.bfloat16)
        fn, elt, peak = agg.ag_gemm_bf16, 2, PEAK_F16_TFLOPS
    else:
        shards, B = synth.make_fp8(case.M, case.K, case.N, case.n_shards, "normal",
                                   1000 * case.case_id)

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()
        fn, elt, peak = agg.ag_gemm_fp8, 1, PEAK_FP8_TFLOPS
    ts = [dev(x) for x in shards]
    tB = dev(B)
    C = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(agg.workspace_bytes(case.n_shards, case.M, case.K, elt), dtype=torch.uint8,
                     device="cuda")
    agg.workspace_reset(ws)
    def make(ev):
        return fn(ts, tB, C, 0, opts=agg.options(workspace=ws, mode=MODES[mode],
                                                 consumer_events=ev), prepare=True)
    if mode == "compute":
        fn(ts, tB, C, 0, opts=agg.options(workspace=ws, mode=MODES["copy"]))
    ramp(torch, make(None), seconds=0.3)
    t, c = timed(torch, make, max(20, args.steps // 2), 20)
    if agg.check():
        raise SystemExit(f"{kind} run failed")
    flops = 2.0 * case.M * case.K * case.N
    return {"workload": case.name.replace("f16", kind, 1), "mode": mode, "ms": round(t, 5),
            "consumer_ms": round(c, 5), "tflops": round(flops / (t * 1e-3) / 1e12, 2),
            "consumer_tflops": round(flops / (c * 1e-3) / 1e12, 2),
            "consumer_frac_of_peak": round(flops / (c * 1e-3) / 1e12 / peak, 4)}


def load_probe(torch, iters=1024):
    """The operand-movement probe (libaggprobe.so): per iteration each of
    256 workgroups (one per CU) moves one 64 KiB K slice into LDS with the
    direct global-to-LDS load, reads 192 KiB out of LDS, or both, then waits
    and meets at a barrier: one K slice of the 256 x 256 fp16 consumer
    tile.  Microseconds per iteration, per pattern."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: build with communication_gemm_amd/build.py")
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.agg_probe_loads
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                   ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    wgs = 256
    pitch_max = 8320
    A = torch.ones(4096 * pitch_max, dtype=torch.uint8, device="cuda")
    B = torch.ones(64 * 64 * pitch_max, dtype=torch.uint8, device="cuda")
    out = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    cases = [
        ("contiguous 64 KiB, loads", 0, 1, 8192, 64),
        ("tile pattern, pitch 8192, loads", 1, 1, 8192, 64),
        ("tile pattern, pitch 8320, loads", 1, 1, 8320, 64),
        ("tile pattern, 4 slices (L2-resident), loads", 1, 1, 8192, 4),
        ("LDS reads only (192 KiB)", 1, 2, 8192, 64),
        ("tile pattern loads + LDS reads", 1, 3, 8192, 64),
    ]
    res = {}
    for name, pattern, what, pitch, ns in cases:
        a_bytes, b_bytes = 4096 * pitch, 64 * 64 * pitch
        def launch(n=iters):
            rc = fn(pattern, what, n, wgs, ctypes.c_void_p(A.data_ptr()), a_bytes,
                    ctypes.c_void_p(B.data_ptr()), b_bytes, pitch, ns,
                    ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
            if rc:
                raise SystemExit(f"load probe launch failed: {rc}")
        ramp(torch, launch, calls=5)
        t, _ = timed(torch, lambda ev: launch, 5, 1, with_consumer=False)
        res[name] = round(t * 1e3 / iters, 3)
        print(json.dumps({"load_probe": name, "us_per_slice": res[name]}), flush=True)
    del A, B
    # whole-matrix streaming into LDS: an int8 16384 x 7168 weight (117 MB),
    # one launch reading all of it, on one buffer (which the 256 MB
    # last-level cache then holds) or rotating over three (351 MB, so each
    # launch reads HBM)
    sfn = lib.agg_probe_stream
    sfn.restype = ctypes.c_int
    sfn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint32,
                    ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    rows, row_bytes = 16384, 7168
    mats = [torch.ones(rows * row_bytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    stream_cases = [
        ("64-byte column strips, 2 parts (224 workgroups)", 0, 2),
        ("contiguous ranges, 224 workgroups", 1, 224),
        ("contiguous ranges, 448 workgroups", 1, 448),
    ]
    srate = {}
    for name, pattern, n in stream_cases:
        for rot in (1, 3):
            k = [0]
            def launch():
                m = mats[k[0] % rot]
                k[0] += 1
                rc = sfn(pattern, n, ctypes.c_void_p(m.data_ptr()), rows, row_bytes,
                         ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
                if rc:
                    raise SystemExit(f"stream probe launch failed: {rc}")
            ramp(torch, launch, calls=20)
            t, _ = timed(torch, lambda ev: launch, 60, 3, with_consumer=False)
            key = f"{name}, {'one buffer' if rot == 1 else 'three buffers'}"
            srate[key] = {"us": round(t * 1e3, 2),
                          "TB_per_s": round(rows * row_bytes / (t * 1e-3) / 1e12, 2)}
            print(json.dumps({"stream_probe": key, **srate[key]}), flush=True)
    return {"us_per_iteration": res, "workgroups": wgs, "iterations": iters,
            "note": "one 64 KiB slice per CU per iteration (A 256 rows x 128 B, B 64 rows x "
                    "512 B), 192 KiB of ds_read_b128 per CU, wait and barrier each iteration",
            "stream_int8_16384x7168": srate}


def only_variant(args, torch, agg, synth):
    """--only: one variant's timed steps in --mode, nothing else (the
    workload hardware-counter runs profile)."""
    if args.only in ("bf16", "fp8"):
        return run_variant(args, torch, agg, synth, args.only, args.mode)
    c = synth.CASES[5]
    w = I8Workload(torch, agg, c, synth.make_case(c))
    ops = 2.0 * c.M * c.K * c.N
    ramp(torch, w.calls[args.mode], seconds=0.3)
    t, cm = timed(torch, lambda ev: w.prep(MODES[args.mode], ev), args.steps, args.warmup)
    if agg.check():
        raise SystemExit("int8 run failed")
    return {"workload": c.name, "mode": args.mode, "ms": round(t, 5),
            "consumer_ms": round(cm, 5), "consumer_tops": round(ops / (cm * 1e-3) / 1e12, 2)}


PRODUCERS = {"kernel": dict(), "sdma": dict(producer=1), "kernel_32cus": dict(producer_cus=32),
             "kernel_64cus": dict(producer_cus=64)}


def producer_variants(torch, agg, synth, i8_inputs=None):
    """What moves the chunks: the producer kernel on every CU (default), the
    DMA engines, or the producer kernel on 32 or 64 CUs of its own.
    Pipelined and copy-only medians, the variants taken in turn.  The DMA
    engines cannot be paced, so C3 runs unpaced here (its link rate
    belongs to the emulated link, not to the engine that copies)."""
    out = {}
    for cid in (3, 4, 5):
        c = synth.CASES[cid]
        if c.kind == "i8":
            if i8_inputs is None:
                continue
            w = I8Workload(torch, agg, c, i8_inputs)

            def prep(mode, kw, w=w):
                return agg.ag_gemm_i8_dequant(
                    w.ts, w.tB, w.tb, w.tsc, w.C, 0,
                    opts=agg.options(workspace=w.ws, mode=mode, **kw), prepare=True)
        else:
            w = F16Workload(torch, agg, c, synth.make_case(c), link_gbps=0.0)

            def prep(mode, kw, w=w):
                return w.prep(mode, **kw)
        calls = {name: {m: prep(MODES[m], kw) for m in ("pipelined", "copy", "compute")}
                 for name, kw in PRODUCERS.items()}
        ramp(torch, calls["kernel"]["pipelined"], seconds=0.3)
        res = {name: {"pipelined": [], "copy": []} for name in PRODUCERS}
        n = 10 if c.kind == "i8" else 20
        comp = []
        for _ in range(3):
            comp.append(timed(torch, lambda ev: calls["kernel"]["compute"], n, 2,
                              with_consumer=False)[0])
            for name in PRODUCERS:
                for m in ("pipelined", "copy"):
                    t, _ = timed(torch, lambda ev, f=calls[name][m]: f, n, 2, with_consumer=False)
                    res[name][m].append(t)
        if agg.check():
            raise SystemExit("producer variants failed")
        t_comp = float(np.median(comp))
        entry = {"workload": c.name + (" (unpaced)" if cid == 3 else ""),
                 "compute_ms": round(t_comp, 5)}
        for name in PRODUCERS:
            tp, tc = float(np.median(res[name]["pipelined"])), float(np.median(res[name]["copy"]))
            entry[name] = {"pipelined_ms": round(tp, 5), "copy_ms": round(tc, 5),
                           "hidden_fraction": round((t_comp + tc - tp) / tc, 4)}
        out[f"C{cid}"] = entry
        del w, calls
    return out


def vendor_gemm(torch, w, steps=50):
    """hipBLASLt (torch.matmul) on the gathered A of the same workload, fp16
    in and fp16 out (torch has no fp32-output fp16 GEMM): a ceiling
    reference for the plain local GEMM, with no gather."""
    A = torch.cat(w.ts, 0)
    out = torch.empty((A.shape[0], w.tB.shape[1]), dtype=torch.float16, device="cuda")
    ramp(torch, lambda: torch.matmul(A, w.tB, out=out), seconds=0.3)
    t, _ = timed(torch, lambda ev: (lambda: torch.matmul(A, w.tB, out=out)), steps, 10,
                 with_consumer=False)
    return {"what": "torch.matmul (hipBLASLt), fp16 in, fp16 out, the whole gathered A",
            "ms": round(t, 5), "tflops": round(w.flops / (t * 1e-3) / 1e12, 2)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_rate(oracle, fn, M, K, N, budget_s, seed=0):
    """The oracle on a bounded sample of rows, sized to about budget_s
    seconds: (rows, seconds, GFLOP/s)."""
    rng = np.random.default_rng(seed)
    rows_all = np.arange(M, dtype=np.int64)
    probe_t = []
    for k in (8, 32):
        k = min(k, M)
        t0 = time.perf_counter()
        fn(np.sort(rng.choice(rows_all, k, replace=False)))
        probe_t.append((k, time.perf_counter() - t0))
    (k0, t0_), (k1, t1_) = probe_t
    per_row = max((t1_ - t0_) / max(k1 - k0, 1), 1e-7)
    n = int(min(M, max(8, budget_s / per_row)))
    rows = np.sort(rng.choice(rows_all, n, replace=False))
    t0 = time.perf_counter()
    fn(rows)
    dt = time.perf_counter() - t0
    return n, dt, 2.0 * n * K * N / dt / 1e9


def cpu_baseline(case, inputs, budget_s, synth, i8_inputs=None):
    """The oracle, as it stands, on a bounded sample of the timed workload's
    rows on every host thread; beside it the same on C1-C3 (and C5) with
    every thread and with one."""
    import oracle
    shards, B = inputs
    n, dt, gflops = oracle_rate(oracle, lambda r: oracle.ag_gemm_f16(shards, B, rows=r,
                                                                      with_abs=False),
                                case.M, case.K, case.N, budget_s)
    out = {"value": round(gflops / 1e3, 5), "unit": "TFLOPS", "cores": oracle.threads_used(),
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{n} of {case.M} rows of C ({2.0 * n * case.K * case.N / 1e9:.1f} GFLOP, "
                     f"fp64 accumulation) in {dt:.1f} s"}
    per = {}
    for threads in (0, 1):
        prev = oracle.set_threads(1) if threads == 1 else None
        try:
            for cid in (1, 2, 3):
                c = synth.CASES[cid]
                sh, Bc = synth.make_case(c)
                rn, rdt, rg = oracle_rate(oracle, lambda r: oracle.ag_gemm_f16(
                    sh, Bc, rows=r, with_abs=False), c.M, c.K, c.N, 0.5 if threads else 1.0)
                per.setdefault(f"C{cid}", {})["one_thread" if threads else "all_threads"] = {
                    "rows": rn, "of_rows": c.M, "seconds": round(rdt, 3),
                    "gflops": round(rg, 3), "full_config_s": round(rdt * c.M / rn, 3)}
        finally:
            if prev is not None:
                oracle.set_threads(prev)
    if i8_inputs is not None:
        c = synth.CASES[5]
        sh, Bc, bias, scale = i8_inputs
        rn, rdt, rg = oracle_rate(oracle, lambda r: oracle.ag_gemm_i8_dequant(
            sh, Bc, bias, scale, rows=r), c.M, c.K, c.N, 2.0)
        per["C5"] = {"all_threads": {"rows": rn, "of_rows": c.M, "seconds": round(rdt, 3),
                                     "gops": round(rg, 3), "full_config_s": round(rdt * c.M / rn, 2)}}
    out["per_config"] = per
    out["note"] = ("all_threads: every host thread (OpenMP over output rows); one_thread: one; "
                   "full_config_s scales the sample to every row of the workload")
    return out


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps, args.skip)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the streamed "
              "AllGather is emulated on a single device; there is no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import communication_gemm_amd as agg
    import synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.mfma_probe:
        print(json.dumps({"mfma_probe": mfma_probe(torch)}), flush=True)
        return
    if args.load_probe:
        print(json.dumps({"load_probe": load_probe(torch)}), flush=True)
        return
    if args.only:
        print(json.dumps(only_variant(args, torch, agg, synth)), flush=True)
        return
    case = synth.CASES[args.case]
    if case.kind != "f16":
        raise SystemExit("--case must name an fp16 workload")
    inputs = synth.make_case(case)
    if args.vendor_only:
        w = F16Workload(torch, agg, case, inputs)
        print(json.dumps({"vendor_gemm": vendor_gemm(torch, w, args.steps),
                          "workload": case.name}), flush=True)
        return
    w = F16Workload(torch, agg, case, inputs, tile=args.tile,
                    link_gbps=args.link_gbps, chunk_rows=args.chunk_rows or None)
    mode = MODES[args.mode]
    if args.mode == "compute":
        w.calls["copy"]()

    # 1. The timed steps: clocks out of idle, W warm-up steps, K steps.
    ramp(torch, w.prep(mode), calls=args.ramp_calls)
    each = []
    t_step, c_step = timed(torch, lambda ev: w.prep(mode, ev), args.steps, args.warmup,
                           with_consumer=args.mode != "copy", per_call=each)
    rc = agg.check()
    if rc:
        raise SystemExit(f"{args.mode} run failed: {agg.status_string(rc)}")
    info = w.plan()
    tflops = w.flops / (t_step * 1e-3) / 1e12
    overlap = {"step_ms": round(t_step, 5)}
    if each:
        overlap.update(consumer_ms=round(c_step, 5), consumer_ms_median=round(float(np.median(each)), 5),
                       consumer_ms_min=round(float(np.min(each)), 5),
                       consumer_launches_timed=len(each))
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGE_TFLOPS_8192, 3) if case.case_id == 4 else None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": case.name + " streamed AllGather+GEMM, fp16 in, fp32 out",
                   "M": case.M, "K": case.K, "N": case.N, "n_shards": case.n_shards,
                   "chunk_rows": info.chunk_rows, "tile": [info.tile_m, info.tile_n],
                   "tile_id": info.tile_id, "link_gbps": w.gbps,
                   "mode": args.mode, "parallelism": "single GPU, shards emulated"},
        "frac_of_peak": round(tflops / PEAK_F16_TFLOPS, 4),
        "roofline": None if not each else {
            "bound": "mfma", "achieved": round(w.flops / (c_step * 1e-3) / 1e12, 2),
            "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(w.flops / (c_step * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
            "traffic": stored_traffic(case.name, info.tile_id) if args.tile == 0 else None,
            "kernel": "consumer (persistent MFMA GEMM)", "kernel_ms": round(c_step, 5)},
        "overlap": overlap,
        "baseline_note": "vs_baseline divides by the PTO-ISA page's 8-card 8192x4096x4096 "
                         "figure on Ascend 910B1 (191.03 TFLOPS): other hardware, context only",
    }
    full = args.mode == "pipelined" and not args.no_modes
    if full:
        # 2. The timed workload's own figures: the four modes in turn, the
        # device trace, the chunk-size sweep, the comparison scheme, clocks.
        c4 = w.entry(max(20, args.steps), trace=True, timed_steps=(t_step, c_step))
        overlap["interleaved"] = c4["interleaved"]
        overlap["trace"] = c4["trace"]
        if not args.no_chunk_sweep:
            sweep = {}
            for rows in (16, 32, 64, 128, 256):
                if rows <= case.shard_rows:
                    t, _ = timed(torch, lambda ev, r=rows: w.prep(MODES["pipelined"], chunk_rows=r),
                                 max(20, args.steps // 2), 10, with_consumer=False)
                    sweep[str(rows)] = round(t, 5)
            barrier = {}
            for name, kw in (("pvalue1", dict(pvalue=1)), ("pvalue2", dict(pvalue=2)),
                             ("pvalue1_stages2", dict(pvalue=1, workspace_stages=2))):
                t, _ = timed(torch, lambda ev, kw=kw: w.prep(
                    MODES["pipelined"], scheme=agg.SCHEME_BARRIER, **kw),
                    max(20, args.steps // 2), 10, with_consumer=False)
                barrier[name] = round(t, 5)
            if agg.check():
                raise SystemExit("sweeps failed")
            overlap["chunk_sweep_ms"] = sweep
            overlap["barrier_scheme_ms"] = barrier
        if not args.no_clocks:
            overlap["gfx_clock_mhz"] = gfx_clocks_under_load(torch, w.calls["pipelined"])
        # 3. Every workload's entry: C1-C3 (C3 with its paced producer), the
        # timed one, and the int8 C5.
        configs = {}
        for cid in (1, 2, 3):
            c = synth.CASES[cid]
            cw = F16Workload(torch, agg, c, synth.make_case(c))
            configs[f"C{cid}"] = cw.entry(max(50, args.steps), trace=cid == 3)
            del cw
        configs[f"C{case.case_id}"] = {k: v for k, v in c4.items() if k != "trace"}
        i8_inputs = None
        if not args.no_int8:
            i8_inputs = synth.make_case(5)
            iw = I8Workload(torch, agg, synth.CASES[5], i8_inputs)
            configs["C5"] = iw.entry(max(10, args.steps // 2))
            del iw
        line["configs"] = configs
        if not args.no_bf16:
            line["bf16"] = run_variant(args, torch, agg, synth, "bf16")
        if not args.no_fp8:
            line["fp8"] = run_variant(args, torch, agg, synth, "fp8")
        if not args.no_ring:
            line["ring"] = run_ring(args, torch, agg, synth)
        if not args.no_producers:
            line["producers"] = producer_variants(torch, agg, synth, i8_inputs)
        line["vendor_gemm"] = vendor_gemm(torch, w)
        # 4. The timed steps again, after everything above has loaded the
        # board for tens of seconds.
        ramp(torch, w.calls["pipelined"], seconds=0.3)
        t2, c2 = timed(torch, lambda ev: w.prep(mode, ev), args.steps, args.warmup)
        if agg.check():
            raise SystemExit("sustained run failed")
        overlap["sustained"] = {"step_ms": round(t2, 5), "consumer_ms": round(c2, 5),
                                "tflops": round(w.flops / (t2 * 1e-3) / 1e12, 2),
                                "note": "the timed steps repeated at the end of the run"}
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(case, inputs, args.cpu_seconds, synth, i8_inputs)
    elif not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, inputs, args.cpu_seconds, synth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
