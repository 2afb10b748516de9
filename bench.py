#!/usr/bin/env python3
"""Benchmark of FlashSampling's fused LM-head matmul + sample (FMMS) on one MI355X.

One step = one fs_fmms_sample call (stream W, logits on chip, scale, noise,
tile argmax, cross-tile reduction) over a fixed synthetic batch, with the step
counter incrementing.  Headline: the mid-size decode head (d=4096, V=151936,
B=64, T=0.7).  Prints ONE JSON line.

  value     achieved HBM GB/s = algorithmic bytes per step (V*d*2 + B*d*2 + B*4)
            / measured time per step (HIP events on the launch stream), after a
            pre-run of at least 1 s that brings the GPU's clocks up
  roofline  the streaming kernel alone: algorithmic bytes per launch / its mean
            duration (HIP events recorded around each launch by the library's
            timing hook) against MI355X's 8 TB/s; `traffic` is the measured HBM
            bytes per launch from the committed rocprofv3 counter summary
  sweep     every B of the small and mid decode heads, the masked and grouped
            workloads, each next to the in-house unfused GEMM -> logits -> sample
  cpu_baseline  the CPU oracle timed on the host's cores on a bounded sample
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/step and achieved HBM GB/s (% of peak) for FMMS at V=151936, B=1–64"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# the calls a --profile run can time: fs_fmms_sample (top_k) or the unfused comparator
PROFILE_OPS = {"fused": dict(top_k=0, unfused=False), "unfused": dict(top_k=0, unfused=True),
               "topk": dict(top_k=50, unfused=False)}


def traffic_summary_path(op, workload="mid_decode", B=64):
    return os.path.join(ROOT, "profiles", f"{op}_{workload}_B{B}_hbm_traffic.md")


CSRC = os.path.join(ROOT, "lm_head_matmul_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
CALIB_BYTES = 1 << 30  # the --profile run's plain device fill + copy


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="mid_decode")
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--no-sweep", action="store_true", help="headline only")
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3: one 1 GiB device copy (counter calibration), then the "
                         "headline steps only, of the call --profile-op names")
    ap.add_argument("--profile-op", default="fused", choices=sorted(PROFILE_OPS),
                    help="the call a --profile run times: the fused sampler, the unfused comparator, or top-k")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC1_CSV", "PMC2_CSV"),
                    help="write the profiles/ counter summary of a --profile run's two counter passes and exit")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write the profiles/ summaries of a --profile run's rocprofv3 csv output (for the "
                         "--profile-op, --workload and --batch given) and exit")
    return ap.parse_args()


def algorithmic_bytes(B, d, V, mask=False):
    return V * d * 2 + B * d * 2 + B * 4 + (B * ((V + 31) // 32) * 4 if mask else 0)


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def floors(B, d, V, mask=False):
    """Lower bounds of a step's time: streaming its algorithmic bytes at peak HBM bandwidth,
    and its 2 B V d multiply-adds at the dense bf16 MFMA peak; with them the step's noise work,
    the vector-ALU side of the epilogue: one Gumbel value per (row, id), i.e. B V / 4
    Philox4x32-10 calls (four words each) and two logarithms per value."""
    return {"hbm_floor_us": round(algorithmic_bytes(B, d, V, mask) / (PEAK_HBM_GBS * 1e3), 2),
            "mfma_floor_us": round(2.0 * B * V * d / (PEAK_BF16_TFLOPS * 1e6), 2),
            "noise_ops": {"gumbel_values": B * V, "philox4x32_10_calls": B * V // 4, "log_evals": 2 * B * V}}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(op="fused", workload="mid_decode", B=64):
    """HBM bytes per step of a call from its committed counter summary, if it matches these kernels."""
    path = traffic_summary_path(op, workload, B)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_step"]))
    except (KeyError, ValueError):
        return None


def profile_cmds(op, workload, B):
    a = f"--profile --profile-op {op} --workload {workload} --batch {B}"
    d = f"gpurun_out/prof_{op}_{workload}_B{B}"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}_trace -o trace "
                 f"-- python3 bench.py {a} --steps 1000 --warmup 50",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}_fetch -o fetch "
                 f"-- python3 bench.py {a} --steps 5 --warmup 2",
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}_write -o write "
                 f"-- python3 bench.py {a} --steps 5 --warmup 2",
        "pmc1": f"rocprofv3 --pmc {' '.join(COUNTER_PASSES[0])} --output-format csv -d {d}_pmc1 -o pmc "
                f"-- python3 bench.py {a} --steps 5 --warmup 2",
        "pmc2": f"rocprofv3 --pmc {' '.join(COUNTER_PASSES[1])} --output-format csv -d {d}_pmc2 -o pmc "
                f"-- python3 bench.py {a} --steps 5 --warmup 2",
    }


# Two counter passes (each within one pass's limits: 8 SQ, 2 TA, 4 TCP counters) for the
# streaming kernel's memory pipeline: how busy the address unit is and how often the L1 (TCP) holds
# it up, the L1-to-L2 requests and their latency, MFMA and VALU activity.
COUNTER_PASSES = (
    ("SQ_BUSY_CYCLES", "SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VMEM_RD", "SQ_LDS_BANK_CONFLICT", "TA_TA_BUSY_sum",
     "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TCP_TCC_READ_REQ_sum", "TCP_TCC_READ_REQ_LATENCY_sum",
     "TCP_PENDING_STALL_CYCLES_sum", "TCP_TCR_TCP_STALL_CYCLES_sum"),
    ("GRBM_GUI_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_INST_LEVEL_VMEM", "TA_FLAT_READ_LDS_WAVEFRONTS_sum",
     "TA_DATA_STALLED_BY_TC_CYCLES_sum", "TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TCP_TA_DATA_STALL_CYCLES_sum"),
)


def summarize_counters(pmc_csvs, op="fused", workload="mid_decode", B=64):
    """The streaming kernel's counters (averaged over its calls) from the two counter passes of a
    --profile run, with the figures they give: address-unit busy and held-up fractions, L1-to-L2
    read requests per CU per clock and their mean latency."""
    import csv
    import synth

    w = synth.WORKLOADS[workload]
    tag = f"{op}_{workload}_B{B}"
    cmds = profile_cmds(op, workload, B)
    per = {}
    for fn in pmc_csvs:
        for r in csv.DictReader(open(fn)):
            if "fsk::" not in r["Kernel_Name"]:
                continue
            k = r["Kernel_Name"].split("(")[0]
            d = per.setdefault(k, {"_n": set(), "_dur": []})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            d["_dur"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    stream = max(per, key=lambda k: sum(per[k]["_dur"]) / len(per[k]["_dur"]))
    c = {k: sum(v) / len(v) for k, v in per[stream].items() if not k.startswith("_")}
    n_cu, n_xcd = 256, 8  # MI355X; GRBM_GUI_ACTIVE adds up the busy clocks of the 8 XCDs
    dur_us = sum(per[stream]["_dur"]) / len(per[stream]["_dur"]) / 1e3
    gui = c.get("GRBM_GUI_ACTIVE")
    gui = gui / n_xcd if gui else None
    lines = [f"# {op}: {workload} head (B={B}, d={w['d']}, V={w['V']}), streaming-kernel counters", "",
             f"counter pass 1: `cd /tmp && export TMPDIR=/tmp && cd <repo root> && {cmds['pmc1']}`", "",
             f"counter pass 2: `cd /tmp && export TMPDIR=/tmp && cd <repo root> && {cmds['pmc2']}`", "",
             f"Kernel: `{stream}`; every value is the average over its calls in the pass (the `_sum` counters "
             "summed over the chip's instances).", "", "| counter | average per call |", "|---|---:|"]
    for k in sorted(c):
        lines.append(f"| {k} | {c[k]:.4g} |")
    lines.append("")
    if gui:
        ta = c.get("TA_TA_BUSY_sum", 0) / (gui * n_cu)
        stall = c.get("TA_ADDR_STALLED_BY_TC_CYCLES_sum", 0) / max(c.get("TA_TA_BUSY_sum", 1), 1)
        req = c.get("TCP_TCC_READ_REQ_sum", 0)
        lat = c.get("TCP_TCC_READ_REQ_LATENCY_sum", 0) / max(req, 1)
        lines += [f"- busy clocks per call (GRBM_GUI_ACTIVE / {n_xcd} XCDs): {gui:.0f} in {dur_us:.1f} us of kernel "
                  f"time in these passes ({gui / dur_us / 1e3:.2f} GHz)",
                  f"- address unit (TA) busy: {ta * 100:.1f}% of those clocks per CU; held up by the L1 (TC) in "
                  f"{stall * 100:.1f}% of its busy clocks",
                  f"- L1-to-L2 read requests: {req:.4g} per call ({req * 128 / 1e6:.0f} MB at 128 B), "
                  f"{req / (gui * n_cu):.3f} per CU per clock, mean latency {lat:.0f} clocks"]
    open(os.path.join(ROOT, "profiles", f"{tag}_counters.md"), "w").write("\n".join(lines) + "\n")
    print(f"wrote the {tag} counter summary ({stream})")


def summarize_profiles(trace_csv, fetch_csv, write_csv, op="fused", workload="mid_decode", B=64):
    """Turn a --profile run's rocprofv3 csv files into the committed text summaries of that call:
    the kernel trace (per-kernel durations) and the HBM traffic per step (FETCH_SIZE + WRITE_SIZE
    of every library kernel of a step, calibrated against a plain fill and copy)."""
    import csv
    import synth

    w = synth.WORKLOADS[workload]
    algo = algorithmic_bytes(B, w["d"], w["V"])
    tag = f"{op}_{workload}_B{B}"
    pre = "cd /tmp && export TMPDIR=/tmp && cd <repo root> && "
    cmds = profile_cmds(op, workload, B)

    per = {}  # the library's kernels: durations of every call
    for r in csv.DictReader(open(trace_csv)):
        if "fsk::" in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    ours = sorted(per, key=lambda n: -sum(per[n]))
    assert ours, "no library kernel in the trace"
    stream = ours[0]  # the streaming kernel: the step's longest
    steps = len(per[stream])
    lines = [f"# {op}: {workload} head (B={B}, d={w['d']}, V={w['V']}), kernel trace", "",
             f"command: `{pre}{cmds['trace']}`", "",
             "The run: one 1 GiB device fill and copy (counter calibration), then the call's warmup, a pre-run of "
             "at least 0.5 s, 1000 timed steps and 1000 steps with the timing events.", "",
             "| kernel | calls | average us | median us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
    for n in ours:
        d = sorted(per[n])
        lines.append(f"| `{n.split('(')[0][:110]}` | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | "
                     f"{d[len(d) // 2] / 1e3:.1f} | {d[0] / 1e3:.1f} | {d[-1] / 1e3:.1f} |")
    avg_us = sum(per[stream]) / steps / 1e3
    lines += ["", f"- streaming_kernel: `{stream.split('(')[0]}`",
              f"- streaming_kernel_average_us: {avg_us:.2f}",
              f"- library_kernels_us_per_step: {sum(sum(v) for v in per.values()) / steps / 1e3:.2f}",
              f"- algorithmic_bytes_per_step: {algo}",
              f"- achieved_GB_per_s_at_streaming_kernel_average: {algo / (avg_us * 1e-6) / 1e9:.1f}",
              f"- kernel_source_sha256_16: {kernel_source_hash()}", ""]
    open(os.path.join(ROOT, "profiles", f"{tag}_kernel_trace.md"), "w").write("\n".join(lines))

    def rows(fn):
        return list(csv.DictReader(open(fn)))

    def calib(rs, counter):
        # the fill kernel writes CALIB_BYTES; the copy that follows it reads CALIB_BYTES
        fill = next(i for i, r in enumerate(rs) if "FillFunctor<short>" in r["Kernel_Name"])
        copy = next(r for r in rs[fill + 1:] if "copyBuffer" in r["Kernel_Name"])
        kib = float((rs[fill] if counter == "WRITE_SIZE" else copy)["Counter_Value"])
        return (CALIB_BYTES / 1024) / kib, kib

    def per_kernel(rs):
        d = {}
        for r in rs:
            if "fsk::" in r["Kernel_Name"]:
                d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return d

    fr, wr = rows(fetch_csv), rows(write_csv)
    f_fac, f_cal = calib(fr, "FETCH_SIZE")
    w_fac, w_cal = calib(wr, "WRITE_SIZE")
    fk, wk = per_kernel(fr), per_kernel(wr)
    n_f, n_w = len(fk.get(stream, [])), len(wk.get(stream, []))
    assert n_f and n_w, "the streaming kernel is missing from a counter pass"
    f_step = sum(sum(v) for v in fk.values()) / n_f * 1024 * f_fac
    w_step = sum(sum(v) for v in wk.values()) / n_w * 1024 * w_fac
    hbm = f_step + w_step
    lines = [f"# {op}: {workload} head (B={B}, d={w['d']}, V={w['V']}), HBM traffic per step", "",
             f"fetch pass: `{pre}{cmds['fetch']}`", "",
             f"write pass: `{pre}{cmds['write']}`", "",
             "Calibration: the same runs first fill 1 GiB (a pure write) and copy it (a 1 GiB read + write).",
             f"FETCH_SIZE reads {f_cal:.1f} KiB for the copy's 1048576 KiB read (factor {f_fac:.5f});",
             f"WRITE_SIZE reads {w_cal:.1f} KiB for the fill's 1048576 KiB write (factor {w_fac:.5f}).",
             f"Steps seen: {n_f} (fetch pass), {n_w} (write pass); every library kernel of a step counts.", "",
             "| kernel | FETCH_SIZE KiB per call (raw) | WRITE_SIZE KiB per call (raw) |", "|---|---:|---:|"]
    for n in sorted(set(fk) | set(wk), key=lambda n: -sum(fk.get(n, [0.0]))):
        fv, wv = fk.get(n, [0.0]), wk.get(n, [0.0])
        lines.append(f"| `{n.split('(')[0][:110]}` | {sum(fv) / len(fv):.1f} | {sum(wv) / len(wv):.1f} |")
    lines += ["", f"- fetch_bytes_per_step: {f_step:.0f}",
              f"- write_bytes_per_step: {w_step:.0f}",
              f"- hbm_bytes_per_step: {hbm:.0f}",
              f"- algorithmic_bytes_per_step: {algo}",
              f"- traffic_over_algorithmic: {hbm / algo:.4f}",
              f"- kernel_source_sha256_16: {kernel_source_hash()}", ""]
    open(traffic_summary_path(op, workload, B), "w").write("\n".join(lines))
    print(f"wrote the {tag} summaries: streaming kernel {avg_us:.1f} us, traffic {hbm / algo:.4f} x algorithmic")


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def run(self, fn, n):
        t = self.torch
        t.cuda.synchronize()
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(n):
            fn(i)
        e1.record(self.stream)
        t.cuda.synchronize()
        wall = time.perf_counter() - w0
        return e0.elapsed_time(e1) / n, wall  # ms per call, seconds

    def run_with_kernel_events(self, fn, n, arm):
        """Like run(), and each call's streaming kernel bracketed by its own pair of events
        (arm(before, after) before the call): returns (ms per call, seconds, mean kernel ms)."""
        t = self.torch
        pairs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in pairs:  # record once so that the HIP events exist before the library records them
            a.record(self.stream)
            b.record(self.stream)
        t.cuda.synchronize()
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(n):
            arm(*pairs[i])
            fn(i)
        e1.record(self.stream)
        t.cuda.synchronize()
        wall = time.perf_counter() - w0
        kern = sum(a.elapsed_time(b) for a, b in pairs) / n
        return e0.elapsed_time(e1) / n, wall, kern

    def warm(self, fn, seconds, batch=50, tol=0.01):
        """Runs fn until `seconds` have passed and two consecutive `batch`-call timings agree
        within `tol` (at most 4 x `seconds`): the GPU's clocks ramp up over the first tens of
        milliseconds of load after an idle spell.  Returns (calls, seconds)."""
        w0 = time.perf_counter()
        calls, prev = 0, None
        while True:
            ms, _ = self.run(lambda i: fn(calls + i), batch)
            calls += batch
            el = time.perf_counter() - w0
            steady = prev is not None and abs(ms - prev) <= tol * prev
            if (el >= seconds and steady) or el >= 4 * seconds:
                return calls, el
            prev = ms


def main():
    args = parse_args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, op=args.profile_op, workload=args.workload, B=args.batch)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, op=args.profile_op, workload=args.workload, B=args.batch)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the sampler runs on one GPU: --gpus must be 1", "n_gpus": args.gpus}),
              flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import lm_head_matmul_amd as fs
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ctx = fs.fs_create(0, max_B=256, max_V=262144, max_top_k=64)
    timer = Timer(torch)
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)  # noqa: E731

    weights = {}

    def load_W(name):
        if name not in weights:
            t0 = time.perf_counter()
            Wh = synth.workload_W(name)
            W = torch.from_numpy(Wh.view(np.int16)).view(torch.bfloat16).to(dev)
            # rotate copies so the step working set is >= 2 GB (MI355X has a 256 MB last-level cache)
            ncopy = max(1, math.ceil(2e9 / (W.numel() * 2)))
            copies = [W] + [W.clone() for _ in range(ncopy - 1)]
            weights[name] = (Wh, copies)
            log(f"{name}: W {tuple(W.shape)} x{ncopy} copies ready in {time.perf_counter() - t0:.1f}s")
        return weights[name]

    def H_for(name, B):
        return torch.from_numpy(synth.workload_H(name, B=B).view(np.int16)).view(torch.bfloat16).to(dev)

    def time_fmms(name, B, steps, warmup, T, mask=None, unfused=False, warm_s=0.3):
        _, Ws = load_W(name)
        H = H_for(name, B)
        out = torch.empty(B, dtype=torch.int32, device=dev)
        V = Ws[0].shape[0]
        logits = torch.empty((B, (V + 3) // 4 * 4), dtype=torch.float32, device=dev) if unfused else None
        call = fs.fs_unfused_sample if unfused else fs.fs_fmms_sample

        def step(i, base):
            kw = dict(mask=mask, out=out)
            if unfused:
                kw["logits_ws"] = logits
            call(ctx, H, Ws[i % len(Ws)], T, 0, base + i, **kw)

        timer.run(lambda i: step(i, 0), warmup)
        if warm_s > 0:  # clocks up after the W upload's idle spell
            timer.warm(lambda i: step(i, 100000), warm_s)
        ms, wall = timer.run(lambda i: step(i, warmup), steps)
        return ms, wall

    if args.profile:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = src.clone()
        torch.cuda.synchronize()
        del src, dst
        args.no_sweep = True
        args.no_cpu_baseline = True

    # --- headline ---------------------------------------------------------------
    w = synth.WORKLOADS[args.workload]
    B, d, V, T = args.batch, w["d"], w["V"], w["T"]
    algo = algorithmic_bytes(B, d, V)
    _, Wsh = load_W(args.workload)
    Hh = H_for(args.workload, B)
    outh = torch.empty(B, dtype=torch.int32, device=dev)

    op = PROFILE_OPS[args.profile_op] if args.profile else PROFILE_OPS["fused"]
    lg_h = torch.empty((B, (V + 3) // 4 * 4), dtype=torch.float32, device=dev) if op["unfused"] else None

    def hstep(i, base):
        if op["unfused"]:
            fs.fs_unfused_sample(ctx, Hh, Wsh[i % len(Wsh)], T, 0, base + i, top_k=op["top_k"], out=outh,
                                 logits_ws=lg_h)
        else:
            fs.fs_fmms_sample(ctx, Hh, Wsh[i % len(Wsh)], T, 0, base + i, top_k=op["top_k"], out=outh)

    log(f"headline {args.workload} B={B} d={d} V={V}: {args.warmup} warmup + {args.steps} timed steps")
    # the driver's warmup, then the same K steps timed at once: what a fresh process sees
    # while the GPU's clocks ramp up
    timer.run(lambda i: hstep(i, 0), args.warmup)
    cold_ms = None if args.profile else timer.run(lambda i: hstep(i, args.warmup), args.steps)[0]
    # pre-run of the same call, outside the timed region: at least 1 s and until two
    # consecutive 50-step batches agree within 1%
    pre_calls, pre_s = timer.warm(lambda i: hstep(i, 10**6), 0.5 if args.profile else 1.0)
    log(f"headline cold {cold_ms and cold_ms * 1e3} us/step; pre-run {pre_calls} steps in {pre_s:.2f}s")
    # the timed region: exactly K steps
    ms, wall = timer.run(lambda i: hstep(i, 2 * 10**6), args.steps)
    gbs = algo / (ms * 1e-3) / 1e9
    # the streaming kernel's own duration: the next K steps with each launch between a pair
    # of events recorded by the library (the extra event records cost the step ~7 us, so
    # the step time above is taken without them)
    _, _, kern_ms = timer.run_with_kernel_events(lambda i: hstep(i, 3 * 10**6), args.steps,
                                                 lambda a, b: fs.fs_profile_next_launch(ctx, a, b))
    kgbs = algo / (kern_ms * 1e-3) / 1e9
    log(f"headline: {ms * 1e3:.1f} us/step ({gbs:.0f} GB/s, {gbs / PEAK_HBM_GBS:.1%} of 8 TB/s); streaming kernel "
        f"{kern_ms * 1e3:.1f} us ({kgbs:.0f} GB/s, {kgbs / PEAK_HBM_GBS:.1%}); wall {wall:.3f}s")
    # five more K-step runs (median), and single-step latency
    reps, lat = [ms] * 5, [ms]
    if not args.profile:
        reps = sorted(timer.run(lambda i, r=r: hstep(i, (4 + r) * 10**6), args.steps)[0] for r in range(5))
        lat = sorted(timer.run(lambda j, i=i: hstep(j, 9 * 10**6 + i), 1)[0] for i in range(20))
    if args.profile:
        ms_u = None
    else:
        ms_u, _ = time_fmms(args.workload, B, min(args.steps, 200), 10, T, unfused=True)
        log(f"headline unfused: {ms_u * 1e3:.1f} us/step")

    tr = {o: measured_traffic(o, args.workload, B) for o in PROFILE_OPS}
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02^2) LM-head weights; no trained weights)",
        "config": {"workload": f"{args.workload}_head", "B": B, "d": d, "V": V, "temperature": T, "top_k": 0,
                   "us_per_step": round(ms * 1e3, 2), "rows_per_s": round(B / (ms * 1e-3)),
                   "pct_of_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                   "stream_kernel_us": round(kern_ms * 1e3, 2),
                   "median_of_5_us_per_step": round(reps[2] * 1e3, 2),
                   "single_step_latency_us_median": round(lat[len(lat) // 2] * 1e3, 2),
                   "cold_us_per_step": None if cold_ms is None else round(cold_ms * 1e3, 2),
                   "cold_note": "the same K steps right after the driver's warmup, before the pre-run: the "
                                "GPU's clocks ramp up over the first ~100 ms of load",
                   "prerun": {"steps": pre_calls, "seconds": round(pre_s, 3)},
                   "unfused_us_per_step": None if ms_u is None else round(ms_u * 1e3, 2),
                   "fused_speedup_vs_unfused": None if ms_u is None else round(ms_u / ms, 3)},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(kgbs / PEAK_HBM_GBS, 4), "traffic": tr["fused"],
                     "traffic_unfused": tr["unfused"], "traffic_top50": tr["topk"],
                     "hbm_bytes_saved_vs_unfused_per_step": (None if tr["fused"] is None or tr["unfused"] is None
                                                             else tr["unfused"] - tr["fused"]),
                     "algorithmic_bytes_per_launch": algo,
                     "kernel_us": round(kern_ms * 1e3, 2),
                     "floors": floors(B, w["d"], w["V"]),
                     "note": "achieved = algorithmic bytes of one launch / the streaming kernel's mean duration "
                             "(HIP events around each launch, K steps right after the timed region); traffic = calibrated "
                             "FETCH_SIZE + WRITE_SIZE per launch from profiles/ (null if the kernels changed)"},
        "context": "pages: up to 19% lower time per output token end to end in vLLM on NVIDIA "
                   "H100/H200/B200/B300 (not comparable; context only)",
    }

    # --- sweep ------------------------------------------------------------------
    if not args.no_sweep:
        sweep = []
        n = args.sweep_steps
        for name, Bs in (("small_decode", synth.WORKLOADS["small_decode"]["Bs"]),
                         ("mid_decode", synth.WORKLOADS["mid_decode"]["Bs"])):
            ww = synth.WORKLOADS[name]
            for b in Bs:
                f_ms, _ = time_fmms(name, b, n, 10, ww["T"])
                u_ms, _ = time_fmms(name, b, max(20, n // 4), 5, ww["T"], unfused=True)
                ab = algorithmic_bytes(b, ww["d"], ww["V"])
                sweep.append({"workload": name, "B": b, "d": ww["d"], "V": ww["V"], "us_per_step": round(f_ms * 1e3, 2),
                              "GB_per_s": round(ab / (f_ms * 1e-3) / 1e9, 1),
                              "pct_peak": round(100 * ab / (f_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                              "rows_per_s": round(b / (f_ms * 1e-3)), "unfused_us_per_step": round(u_ms * 1e3, 2),
                              "speedup_vs_unfused": round(u_ms / f_ms, 3), **floors(b, ww["d"], ww["V"])})
                log(f"sweep {sweep[-1]}")
            del weights[name]
            torch.cuda.empty_cache()
        # the mid decode head's top-k variant (k = 50)
        wt = synth.WORKLOADS["mid_decode"]
        for b in (8, 64):
            _, Wt = load_W("mid_decode")
            Ht = H_for("mid_decode", b)
            outt = torch.empty(b, dtype=torch.int32, device=dev)
            lgt = torch.empty((b, (wt["V"] + 3) // 4 * 4), dtype=torch.float32, device=dev)

            def tk(i, base, unf):
                if unf:
                    fs.fs_unfused_sample(ctx, Ht, Wt[i % len(Wt)], wt["T"], 0, base + i, top_k=50, out=outt,
                                         logits_ws=lgt)
                else:
                    fs.fs_fmms_sample(ctx, Ht, Wt[i % len(Wt)], wt["T"], 0, base + i, top_k=50, out=outt)

            # warmed up like the plain sampler's lines (clocks ramp after the idle spell)
            timer.run(lambda i: tk(i, 0, False), 5)
            timer.warm(lambda i: tk(i, 100000, False), 0.3)
            k_ms, _ = timer.run(lambda i: tk(i, 10, False), n)
            timer.run(lambda i: tk(i, 0, True), 5)
            timer.warm(lambda i: tk(i, 100000, True), 0.3)
            ku_ms, _ = timer.run(lambda i: tk(i, 10, True), max(20, n // 4))
            ab = algorithmic_bytes(b, wt["d"], wt["V"])
            sweep.append({"workload": "mid_decode_top50", "B": b, "d": wt["d"], "V": wt["V"], "top_k": 50,
                          "us_per_step": round(k_ms * 1e3, 2), "GB_per_s": round(ab / (k_ms * 1e-3) / 1e9, 1),
                          "pct_peak": round(100 * ab / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                          "unfused_us_per_step": round(ku_ms * 1e3, 2)})
            log(f"sweep {sweep[-1]}")
        # the conventional comparator (logits, softmax, prefix sum, inverse-CDF search) and the
        # LM-head GEMM alone through hipBLASLt (torch's linear, bf16 logits), next to the fused sampler
        for b in (1, 8, 64):
            _, Wt = load_W("mid_decode")
            Ht = H_for("mid_decode", b)
            outc = torch.empty(b, dtype=torch.int32, device=dev)
            lgc = torch.empty((b, (wt["V"] + 3) // 4 * 4), dtype=torch.float32, device=dev)

            def cs(i, base):
                fs.fs_softmax_sample(ctx, Ht, Wt[i % len(Wt)], wt["T"], 0, base + i, out=outc, logits_ws=lgc)

            def mm(i, base):
                torch.nn.functional.linear(Ht, Wt[i % len(Wt)])

            timer.run(lambda i: cs(i, 0), 5)
            c_ms, _ = timer.run(lambda i: cs(i, 10), max(20, n // 4))
            timer.run(lambda i: mm(i, 0), 5)
            g_ms, _ = timer.run(lambda i: mm(i, 10), max(20, n // 4))
            f_ms, _ = time_fmms("mid_decode", b, max(20, n // 4), 5, wt["T"])
            sweep.append({"workload": "mid_decode_conventional", "B": b, "d": wt["d"], "V": wt["V"],
                          "conventional_us_per_step": round(c_ms * 1e3, 2), "fmms_us_per_step": round(f_ms * 1e3, 2),
                          "torch_linear_gemm_only_us": round(g_ms * 1e3, 2),
                          "fmms_speedup_vs_conventional": round(c_ms / f_ms, 3)})
            log(f"sweep {sweep[-1]}")
        # several samples per row from one pass over W, against as many single-sample steps
        for b, S in ((8, 4), (16, 4)):
            _, Wt = load_W("mid_decode")
            Ht = H_for("mid_decode", b)
            outm = torch.empty((b, S), dtype=torch.int32, device=dev)
            outs = torch.empty(b, dtype=torch.int32, device=dev)

            def ms(i, base):
                fs.fs_fmms_sample_multi(ctx, Ht, Wt[i % len(Wt)], wt["T"], 0, (base + i) * S, S, out=outm)

            def ss(i, base):
                fs.fs_fmms_sample(ctx, Ht, Wt[(i // S) % len(Wt)], wt["T"], 0, base + i, out=outs)

            timer.run(lambda i: ms(i, 0), 5)
            m_ms, _ = timer.run(lambda i: ms(i, 10), max(20, n // 4))
            timer.run(lambda i: ss(i, 0), 5)
            s_ms, _ = timer.run(lambda i: ss(i, 10), max(20, n // 4) * S)
            sweep.append({"workload": "mid_decode_multi", "B": b, "num_samples": S, "d": wt["d"], "V": wt["V"],
                          "us_per_call": round(m_ms * 1e3, 2), "us_for_same_samples_one_per_call":
                          round(s_ms * S * 1e3, 2), "speedup": round(s_ms * S / m_ms, 3)})
            log(f"sweep {sweep[-1]}")
        del weights["mid_decode"]
        torch.cuda.empty_cache()
        # masked workload
        wm = synth.WORKLOADS["masked"]
        mask = torch.from_numpy(synth.workload_mask("masked").view(np.int32)).to(dev)
        f_ms, _ = time_fmms("masked", wm["B"], n, 10, wm["T"], mask=mask)
        u_ms, _ = time_fmms("masked", wm["B"], max(20, n // 4), 5, wm["T"], mask=mask, unfused=True)
        ab = algorithmic_bytes(wm["B"], wm["d"], wm["V"], mask=True)
        sweep.append({"workload": "masked", "B": wm["B"], "d": wm["d"], "V": wm["V"], "us_per_step": round(f_ms * 1e3, 2),
                      "GB_per_s": round(ab / (f_ms * 1e-3) / 1e9, 1),
                      "pct_peak": round(100 * ab / (f_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                      "unfused_us_per_step": round(u_ms * 1e3, 2), "speedup_vs_unfused": round(u_ms / f_ms, 3)})
        log(f"sweep {sweep[-1]}")
        del weights["masked"]
        torch.cuda.empty_cache()
        # grouped workload: 8 group summaries + combine per step
        wg = synth.WORKLOADS["grouped"]
        _, Wg = load_W("grouped")
        Hg = H_for("grouped", wg["B"])
        G = wg["V"] // wg["n_groups"]
        summ = torch.empty((wg["n_groups"], wg["B"], 3), dtype=torch.int32, device=dev)
        outg = torch.empty(wg["B"], dtype=torch.int32, device=dev)

        def gstep(i):
            Wc = Wg[i % len(Wg)]
            for k in range(wg["n_groups"]):
                fs.fs_group_summary(ctx, Hg, Wc[k * G:(k + 1) * G], k * G, wg["T"], 0, i, out=summ[k])
            fs.fs_group_combine(ctx, summ, 0, i, fs.FS_COMBINE_GUMBEL, out=outg)

        timer.run(gstep, 5)
        g_ms, _ = timer.run(gstep, max(20, n // 4))
        ab = algorithmic_bytes(wg["B"], wg["d"], wg["V"]) + wg["n_groups"] * wg["B"] * wg["d"] * 2
        sweep.append({"workload": "grouped", "B": wg["B"], "d": wg["d"], "V": wg["V"], "groups": wg["n_groups"],
                      "launch": "one per group", "us_per_step": round(g_ms * 1e3, 2),
                      "GB_per_s": round(ab / (g_ms * 1e-3) / 1e9, 1),
                      "pct_peak": round(100 * ab / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)})
        log(f"sweep {sweep[-1]}")

        # the same summaries for all groups in one launch, then the combine
        def gstep1(i):
            fs.fs_group_summaries(ctx, Hg, Wg[i % len(Wg)], 0, G, wg["T"], 0, i, out=summ)
            fs.fs_group_combine(ctx, summ, 0, i, fs.FS_COMBINE_GUMBEL, out=outg)

        timer.run(gstep1, 5)
        g1_ms, _ = timer.run(gstep1, max(20, n // 4))
        ab1 = algorithmic_bytes(wg["B"], wg["d"], wg["V"])
        sweep.append({"workload": "grouped", "B": wg["B"], "d": wg["d"], "V": wg["V"], "groups": wg["n_groups"],
                      "launch": "all groups in one", "us_per_step": round(g1_ms * 1e3, 2),
                      "GB_per_s": round(ab1 / (g1_ms * 1e-3) / 1e9, 1),
                      "pct_peak": round(100 * ab1 / (g1_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)})
        log(f"sweep {sweep[-1]}")

        # the online producer: one launch whose group k starts once its flag is published (here every
        # flag carries the step's epoch before the launch, so no tile waits), then the combine
        ready = torch.zeros(wg["n_groups"], dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def gstep2(i):
            ready.fill_(i + 1)  # the producer publishes every group of step i (epoch i + 1)
            fs.fs_group_summaries_online(ctx, Hg, Wg[i % len(Wg)], 0, G, wg["T"], 0, i, ready, i + 1, status,
                                         out=summ)
            fs.fs_group_combine(ctx, summ, 0, i, fs.FS_COMBINE_GUMBEL, out=outg)

        timer.run(gstep2, 5)
        g2_ms, _ = timer.run(gstep2, max(20, n // 4))
        torch.cuda.synchronize()
        sweep.append({"workload": "grouped", "B": wg["B"], "d": wg["d"], "V": wg["V"], "groups": wg["n_groups"],
                      "launch": "online producer (one launch; each group starts once published)",
                      "us_per_step": round(g2_ms * 1e3, 2), "GB_per_s": round(ab1 / (g2_ms * 1e-3) / 1e9, 1),
                      "pct_peak": round(100 * ab1 / (g2_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                      "waits_given_up": int(status.item())})
        log(f"sweep {sweep[-1]}")
        del weights["grouped"]
        result["sweep"] = sweep

    # --- CPU baseline: the oracle on the host's cores -----------------------------
    if not args.no_cpu_baseline:
        import oracle

        Wh = synth.workload_W(args.workload)
        Hh = synth.workload_H(args.workload, B=B)
        oracle.lib()
        cores = oracle.num_threads()
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as fh:
                cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
        except (OSError, StopIteration):
            pass
        # runs of r rows each, until the time budget or the step's rows are used up; the per-row
        # cost is the median over runs (the oracle's cost is linear in the rows it samples)
        r = min(8, B)
        per_row, rows_done, t_used = [], 0, 0.0
        t0 = time.perf_counter()
        while t_used < args.cpu_seconds and (rows_done < B or len(per_row) < 3):
            r0 = rows_done % B
            t1 = time.perf_counter()
            oracle.fmms_sample(Hh[r0:r0 + r], Wh, T, 0, 0)
            per_row.append((time.perf_counter() - t1) / len(Hh[r0:r0 + r]))
            rows_done += len(Hh[r0:r0 + r])
            t_used = time.perf_counter() - t0
        per_row.sort()
        per_step = per_row[len(per_row) // 2] * B
        cpu_gbs = algo / per_step / 1e9
        sample = (f"{len(per_row)} runs of {r} rows of the headline step (full V={V}, d={d}: fp64 logits, noise, "
                  f"argmax), {rows_done} rows in {t_used:.1f}s; step time = median per-row time x {B} rows")
        result["cpu_baseline"] = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                                  "sample": sample, "cpu_model": cpu_model, "runs": len(per_row),
                                  "seconds_per_step": round(per_step, 3), "us_per_step": round(per_step * 1e6, 1),
                                  "per_row_seconds_min_median_max": [round(per_row[0], 4),
                                                                     round(per_row[len(per_row) // 2], 4),
                                                                     round(per_row[-1], 4)]}
        # the tiny configuration (B=4, d=256, V=4096) on one thread, median of 20 calls
        try:
            import ctypes
            gomp = ctypes.CDLL("libgomp.so.1")
            wt = synth.WORKLOADS["tiny"]
            Ht = synth.workload_H("tiny", B=wt["B"])
            Wt0 = synth.workload_W("tiny")
            gomp.omp_set_num_threads(1)
            ts = []
            for _ in range(20):
                t1 = time.perf_counter()
                oracle.fmms_sample(Ht, Wt0, wt["T"], 0, 0)
                ts.append(time.perf_counter() - t1)
            gomp.omp_set_num_threads(cores)
            ts.sort()
            result["cpu_baseline"]["tiny_single_thread"] = {
                "config": f"B={wt['B']} d={wt['d']} V={wt['V']}", "threads": 1, "calls": len(ts),
                "us_per_step_median": round(ts[len(ts) // 2] * 1e6, 1)}
        except OSError as e:
            result["cpu_baseline"]["tiny_single_thread"] = {"error": str(e)}
        log(f"cpu baseline {result['cpu_baseline']}")

    fs.fs_destroy(ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
