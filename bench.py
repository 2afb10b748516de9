#!/usr/bin/env python3
"""Benchmark of FlashSampling's fused LM-head matmul + sample (FMMS) on one MI355X.

One step = one fs_fmms_sample call (stream W, logits on chip, scale, noise,
tile argmax, cross-tile reduction) over a fixed synthetic batch, with the step
counter incrementing.  Headline: the mid-size decode head (d=4096, V=151936,
B=64, T=0.7).  Prints ONE JSON line.

  value     achieved HBM GB/s = algorithmic bytes per step (V*d*2 + B*d*2 + B*4)
            / measured time per step (HIP events on the launch stream)
  roofline  that figure against MI355X's 8 TB/s; `traffic` is the measured
            HBM bytes per launch from the committed rocprofv3 counter summary
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
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fmms_mid_decode_B64_hbm_traffic.md")
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
                         "headline steps only")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write the profiles/ summaries from a --profile run's rocprofv3 csv output and exit")
    return ap.parse_args()


def algorithmic_bytes(B, d, V, mask=False):
    return V * d * 2 + B * d * 2 + B * 4 + (B * ((V + 31) // 32) * 4 if mask else 0)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches these kernels."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    with open(TRAFFIC_SUMMARY) as fh:
        for line in fh:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace -o trace "
             "-- python3 bench.py --profile --steps 1000 --warmup 50",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fetch -o fetch "
             "-- python3 bench.py --profile --steps 5 --warmup 2",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_write -o write "
             "-- python3 bench.py --profile --steps 5 --warmup 2",
}

def headline_kernel_name(names):
    """The streaming kernel of the step: the library's kernel with the largest total time."""
    ours = [n for n in names if "fsk::" in n and "reduce_tiles" not in n]
    return ours[0] if ours else None


def summarize_profiles(trace_csv, fetch_csv, write_csv, workload="mid_decode", B=64):
    """Turn a --profile run's rocprofv3 csv files into the two committed text summaries."""
    import csv
    import synth

    w = synth.WORKLOADS[workload]
    algo = algorithmic_bytes(B, w["d"], w["V"])
    tag = f"{workload}_B{B}"
    pre = "cd /tmp && export TMPDIR=/tmp && cd <repo root> && "

    stats = sorted(csv.DictReader(open(trace_csv)), key=lambda r: -float(r["TotalDurationNs"]))
    kname = headline_kernel_name([r["Name"] for r in stats])
    assert kname is not None, "no library kernel in the trace"
    head = [r for r in stats if r["Name"] == kname]
    avg_us = float(head[0]["AverageNs"]) / 1e3
    short = kname.split("(")[0].split("::")[-1].split("<")[0]
    lines = [f"# {short}: {workload} head (B={B}, d={w['d']}, V={w['V']}), kernel trace", "",
             f"headline kernel: `{kname}`", "",
             f"command: `{pre}{PROFILE_CMDS['trace']}`", "",
             "The run: one 1 GiB device fill and copy (counter calibration), 50 warmup and 1000 timed steps.", "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    lines += ["", f"- headline_kernel_average_us: {avg_us:.2f}",
              f"- algorithmic_bytes_per_launch: {algo}",
              f"- achieved_GB_per_s_at_trace_average: {algo / (avg_us * 1e-6) / 1e9:.1f}",
              f"- kernel_source_sha256_16: {kernel_source_hash()}", ""]
    path = os.path.join(ROOT, "profiles", f"{short}_{tag}_kernel_trace.md")
    open(path, "w").write("\n".join(lines))

    def rows(fn):
        return list(csv.DictReader(open(fn)))

    def calib(rs, counter):
        # the fill kernel writes CALIB_BYTES; the copy that follows it reads CALIB_BYTES
        fill = next(i for i, r in enumerate(rs) if "FillFunctor<short>" in r["Kernel_Name"])
        copy = next(r for r in rs[fill + 1:] if "copyBuffer" in r["Kernel_Name"])
        kib = float((rs[fill] if counter == "WRITE_SIZE" else copy)["Counter_Value"])
        return (CALIB_BYTES / 1024) / kib, kib

    fr, wr = rows(fetch_csv), rows(write_csv)
    f_fac, f_cal = calib(fr, "FETCH_SIZE")
    w_fac, w_cal = calib(wr, "WRITE_SIZE")
    f_k = [float(r["Counter_Value"]) for r in fr if r["Kernel_Name"] == kname]
    w_k = [float(r["Counter_Value"]) for r in wr if r["Kernel_Name"] == kname]
    assert f_k and w_k, "the headline kernel is missing from a counter pass"
    f_kib, w_kib = sum(f_k) / len(f_k), sum(w_k) / len(w_k)
    hbm = f_kib * 1024 * f_fac + w_kib * 1024 * w_fac
    lines = [f"# {short}: {workload} head (B={B}, d={w['d']}, V={w['V']}), HBM traffic per launch", "",
             f"kernel: `{kname}`", "",
             f"fetch pass: `{pre}{PROFILE_CMDS['fetch']}`", "",
             f"write pass: `{pre}{PROFILE_CMDS['write']}`", "",
             "Calibration: the same runs first fill 1 GiB (a pure write) and copy it (a 1 GiB read + write).",
             f"FETCH_SIZE reads {f_cal:.1f} KiB for the copy's 1048576 KiB read (factor {f_fac:.5f});",
             f"WRITE_SIZE reads {w_cal:.1f} KiB for the fill's 1048576 KiB write (factor {w_fac:.5f}).",
             f"Kernel dispatches seen: {len(f_k)} (fetch pass), {len(w_k)} (write pass).", "",
             f"- fetch_kib_per_launch_raw: {f_kib:.1f}",
             f"- write_kib_per_launch_raw: {w_kib:.1f}",
             f"- fetch_scale: {f_fac:.5f}",
             f"- write_scale: {w_fac:.5f}",
             f"- hbm_bytes_per_launch: {hbm:.0f}",
             f"- algorithmic_bytes_per_launch: {algo}",
             f"- traffic_over_algorithmic: {hbm / algo:.4f}",
             f"- kernel_source_sha256_16: {kernel_source_hash()}", ""]
    open(TRAFFIC_SUMMARY, "w").write("\n".join(lines))
    print(f"wrote {path} and {TRAFFIC_SUMMARY}: avg {avg_us:.1f} us, traffic {hbm / algo:.4f} x algorithmic")


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


def main():
    args = parse_args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles)
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

    def time_fmms(name, B, steps, warmup, T, mask=None, unfused=False):
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
    log(f"headline {args.workload} B={B} d={d} V={V}: {args.warmup} warmup + {args.steps} timed steps")
    ms, wall = time_fmms(args.workload, B, args.steps, args.warmup, T)
    algo = algorithmic_bytes(B, d, V)
    gbs = algo / (ms * 1e-3) / 1e9
    log(f"headline: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of 8 TB/s), wall {wall:.3f}s")
    if args.profile:
        ms_u = None
    else:
        ms_u, _ = time_fmms(args.workload, B, min(args.steps, 200), 10, T, unfused=True)
        log(f"headline unfused: {ms_u * 1e3:.1f} us/step")

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
                   "unfused_us_per_step": None if ms_u is None else round(ms_u * 1e3, 2),
                   "fused_speedup_vs_unfused": None if ms_u is None else round(ms_u / ms, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": algo},
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
                              "speedup_vs_unfused": round(u_ms / f_ms, 3)})
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

            timer.run(lambda i: tk(i, 0, False), 5)
            k_ms, _ = timer.run(lambda i: tk(i, 10, False), max(20, n // 4))
            timer.run(lambda i: tk(i, 0, True), 5)
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
        del weights["grouped"]
        result["sweep"] = sweep

    # --- CPU baseline: the oracle on the host's cores -----------------------------
    if not args.no_cpu_baseline:
        import oracle

        Wh = synth.workload_W(args.workload)
        Hh = synth.workload_H(args.workload, B=B)
        oracle.lib()
        cores = oracle.num_threads()
        rows_done, t_used = 0, 0.0
        t0 = time.perf_counter()
        r = min(8, B)
        while t_used < args.cpu_seconds and rows_done < B:
            oracle.fmms_sample(Hh[rows_done:rows_done + r], Wh, T, 0, 0)
            rows_done += r
            t_used = time.perf_counter() - t0
        per_step = t_used / rows_done * B  # the oracle's cost is linear in the rows it samples
        cpu_gbs = algo / per_step / 1e9
        sample = (f"{rows_done} of the {B} rows of one step (full V={V}, d={d}: fp64 logits, noise, argmax) "
                  f"in {t_used:.1f}s" + ("" if rows_done == B else f"; step time scaled by {B}/{rows_done}"))
        result["cpu_baseline"] = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                                  "sample": sample, "seconds_per_step": round(per_step, 3),
                                  "us_per_step": round(per_step * 1e6, 1)}
        log(f"cpu baseline {result['cpu_baseline']}")

    fs.fs_destroy(ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
