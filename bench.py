"""Benchmark of the fused memory-bound chains on one MI355X.

One step = one call of every fused entry point on its full workload (the whole
hot path): the pointwise chain (4M fp32), the 10-op graph (1024x1024 fp32),
LayerNorm (8192x4096 fp32), residual + LayerNorm + GeLU (16384x8192 bf16) and
the hidden-size sweep (262144x768, 32768x4095, 16384x12288 bf16).  Inputs are
resident in HBM before the timed region.  The step touches ~4.4 GB, so each
kernel finds its inputs evicted from the 256 MB Infinity Cache by the others
(cold-cache timing without buffer rotation).

Printed: one JSON line with
  value        whole-step effective bandwidth: compulsory bytes of all seven
               calls / wall time per step (GB/s, 1e9 B/s);
  per_workload per kernel: mean/median duration from HIP events on the launch
               stream (a pass of K steps before the timed region, every call
               bracketed), effective GB/s, fraction of 8 TB/s, the unfused
               variant's time (all its launches) and the speedup;
  roofline     the dominant kernel (largest time per step), its duration from
               HIP events around it inside the timed region, against 8 TB/s;
  cpu_baseline the CPU oracle timed on a bounded sample of the same workloads.

Other modes (for rocprofv3 counter runs): --only NAME runs just one workload's
fused kernel; --copy-bytes B runs the library's streaming copy of B bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-kernel effective HBM GB/s (% of ~8 TB/s peak) + µs/call vs unfused"
PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--unfused-reps", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=2,
                   help="the oracle runs on 1/K of each workload's rows")
    p.add_argument("--only", default=None, help="run only this workload's fused kernel")
    p.add_argument("--unfused-only", default=None, help="run only this workload's unfused variant")
    p.add_argument("--copy-bytes", type=int, default=0, help="run the streaming copy of this size")
    return p.parse_args()


def library_sha256() -> str:
    """Hash of the library sources and build flags (identifies the kernels)."""
    h = hashlib.sha256()
    base = os.path.join(ROOT, "memory_bound_pointwise_amd")
    files = [os.path.join(base, "build.py")]
    files += sorted(os.path.join(base, "csrc", f) for f in os.listdir(os.path.join(base, "csrc")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(name: str, sha: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernels."""
    path = os.path.join(PROFILES, f"hbm_traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("library_sha256") != sha:
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"])) + int(float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the fused kernels "
              "are single-GPU; sharding is described, not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import memory_bound_pointwise_amd as mbp
    import workloads as W
    to_dev = lambda a: W.to_device(a, dev)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            mbp.stream_copy(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes": n * 4, "launches": args.warmup + args.steps}))
        return

    names = [w.name for w in W.WORKLOADS]
    if args.only:
        names = [args.only]
    if args.unfused_only:
        names = [args.unfused_only]
    wl = [W.BY_NAME[n] for n in names]

    # ---- inputs resident in HBM
    t_gen = time.time()
    host, calls, ucalls, uinfo = {}, {}, {}, {}
    for w in wl:
        d = W.generate(w)
        host[w.name] = d
        if w.kind == "chain":
            x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
            y = torch.empty_like(x)
            s = w.params["scale"]
            ws = torch.empty(mbp.workspace_bytes(mbp.OP_CHAIN, mbp.F32, 1, w.n), dtype=torch.uint8, device=dev)
            uy = torch.empty_like(x)
            calls[w.name] = lambda x=x, b1=b1, b2=b2, y=y, s=s: mbp.fused_pointwise_chain(x, b1, b2, s, out=y)
            ucalls[w.name] = lambda x=x, b1=b1, b2=b2, y=uy, s=s, ws=ws: mbp.unfused_pointwise_chain(
                x, b1, b2, s, out=y, workspace=ws)
            uinfo[w.name] = mbp.launches_per_call(mbp.OP_CHAIN, False)
        elif w.kind == "row_mean":
            x, bias, g, b = (to_dev(d[k]) for k in ("x", "bias", "gamma", "beta"))
            y = torch.empty_like(x)
            al, c = w.params["alpha"], w.params["c"]
            ws = torch.empty(mbp.workspace_bytes(mbp.OP_ROW_MEAN, mbp.F32, w.rows, w.cols), dtype=torch.uint8,
                             device=dev)
            uy = torch.empty_like(x)
            calls[w.name] = lambda x=x, bias=bias, g=g, b=b, y=y, al=al, c=c: mbp.fused_row_mean_epilogue(
                x, bias, g, b, al, c, out=y)
            ucalls[w.name] = lambda x=x, bias=bias, g=g, b=b, y=uy, al=al, c=c, ws=ws: \
                mbp.unfused_row_mean_epilogue(x, bias, g, b, al, c, out=y, workspace=ws)
            uinfo[w.name] = mbp.launches_per_call(mbp.OP_ROW_MEAN, False)
        else:
            x, r, g, b = (to_dev(d[k]) for k in ("x", "residual", "gamma", "beta"))
            y = torch.empty_like(x)
            eps, act = w.params["eps"], w.act
            dcode = mbp.BF16 if w.dtype == "bf16" else mbp.F32
            ws = torch.empty(mbp.workspace_bytes(mbp.OP_LAYERNORM, dcode, w.rows, w.cols, r is not None, act),
                             dtype=torch.uint8, device=dev)
            uy = torch.empty_like(x)
            calls[w.name] = lambda x=x, r=r, g=g, b=b, y=y, eps=eps, act=act: mbp.fused_add_layernorm_gelu(
                x, r, g, b, eps, act, out=y)
            ucalls[w.name] = lambda x=x, r=r, g=g, b=b, y=uy, eps=eps, act=act, ws=ws: \
                mbp.unfused_add_layernorm_gelu(x, r, g, b, eps, act, out=y, workspace=ws)
            uinfo[w.name] = mbp.launches_per_call(mbp.OP_LAYERNORM, False, has_residual=r is not None, act=act)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    if args.unfused_only:
        for _ in range(args.warmup + args.steps):
            ucalls[names[0]]()
        torch.cuda.synchronize()
        print(json.dumps({"mode": "unfused-only", "workload": names[0], "calls": args.warmup + args.steps}))
        return

    stream = torch.cuda.current_stream(dev)

    def step_events(k_steps):
        """k_steps steps with every fused call bracketed by HIP events on its
        launch stream; returns per-workload durations in us."""
        ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(k_steps)] for n in names}
        for k in range(k_steps):
            for n in names:
                e0, e1 = ev[n][k]
                e0.record(stream)
                calls[n]()
                e1.record(stream)
        torch.cuda.synchronize()
        return {n: [ev[n][k][0].elapsed_time(ev[n][k][1]) * 1e3 for k in range(k_steps)] for n in names}

    # ---- per-kernel pass: every call timed on its own (not the timed region;
    # the events between kernels add launch gaps that the timed region avoids)
    for n in names:
        calls[n]()
    torch.cuda.synchronize()
    fused_us = step_events(args.steps)
    dominant = max(names, key=lambda n: statistics.fmean(fused_us[n]))

    for _ in range(args.warmup):
        for n in names:
            calls[n]()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps; only the dominant kernel is bracketed
    # by events (its live duration feeds the roofline)
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for n in names:
            if n == dominant:
                dom_ev[k][0].record(stream)
                calls[n]()
                dom_ev[k][1].record(stream)
            else:
                calls[n]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_us_live = [a.elapsed_time(b) * 1e3 for a, b in dom_ev]

    # ---- unfused variants, same interleaved protocol
    unf_us = {n: [] for n in names}
    if args.unfused_reps and not args.only:
        for n in names:
            ucalls[n]()
        torch.cuda.synchronize()
        uev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.unfused_reps)] for n in names}
        for k in range(args.unfused_reps):
            for n in names:
                e0, e1 = uev[n][k]
                e0.record(stream)
                ucalls[n]()
                e1.record(stream)
        torch.cuda.synchronize()
        unf_us = {n: [uev[n][k][0].elapsed_time(uev[n][k][1]) * 1e3 for k in range(args.unfused_reps)]
                  for n in names}

    per = {}
    total_bytes = 0
    for w in wl:
        n = w.name
        B = w.compulsory_bytes
        total_bytes += B
        mean_us = statistics.fmean(fused_us[n])
        med_us = statistics.median(fused_us[n])
        rec = {
            "compulsory_bytes": B,
            "fused_us_mean": round(mean_us, 3),
            "fused_us_median": round(med_us, 3),
            "fused_us_min": round(min(fused_us[n]), 3),
            "gbps": round(B / (mean_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(B / (mean_us * 1e-6) / 1e9 / PEAK_GBPS, 4),
            "launches_fused": 1,
        }
        if unf_us[n]:
            um = statistics.median(unf_us[n])
            rec.update({"unfused_us_median": round(um, 3), "launches_unfused": uinfo[n],
                        "speedup_vs_unfused": round(um / med_us, 3)})
        per[n] = rec

    dw = W.BY_NAME[dominant]
    dom_us = statistics.fmean(dom_us_live)
    achieved = dw.compulsory_bytes / (dom_us * 1e-6) / 1e9
    sha = library_sha256()
    traffic = read_traffic(dominant, sha)
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": dw.compulsory_bytes, "avg_launch_us": round(dom_us, 3)}

    cpu = None
    if not args.no_cpu_baseline and not args.only:
        cpu = cpu_baseline(wl, host, args.cpu_sample)

    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64 (fp32 I/O) / f32 (bf16 I/O)",
        "data": "synthetic (seeded; shapes and distributions of the five workloads)",
        "config": {"workload": "one call each: " + ", ".join(names), "bytes_per_step": total_bytes,
                   "kernels_per_step": len(names), "frac_of_peak": round(value / PEAK_GBPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_workload": per,
        "library_sha256": sha[:16],
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(out))


def cpu_baseline(wl, host, frac):
    """The oracle (plain C, single thread, binary64) on the first 1/frac of each
    workload's rows (elements for the chain); GB/s on the same compulsory bytes."""
    import oracle
    import workloads as W

    t_total = 0.0
    b_total = 0
    for w in wl:
        d = host[w.name]
        if w.kind == "chain":
            n = w.n // frac
            t = time.perf_counter()
            oracle.pointwise_chain(d["x"][:n], d["b1"][:n], d["b2"][:n], w.params["scale"])
            t_total += time.perf_counter() - t
            b_total += W.scaled(w, n=n).compulsory_bytes
            continue
        rows = max(1, w.rows // frac)
        t = time.perf_counter()
        if w.kind == "row_mean":
            oracle.row_mean_epilogue(d["x"][:rows], d["bias"], d["gamma"], d["beta"], w.params["alpha"],
                                     w.params["c"])
        else:
            r = None if d["residual"] is None else d["residual"][:rows]
            oracle.add_layernorm_gelu(d["x"][:rows], r, d["gamma"], d["beta"], w.params["eps"],
                                      oracle.ACT_GELU_TANH if w.act == "gelu_tanh" else oracle.ACT_NONE)
        t_total += time.perf_counter() - t
        b_total += W.scaled(w, rows=rows).compulsory_bytes
    return {"value": round(b_total / t_total / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first 1/{frac} of the rows (elements) of each of the {len(wl)} workloads, "
                      f"{b_total} compulsory bytes, {t_total:.1f} s, binary64, single thread"}


if __name__ == "__main__":
    main()
