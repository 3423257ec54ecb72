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
  per_workload per kernel: GPU time per call from batches of N back-to-back
               calls between two HIP events on the launch stream (N such that
               a batch takes about 1 ms; median, min and p90 over the
               batches), the calls rotating over B copies of the inputs and
               outputs with B x working set >= 1 GiB so every call starts
               cold.  Each batch is captured once as a HIP graph and replayed,
               so host work (Python, ctypes, the launch call) stays out of
               the kernels' time; the same batch issued eagerly from Python
               is reported beside it (eager_us_median: for the small
               workloads that one is bound by the host's issue rate).
               Effective GB/s, fraction of 8 TB/s and of the measured copy
               ceiling; the same kernel on one set of inputs (cache-warm,
               labelled warm); the unfused variant timed the same way (all its
               launches per call) and the speedups;
  calibration  the library's streaming copy (128-bit loads and stores) of
               256 MiB, rotating over 4 buffer pairs, same protocol: the
               attainable read+write bandwidth;
  roofline     the dominant kernel (largest time per call), its duration from
               HIP events around each of its calls inside the timed region,
               against 8 TB/s;
  cpu_baseline the CPU oracle timed on a bounded sample of the same workloads,
               on every host core available to the process (row chunks in
               parallel threads; the oracle's C code releases the GIL) and on
               one core;
  next         the two-dimensional forms (bf16 chain with a broadcast bias
               row, fp16 10-op graph on padded rows) and the row softmax
               (bf16, attention-probability shape), same batch protocol,
               not part of `value`.
  launch_study launch cost against bytes: each variant (unfused, TVM's
               three groups, fused) of small expressions called eagerly
               through the C ABI, replayed from a graph of one call, and
               replayed from a graph of many calls (GPU time per call with no
               host work in between); one set of buffers (cache-warm).

Other modes (for rocprofv3 counter runs): --only NAME runs just one workload's
fused kernel; --copy-bytes B runs the library's streaming copy of B bytes;
--no-graphs times every batch as eager calls (no graph capture, no launch
study), so that each kernel is an ordinary dispatch; --element-check runs the
fp32 two-dimensional chain on rows one element off 16-byte boundaries (its
element path: 4-byte accesses), whose bytes are known, to check the HBM
counters' scale on a request mix other than the copy's.
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
    p.add_argument("--unfused-reps", type=int, default=20, help="batches for the unfused timing (0: skip)")
    p.add_argument("--batches", type=int, default=20, help="batches per workload for the per-call times")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=2,
                   help="the oracle runs on 1/K of each workload's rows")
    p.add_argument("--only", default=None, help="run only this workload's fused kernel")
    p.add_argument("--no-next", action="store_true", help="skip the two-dimensional forms")
    p.add_argument("--no-floors", action="store_true", help="skip the per-workload bare-stream floors")
    p.add_argument("--no-launch-study", action="store_true", help="skip the eager vs graph study")
    p.add_argument("--no-graphs", action="store_true",
                   help="time the batches as eager calls only (no graph capture; for counter runs)")
    p.add_argument("--unfused-only", default=None, help="run only this workload's unfused variant")
    p.add_argument("--copy-bytes", type=int, default=0, help="run the streaming copy of this size")
    p.add_argument("--element-check", action="store_true",
                   help="run the fp32 chain on rows off 16-byte boundaries (one element per access), "
                        "for checking the HBM counters' scale on that request mix")
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

    if args.element_check:
        # [8192, 4095] fp32 operands in rows of 4096, one element past a
        # 16-byte boundary: the two-dimensional chain takes its element path
        rows, cols, ld = 8192, 4095, 4096
        bufs = [torch.randn(rows * ld + 4, device=dev) for _ in range(4)]
        x, b1, b2, y = (b[1:1 + rows * ld].view(rows, ld)[:, :cols] for b in bufs)
        for _ in range(args.warmup + args.steps):
            mbp.fused_pointwise_chain_2d(x, b1, b2, 0.5, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "element-check", "rows": rows, "cols": cols, "row_stride": ld,
                          "bytes_read_per_call": 3 * rows * cols * 4, "bytes_written_per_call": rows * cols * 4,
                          "launches": args.warmup + args.steps}))
        return

    names = [w.name for w in W.WORKLOADS]
    if args.only:
        names = [args.only]
    if args.unfused_only:
        names = [args.unfused_only]
    wl = [W.BY_NAME[n] for n in names]

    # ---- inputs resident in HBM: B copies per workload (B x working set >= 1 GiB)
    def n_sets(w):
        if args.only or args.unfused_only:
            return 1
        return max(1, min(128, -(-(1 << 30) // w.compulsory_bytes)))

    def build(w, d):
        """(fused call, unfused call) on fresh device copies of the inputs."""
        if w.kind == "chain":
            x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
            y, uy = torch.empty_like(x), torch.empty_like(x)
            s = w.params["scale"]
            return (lambda: mbp.fused_pointwise_chain(x, b1, b2, s, out=y),
                    lambda ws: mbp.unfused_pointwise_chain(x, b1, b2, s, out=uy, workspace=ws))
        if w.kind == "row_mean":
            x, bias, g, b = (to_dev(d[k]) for k in ("x", "bias", "gamma", "beta"))
            y, uy = torch.empty_like(x), torch.empty_like(x)
            al, c = w.params["alpha"], w.params["c"]
            return (lambda: mbp.fused_row_mean_epilogue(x, bias, g, b, al, c, out=y),
                    lambda ws: mbp.unfused_row_mean_epilogue(x, bias, g, b, al, c, out=uy, workspace=ws))
        x, r, g, b = (to_dev(d[k]) for k in ("x", "residual", "gamma", "beta"))
        y, uy = torch.empty_like(x), torch.empty_like(x)
        eps, act = w.params["eps"], w.act
        return (lambda: mbp.fused_add_layernorm_gelu(x, r, g, b, eps, act, out=y),
                lambda ws: mbp.unfused_add_layernorm_gelu(x, r, g, b, eps, act, out=uy, workspace=ws))

    t_gen = time.time()
    host, sets, usets, uinfo = {}, {}, {}, {}
    for w in wl:
        d = W.generate(w)
        host[w.name] = d
        if w.kind == "chain":
            ws_bytes = mbp.workspace_bytes(mbp.OP_CHAIN, mbp.F32, 1, w.n)
            uinfo[w.name] = mbp.launches_per_call(mbp.OP_CHAIN, False)
        elif w.kind == "row_mean":
            ws_bytes = mbp.workspace_bytes(mbp.OP_ROW_MEAN, mbp.F32, w.rows, w.cols)
            uinfo[w.name] = mbp.launches_per_call(mbp.OP_ROW_MEAN, False)
        else:
            has_r = d.get("residual") is not None
            dcode = mbp.BF16 if w.dtype == "bf16" else mbp.F32
            ws_bytes = mbp.workspace_bytes(mbp.OP_LAYERNORM, dcode, w.rows, w.cols, has_r, w.act)
            uinfo[w.name] = mbp.launches_per_call(mbp.OP_LAYERNORM, False, has_residual=has_r, act=w.act)
        # one workspace per workload, shared by its copies (as a caching allocator would)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        pairs = [build(w, d) for _ in range(n_sets(w))]
        sets[w.name] = [f for f, _ in pairs]
        usets[w.name] = [lambda u=u, ws=ws: u(ws) for _, u in pairs]
    calls = {n: sets[n][0] for n in names}
    ucalls = {n: usets[n][0] for n in names}
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    if args.unfused_only:
        for _ in range(args.warmup + args.steps):
            ucalls[names[0]]()
        torch.cuda.synchronize()
        print(json.dumps({"mode": "unfused-only", "workload": names[0], "calls": args.warmup + args.steps}))
        return

    # everything runs on one created stream (graph capture cannot use the
    # NULL stream); the library calls take the current stream
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)

    def batch_times(fns, batches, eager=None):
        """Per-call GPU times (us) of `batches` batches of N back-to-back calls
        rotating over `fns`, each batch replayed from a captured graph between
        two events on the stream; with eager=list, also the eager per-call
        times of the same batches issued from Python, appended to it."""
        for f in fns[:3]:
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(3):
            fns[i % len(fns)]()
        e1.record(stream)
        torch.cuda.synchronize()
        est = e0.elapsed_time(e1) * 1e3 / 3
        n_calls = max(1, min(2000, int(1000.0 / max(est, 1e-3))))

        def events():
            return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(batches)]

        if eager is not None or args.no_graphs:
            ev = events()
            k = 0
            for a, b in ev:
                a.record(stream)
                for _ in range(n_calls):
                    fns[k % len(fns)]()
                    k += 1
                b.record(stream)
            torch.cuda.synchronize()
            times = [a.elapsed_time(b) * 1e3 / n_calls for a, b in ev]
            if args.no_graphs:
                if eager is not None:
                    eager.extend(times)
                return times, n_calls
            eager.extend(times)
        with mbp.capture(stream) as cap:
            for k in range(n_calls):
                fns[k % len(fns)]()
        g = cap.graph
        g.launch(stream)
        ev = events()
        for a, b in ev:
            a.record(stream)
            g.launch(stream)
            b.record(stream)
        torch.cuda.synchronize()
        g.close()
        return [a.elapsed_time(b) * 1e3 / n_calls for a, b in ev], n_calls

    # ---- per-call times, one workload at a time (not the timed region)
    fused_us, fused_n, fused_eager, fused_warm = {}, {}, {}, {}
    for n in names:
        fused_eager[n] = []
        fused_us[n], fused_n[n] = batch_times(sets[n], args.batches, fused_eager[n])
        fused_warm[n], _ = batch_times(sets[n][:1], args.batches)

    # ---- calibration: the attainable copy bandwidth, same protocol
    calibration = None
    if not args.only:
        cb = 256 << 20
        pairs = [(torch.empty(cb // 4, device=dev), torch.empty(cb // 4, device=dev)) for _ in range(4)]
        for a, _ in pairs:
            a.fill_(1.0)
        cus, _ = batch_times([lambda a=a, b=b: mbp.stream_copy(a, b) for a, b in pairs], args.batches)
        cmed = statistics.median(cus)
        calibration = {"kernel": "mbp_stream_copy", "bytes_per_call": 2 * cb,
                       "us_median": round(cmed, 3), "gbps": round(2 * cb / (cmed * 1e-6) / 1e9, 1),
                       "frac_of_peak": round(2 * cb / (cmed * 1e-6) / 1e9 / PEAK_GBPS, 4)}
        del pairs
    # ---- like-for-like floors: the bare stream of each workload's own reads
    # and write (mbp_stream_rw: nsrc inputs, one output, the tensors' sizes, no
    # arithmetic), same rotation over input copies and the same batches
    def floor_spec(w):
        """(tensors read, bytes per tensor) of the workload's streams (the
        per-column vectors, at most 48 KiB, left out)"""
        es = 4 if w.dtype == "f32" else 2
        if w.kind == "chain":
            return 3, 4 * w.n
        if w.kind == "chain2d":
            return 2, es * w.rows * w.cols
        if w.kind in ("layernorm", "layernorm2d"):
            return (2 if w.residual else 1), es * w.rows * w.cols
        return 1, es * w.rows * w.cols       # row_mean, row_mean2d, softmax, ln_relu_dropout

    def copy_floor(w):
        nsrc, nb = floor_spec(w)
        nb = -(-nb // 16) * 16
        sets = [([torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(nsrc)],
                 torch.empty(nb, dtype=torch.uint8, device=dev)) for _ in range(n_sets(w))]
        us, _ = batch_times([lambda s=s, d=d: mbp.stream_rw(s, d) for s, d in sets], args.batches)
        del sets
        return {"copy_floor_us": round(statistics.median(us), 3), "copy_floor_reads": nsrc}

    floors = {}
    if not args.only and not args.no_floors:
        for n in names:
            floors[n] = copy_floor(W.BY_NAME[n])
    dominant = max(names, key=lambda n: statistics.median(fused_us[n]))

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

    # ---- unfused variants, same batch protocol
    unf_us = {n: [] for n in names}
    unf_eager = {n: [] for n in names}
    if args.unfused_reps and not args.only:
        for n in names:
            unf_us[n], _ = batch_times(usets[n], args.unfused_reps, unf_eager[n])

    # ---- the two-dimensional forms (16-bit storage, broadcast rows, row
    # strides) and the row softmax: same batch protocol, reported beside the
    # step, not in `value`
    nxt = {}
    if not args.only and not args.no_next:
        def padded(a, ld):
            """a [rows, cols] view of a device copy of `a` inside rows of ld elements"""
            t = to_dev(a)
            buf = torch.zeros((t.shape[0], ld), dtype=t.dtype, device=dev)
            v = buf[:, :t.shape[1]]
            v.copy_(t)
            return v

        def build_next(w, d):
            if w.kind == "layernorm2d":
                ld = w.params["ld"]
                x, r, y = padded(d["x"], ld), padded(d["residual"], ld), padded(np.zeros_like(d["x"]), ld)
                g, b = to_dev(d["gamma"]), to_dev(d["beta"])
                return lambda: mbp.fused_add_layernorm_gelu(x, r, g, b, w.params["eps"], w.act, out=y)
            if w.kind == "ln_relu_dropout":
                x, g, b = (to_dev(d[k]) for k in ("x", "gamma", "beta"))
                y = torch.empty_like(x)
                pr = w.params
                return lambda: mbp.fused_layernorm_relu_dropout(x, g, b, pr["p"], pr["seed"], pr["offset"],
                                                                pr["eps"], out=y)
            if w.kind == "softmax":
                x = to_dev(d["x"])
                y = torch.empty_like(x)
                return lambda: mbp.fused_softmax(x, out=y)
            if w.kind == "chain2d":
                x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
                y = torch.empty_like(x)
                sc = w.params["scale"]
                return lambda: mbp.fused_pointwise_chain_2d(x, b1, b2, sc, out=y)
            xd = to_dev(d["x"])
            ld = w.params["ld"]
            xb = torch.zeros((w.rows, ld), dtype=xd.dtype, device=dev)
            x = xb[:, :w.cols]
            x.copy_(xd)
            y = torch.empty_like(xb)[:, :w.cols]
            vec = [to_dev(d[k]) for k in ("bias", "gamma", "beta")]
            al, c = w.params["alpha"], w.params["c"]
            return lambda: mbp.fused_row_mean_epilogue_2d(x, *vec, alpha=al, c=c, out=y)

        for w in W.NEXT_WORKLOADS:
            d = W.generate(w)
            fns = [build_next(w, d) for _ in range(n_sets(w))]
            us, ncalls = batch_times(fns, args.batches)
            med = statistics.median(us)
            nxt[w.name] = {"compulsory_bytes": w.compulsory_bytes, "fused_us_median": round(med, 3),
                           "fused_us_min": round(min(us), 3), "calls_per_batch": ncalls,
                           "input_copies": len(fns),
                           "gbps": round(w.compulsory_bytes / (med * 1e-6) / 1e9, 1),
                           "frac_of_peak": round(w.compulsory_bytes / (med * 1e-6) / 1e9 / PEAK_GBPS, 4)}
            del fns
            if not args.no_floors:
                fl = copy_floor(w)
                nxt[w.name].update(fl)
                nxt[w.name]["frac_of_copy_floor"] = round(fl["copy_floor_us"] / med, 4)
            if w.kind == "softmax" and args.unfused_reps:
                # the five eager launches: max, x - m, exp, sum, divide
                x = to_dev(d["x"])
                y = torch.empty_like(x)
                ws = torch.empty(mbp.workspace_bytes(mbp.OP_SOFTMAX, mbp.BF16, w.rows, w.cols),
                                 dtype=torch.uint8, device=dev)
                ufn = lambda: mbp.unfused_softmax(x, out=y, workspace=ws)
                uus, _ = batch_times([ufn], args.unfused_reps)
                um = statistics.median(uus)
                del ufn
                nxt[w.name].update({"unfused_us_median": round(um, 3), "launches_unfused": 5,
                                    "speedup_vs_unfused": round(um / med, 3)})
                del x, y, ws
            if w.kind == "ln_relu_dropout" and args.unfused_reps:
                # the three eager launches of the same expression
                x, g, b = (to_dev(d[k]) for k in ("x", "gamma", "beta"))
                y = torch.empty_like(x)
                ws = torch.empty(mbp.workspace_bytes(mbp.OP_LN_RELU_DROPOUT, mbp.BF16, w.rows, w.cols),
                                 dtype=torch.uint8, device=dev)
                pr = w.params
                ufn = lambda: mbp.unfused_layernorm_relu_dropout(x, g, b, pr["p"], pr["seed"], pr["offset"],
                                                                 pr["eps"], out=y, workspace=ws)
                uus, _ = batch_times([ufn], args.unfused_reps)
                um = statistics.median(uus)
                del ufn
                nxt[w.name].update({"unfused_us_median": round(um, 3), "launches_unfused": 3,
                                    "speedup_vs_unfused": round(um / med, 3)})
                del x, g, b, y, ws
        torch.cuda.synchronize()

    study = None
    if not args.only and not args.no_launch_study and not args.no_graphs:
        study = launch_study(mbp, W, dev, args.batches)

    per = {}
    total_bytes = 0
    for w in wl:
        n = w.name
        B = w.compulsory_bytes
        total_bytes += B
        med_us = statistics.median(fused_us[n])
        srt = sorted(fused_us[n])
        rec = {
            "compulsory_bytes": B,
            "fused_us_median": round(med_us, 3),
            "fused_us_min": round(srt[0], 3),
            "fused_us_p90": round(srt[min(len(srt) - 1, int(0.9 * len(srt)))], 3),
            "eager_us_median": round(statistics.median(fused_eager[n]), 3),
            "calls_per_batch": fused_n[n],
            "input_copies": len(sets[n]),
            "gbps": round(B / (med_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(B / (med_us * 1e-6) / 1e9 / PEAK_GBPS, 4),
            "frac_of_copy": (round(B / (med_us * 1e-6) / 1e9 / calibration["gbps"], 4)
                             if calibration else None),
            "warm_us_median": round(statistics.median(fused_warm[n]), 3),
            "launches_fused": 1,
        }
        if n in floors:
            rec.update(floors[n])
            rec["frac_of_copy_floor"] = round(floors[n]["copy_floor_us"] / med_us, 4)
        if unf_us[n]:
            um = statistics.median(unf_us[n])
            ue = statistics.median(unf_eager[n])
            rec.update({"unfused_us_median": round(um, 3), "launches_unfused": uinfo[n],
                        "speedup_vs_unfused": round(um / med_us, 3),
                        "unfused_eager_us_median": round(ue, 3),
                        "speedup_vs_unfused_eager": round(ue / statistics.median(fused_eager[n]), 3)})
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
        "calibration": calibration,
        "cpu_baseline": cpu,
        "per_workload": per,
        "next": nxt,
        "launch_study": study,
        "library_sha256": sha[:16],
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(out))


def launch_study(mbp, W, dev, batches):
    """Eager launches against graph replay on small expressions, where the
    per-launch cost is comparable to the kernels' own time."""
    import ctypes
    import functools

    import torch

    L = mbp.lib
    side = torch.cuda.Stream(dev)
    sh = side.cuda_stream
    P = lambda t: t.data_ptr()
    to_dev = lambda a: W.to_device(a, dev)

    def ws_for(nbytes):
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    keep = []  # buffers referenced by raw pointers below

    def chain_case(n):
        d = W.generate(W.scaled(W.BY_NAME["chain_4M_f32"], n=n))
        x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
        y = torch.empty_like(x)
        ws = ws_for(mbp.workspace_bytes(mbp.OP_CHAIN, mbp.F32, 1, n))
        keep.extend([x, b1, b2, y, ws])
        a = (P(x), P(b1), P(b2), P(y), n, 0.5)
        return 16 * n, {
            "unfused": (functools.partial(L.unfused_pointwise_chain, *a, P(ws), ws.numel(), sh), 4),
            "fused": (functools.partial(L.fused_pointwise_chain, *a, sh), 1)}

    def tenop_case(rows, cols):
        d = W.generate(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), cols=cols)
        x, bias, g, b = (to_dev(d[k]) for k in ("x", "bias", "gamma", "beta"))
        y = torch.empty_like(x)
        wu = ws_for(mbp.workspace_bytes(mbp.OP_ROW_MEAN, mbp.F32, rows, cols))
        wg = ws_for(mbp.workspace_bytes(mbp.OP_ROW_MEAN, mbp.F32, rows, cols,
                                        granularity=mbp.UNFUSED_GROUPED))
        keep.extend([x, bias, g, b, y, wu, wg])
        a = (P(x), P(bias), P(g), P(b), P(y), rows, cols, 1.1, 0.1)
        return 8 * rows * cols + 12 * cols, {
            "unfused": (functools.partial(L.unfused_row_mean_epilogue, *a, P(wu), wu.numel(), sh), 10),
            "grouped": (functools.partial(L.grouped_row_mean_epilogue, *a, P(wg), wg.numel(), sh), 3),
            "fused": (functools.partial(L.fused_row_mean_epilogue, *a, sh), 1)}

    def addln_case(rows, cols):
        w = W.scaled(W.BY_NAME["addln_gelu_16384x8192_bf16"], rows=rows)
        d = W.generate(w, cols=cols)
        x, r, g, b = (to_dev(d[k]) for k in ("x", "residual", "gamma", "beta"))
        y = torch.empty_like(x)
        wp = ws_for(mbp.workspace_bytes(mbp.OP_LAYERNORM, mbp.BF16, rows, cols, True, "gelu_tanh"))
        we = ws_for(mbp.workspace_bytes(mbp.OP_LAYERNORM, mbp.BF16, rows, cols, True, "gelu_tanh",
                                        mbp.UNFUSED_EAGER))
        keep.extend([x, r, g, b, y, wp, we])
        a = (mbp.BF16, P(x), P(r), P(g), P(b), P(y), rows, cols, 1e-5, mbp.ACT_GELU_TANH)
        return 6 * rows * cols + 4 * cols, {
            "unfused": (functools.partial(L.unfused_add_layernorm_gelu, *a, mbp.UNFUSED_PRIMITIVE, P(wp),
                                          wp.numel(), sh), 7),
            "eager_ln": (functools.partial(L.unfused_add_layernorm_gelu, *a, mbp.UNFUSED_EAGER, P(we),
                                           we.numel(), sh), 3),
            "fused": (functools.partial(L.fused_add_layernorm_gelu, *a, sh), 1)}

    def lnrd_case(rows, cols):
        w = W.scaled(W.BY_NAME["addln_gelu_16384x8192_bf16"], rows=rows)
        d = W.generate(w, cols=cols)
        x, g, b = (to_dev(d[k]) for k in ("x", "gamma", "beta"))
        y = torch.empty_like(x)
        ws = ws_for(mbp.workspace_bytes(mbp.OP_LN_RELU_DROPOUT, mbp.BF16, rows, cols))
        keep.extend([x, g, b, y, ws])
        a = (mbp.BF16, P(x), P(g), P(b), P(y), rows, cols, 1e-5, 0.1, 0x5EED, 0)
        return 4 * rows * cols + 4 * cols, {
            "unfused": (functools.partial(L.unfused_layernorm_relu_dropout, *a, P(ws), ws.numel(), sh), 3),
            "fused": (functools.partial(L.fused_layernorm_relu_dropout, *a, sh), 1)}

    cases = {
        "chain_4M_f32": chain_case(4 * 1024 * 1024),
        "chain_64K_f32": chain_case(64 * 1024),
        "tenop_1024x1024_f32": tenop_case(1024, 1024),
        "tenop_8x1024_f32": tenop_case(8, 1024),
        "addln_gelu_16x768_bf16": addln_case(16, 768),
        "ln_relu_dropout_16x768_bf16": lnrd_case(16, 768),
    }

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {mbp.STATUS_NAMES.get(st, st)}: {L.mbp_last_error().decode()}")

    def capture(fn, m):
        check(L.mbp_graph_capture_begin(sh), "capture begin")
        for _ in range(m):
            check(fn(), "captured call")
        h = ctypes.c_void_p()
        check(L.mbp_graph_capture_end(sh, ctypes.byref(h)), "capture end")
        return h

    def timed(fn, calls_per_fn):
        """Median GPU us per call and host us per call over `batches` batches."""
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        for _ in range(3):
            fn()
        e1.record(side)
        side.synchronize()
        est = e0.elapsed_time(e1) * 1e3 / 3
        n = max(1, min(5000, int(1000.0 / max(est, 1e-3))))
        gpu, host = [], []
        for _ in range(batches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(side)
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            t1 = time.perf_counter()
            b.record(side)
            side.synchronize()
            gpu.append(a.elapsed_time(b) * 1e3 / (n * calls_per_fn))
            host.append((t1 - t0) * 1e6 / (n * calls_per_fn))
        return round(statistics.median(gpu), 3), round(statistics.median(host), 3)

    out = {}
    torch.cuda.synchronize()
    for cname, (nbytes, variants) in cases.items():
        rec = {"compulsory_bytes": nbytes}
        for vname, (fn, launches) in variants.items():
            check(fn(), f"{cname} {vname}")
            side.synchronize()
            eager_gpu, eager_host = timed(fn, 1)
            g1 = capture(fn, 1)
            nodes = L.mbp_graph_nodes(g1)
            g1_gpu, g1_host = timed(functools.partial(L.mbp_graph_launch, g1, sh), 1)
            m = max(1, 400 // launches)
            gm = capture(fn, m)
            gm_gpu, _ = timed(functools.partial(L.mbp_graph_launch, gm, sh), m)
            side.synchronize()
            check(L.mbp_graph_destroy(g1), "destroy")
            check(L.mbp_graph_destroy(gm), "destroy")
            rec[vname] = {"launches": launches, "graph_nodes": nodes,
                          "eager_us": eager_gpu, "eager_host_us": eager_host,
                          "graph1_us": g1_gpu, "graph1_host_us": g1_host,
                          "graph_batch_us": gm_gpu, "graph_batch_calls": m,
                          "graph_batch_gbps": round(nbytes / (gm_gpu * 1e-6) / 1e9, 1)}
        out[cname] = rec
    torch.cuda.synchronize()
    del keep
    return out


def cpu_baseline(wl, host, frac):
    """The oracle (plain C, binary64) on the first 1/frac of each workload's
    rows (elements for the chain); GB/s on the same compulsory bytes.  Timed
    twice: the rows split into chunks run by one thread per available core
    (the oracle is called unchanged on each chunk), then on one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import workloads as W

    cores = max(1, min(16, len(os.sched_getaffinity(0))))

    def jobs(w):
        """(compulsory bytes, list of zero-argument calls covering the sample)."""
        d = host[w.name]
        if w.kind == "chain":
            n = w.n // frac
            cuts = [n * i // cores for i in range(cores + 1)]
            sc = w.params["scale"]
            return W.scaled(w, n=n).compulsory_bytes, [
                (lambda a=a, b=b: oracle.pointwise_chain(d["x"][a:b], d["b1"][a:b], d["b2"][a:b], sc))
                for a, b in zip(cuts, cuts[1:]) if b > a]
        rows = max(1, w.rows // frac)
        cuts = [rows * i // cores for i in range(cores + 1)]
        spans = [(a, b) for a, b in zip(cuts, cuts[1:]) if b > a]
        if w.kind == "row_mean":
            al, c = w.params["alpha"], w.params["c"]
            calls = [(lambda a=a, b=b: oracle.row_mean_epilogue(d["x"][a:b], d["bias"], d["gamma"], d["beta"],
                                                                al, c)) for a, b in spans]
        else:
            act = oracle.ACT_GELU_TANH if w.act == "gelu_tanh" else oracle.ACT_NONE
            eps = w.params["eps"]
            r = d["residual"]
            calls = [(lambda a=a, b=b: oracle.add_layernorm_gelu(d["x"][a:b], None if r is None else r[a:b],
                                                                 d["gamma"], d["beta"], eps, act))
                     for a, b in spans]
        return W.scaled(w, rows=rows).compulsory_bytes, calls

    t_par = t_one = 0.0
    b_total = 0
    with ThreadPoolExecutor(cores) as ex:
        for w in wl:
            nbytes, calls = jobs(w)
            b_total += nbytes
            t = time.perf_counter()
            list(ex.map(lambda f: f(), calls))
            t_par += time.perf_counter() - t
    for w in wl:
        _, calls = jobs(w)
        t = time.perf_counter()
        for f in calls:
            f()
        t_one += time.perf_counter() - t
    return {"value": round(b_total / t_par / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "single_core_value": round(b_total / t_one / 1e9, 3),
            "sample": f"first 1/{frac} of the rows (elements) of each of the {len(wl)} workloads, "
                      f"{b_total} compulsory bytes, binary64; {t_par:.1f} s on {cores} threads "
                      f"(row chunks), {t_one:.1f} s on one thread"}


if __name__ == "__main__":
    main()
