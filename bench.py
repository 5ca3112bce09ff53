#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 GEMM on one MI355X.

A step is one pass over the workload: every GEMM shape of the chosen family
run once, back to back, on one stream (default: the dense prefill sweep,
M = 4096 x six (N, K) shapes).  Inputs are synthetic, seeded, and resident in
HBM before timing starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--family F] [--eager] [--no-cpu-baseline]

The K timed steps are captured in one HIP graph and replayed once (--eager: launched
one by one from Python, which also times the host's per-call overhead); each shape's
launch times come from an event pair around every launch of a second pass of K steps,
enqueued while the stream is held so that the kernels then run back to back.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 TFLOP/s and % of MI355X FP8 MFMA peak (HBM GB/s for small M), 1 GPU"
PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E, published
KERNEL_SOURCES = ["moe_grouped_gemm_block_amd/csrc/fp8bs_gemm.hip",
                  "moe_grouped_gemm_block_amd/csrc/fp8bs_instances.inc"]
FAMILY_NAMES = {
    0: "dense M=128 N=2112 K=7168",
    1: "dense prefill sweep M=4096, (N,K) in {(2112,7168),(24576,1536),(32768,512),"
       "(7168,16384),(4096,7168),(7168,2048)}",
    2: "dense decode sweep M in {64,128,256} x (N,K) in {(7168,7168),(7168,2048),(4096,7168)}",
    3: "MoE contiguous G=8, multinomial rows ~32768, (N,K) in {(4096,7168),(7168,2048)}",
    4: "MoE masked G=16, max_m=256, masked_m~U{1..256}, (N,K) in {(4096,7168),(7168,2048)}",
    5: "MoE K-grouped weight gradients G=8, tokens ~ Multinomial(32768) padded to 128 per "
       "group, (M,N) in {(4096,7168),(7168,2048)}, FP32 D",
    6: "dense stored forms nn, tn, tt at M=4096 N=4096 K=7168",
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic(name: str):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE + WRITE_SIZE, scaled
    by a plain copy kernel) for this kernel source; None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    if data.get("source_sha256") != kernel_source_hash():
        return None
    entry = data.get("shapes", {}).get(name)
    return None if entry is None else entry.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--family", type=int, default=1, choices=sorted(FAMILY_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", default="",
                    help="run only this shape (3 launches) and a 512 MiB device copy (3 launches), "
                         "for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two rocprofv3 --pmc output directories of a traffic probe into "
                         "profiles/traffic.json")
    ap.add_argument("--summarize-trace", default="",
                    help="per-shape average kernel durations from a rocprofv3 --kernel-trace output "
                         "directory of a bench.py run (dispatches attributed in launch order)")
    ap.add_argument("--cpu-rows", type=int, default=1536,
                    help="rows of D per shape the oracle computes for the CPU baseline")
    ap.add_argument("--per-shape-out", default="", help="also write per-shape results here")
    ap.add_argument("--eager", action="store_true",
                    help="launch the K timed steps one call at a time from Python instead of "
                         "replaying them as one captured graph")
    ap.add_argument("--graph", action="store_true", help="(the default; kept for old command lines)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.family)
        return
    if args.ingest_traffic:
        if not args.traffic_probe:
            raise SystemExit("--ingest-traffic needs --traffic-probe NAME (the probed shape)")
        ingest_traffic(args.ingest_traffic[0], args.ingest_traffic[1], args.traffic_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); there is "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_grouped_gemm_block_amd as fp8bs
    from moe_grouped_gemm_block_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fp8bs._load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM ----
    t0 = time.time()
    problems = []
    for desc in synth.workload_shapes(args.family):
        p = synth.make(desc)
        if p.kind == "k_grouped":
            ws = torch.empty(max(fp8bs.workspace_size(fp8bs.LAYOUT_K_GROUPED, p.M, p.N, p.K, p.G),
                                 16), dtype=torch.uint8, device=dev)
            problems.append(dict(
                desc=desc, p=p, a=torch.from_numpy(p.A).to(dev),
                sfa=fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).to(dev),
                b=torch.from_numpy(p.B).to(dev),
                sfb=fp8bs.sfa_mn_major(torch.from_numpy(p.SB)).to(dev),
                d=torch.empty((p.G, p.M, p.N), dtype=torch.float32, device=dev),
                extra=[int(x) for x in p.ks], ws=ws))
            continue
        form = desc.get("form", "nt")
        if form != "nt":
            A_st, B_st = synth.stored_operands(p, form)
            code = {"nn": fp8bs.LAYOUT_DENSE_NN, "tn": fp8bs.LAYOUT_DENSE_TN,
                    "tt": fp8bs.LAYOUT_DENSE_TT}[form]
            ws = torch.empty(max(fp8bs.workspace_size(code, p.M, p.N, p.K), 16),
                             dtype=torch.uint8, device=dev)
            problems.append(dict(
                desc=desc, p=p, a=torch.from_numpy(A_st).to(dev),
                sfa=fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).to(dev),
                b=torch.from_numpy(B_st).to(dev),
                sfb=torch.from_numpy(np.ascontiguousarray(p.SB[0])).to(dev),
                d=torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev), extra=form, ws=ws))
            continue
        a = torch.from_numpy(p.A).to(dev)
        sfa = fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).to(dev)
        b = torch.from_numpy(np.ascontiguousarray(p.B if p.kind != "dense" else p.B[0])).to(dev)
        sfb = torch.from_numpy(np.ascontiguousarray(p.SB if p.kind != "dense" else p.SB[0])).to(dev)
        if p.kind == "masked":
            d = torch.empty((p.G, p.max_m, p.N), dtype=torch.bfloat16, device=dev)
        else:
            d = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
        extra = None
        if p.kind == "contiguous":
            extra = torch.from_numpy(p.layout).to(dev)
        elif p.kind == "masked":
            extra = torch.from_numpy(p.masked_m).to(dev)
        # split-K workspace, allocated once per shape outside the timed region
        layout = {"dense": fp8bs.LAYOUT_DENSE, "contiguous": fp8bs.LAYOUT_CONTIGUOUS,
                  "masked": fp8bs.LAYOUT_MASKED}[p.kind]
        wsz = fp8bs.workspace_size(layout, p.max_m if p.kind == "masked" else p.M, p.N, p.K, p.G,
                                   p.expected_m if p.kind == "masked" else 0)
        ws = torch.empty(max(wsz, 16), dtype=torch.uint8, device=dev)
        problems.append(dict(desc=desc, p=p, a=a, sfa=sfa, b=b, sfb=sfb, d=d, extra=extra, ws=ws))
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    def launch(q):
        p = q["p"]
        if p.kind == "k_grouped":
            fp8bs.fp8bs_k_grouped_tn_contiguous(q["a"], q["sfa"], q["b"], q["sfb"], q["d"],
                                                q["extra"], workspace=q["ws"])
        elif isinstance(q["extra"], str):
            getattr(fp8bs, "fp8bs_dense_" + q["extra"])(q["a"], q["sfa"], q["b"], q["sfb"], q["d"],
                                                        workspace=q["ws"])
        elif p.kind == "dense":
            fp8bs.fp8bs_dense_nt_ws(q["a"], q["sfa"], q["b"], q["sfb"], q["d"], workspace=q["ws"])
        elif p.kind == "contiguous":
            fp8bs.fp8bs_grouped_contiguous_nt_ws(q["a"], q["sfa"], q["b"], q["sfb"], q["d"],
                                                 q["extra"], workspace=q["ws"])
        else:
            fp8bs.fp8bs_grouped_masked_nt_ws(q["a"], q["sfa"], q["b"], q["sfb"], q["d"], q["extra"],
                                             expected_m=p.expected_m, workspace=q["ws"])

    if args.traffic_probe:
        sel = [q for q in problems if q["desc"]["name"] == args.traffic_probe]
        if not sel:
            raise SystemExit(f"no shape {args.traffic_probe} in family {args.family}")
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            launch(sel[0])
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": args.traffic_probe, "copy_bytes": COPY_PROBE_BYTES}))
        return

    for _ in range(args.warmup):
        for q in problems:
            launch(q)
    torch.cuda.synchronize()

    # ---- timed region: K steps; events around every launch on the launch stream ----
    stream = torch.cuda.current_stream(dev)
    step_start = torch.cuda.Event(enable_timing=True)
    step_end = torch.cuda.Event(enable_timing=True)
    def eager_steps(queue_ahead):
        """K steps launched one by one, an event pair around every launch; returns the
        per-launch times (ms) per shape and the wall time.  queue_ahead: hold the stream in
        a spin kernel (not timed) while the host enqueues everything, so that the launches
        then run back to back and each event pair brackets its kernel alone rather than
        also the host's time to issue it."""
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in problems] for _ in range(args.steps)]
        torch.cuda.synchronize()
        sleep = getattr(torch.cuda, "_sleep", None)     # torch's spin kernel
        if queue_ahead and sleep is not None:
            # ~60 us of host time per launch, at a 2.4 GHz shader clock
            sleep(int(60e-6 * 2.4e9 * args.steps * len(problems)))
        w0 = time.perf_counter()
        step_start.record(stream)
        for s_ in range(args.steps):
            for i, q in enumerate(problems):
                ev[s_][i][0].record(stream)
                launch(q)
                ev[s_][i][1].record(stream)
        step_end.record(stream)
        torch.cuda.synchronize()
        w = time.perf_counter() - w0
        return [[ev[s_][i][0].elapsed_time(ev[s_][i][1]) for s_ in range(args.steps)]
                for i in range(len(problems))], w

    if not args.eager:
        # The K timed steps are captured as one graph (K back-to-back steps) and replayed
        # once, so the host's per-call overhead is not timed.  Events cannot be recorded
        # inside a captured graph here, so per-launch times come from a second pass of K
        # steps launched one by one with an event pair around every launch.
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for q in problems:
                launch(q)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph):
            for _ in range(args.steps):
                for q in problems:
                    launch(q)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            for q in problems:
                launch(q)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        step_start.record(stream)
        step_graph.replay()
        step_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = step_start.elapsed_time(step_end)
        shape_ms, _ = eager_steps(queue_ahead=True)
    else:
        shape_ms, wall = eager_steps(queue_ahead=False)
        total_ms = step_start.elapsed_time(step_end)
    ms_per_step = total_ms / args.steps

    flops_step = sum(q["p"].flops() for q in problems)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    per_shape = []
    for i, q in enumerate(problems):
        p = q["p"]
        times = sorted(shape_ms[i])
        avg_ms = sum(times) / len(times)
        med_ms = times[len(times) // 2]
        tflops = p.flops() / (avg_ms * 1e-3) / 1e12
        gbs = p.algorithmic_bytes() / (avg_ms * 1e-3) / 1e9
        t_mfma = p.flops() / (PEAK_FP8_TFLOPS * 1e12)
        t_hbm = p.algorithmic_bytes() / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        if p.kind == "k_grouped":
            plan = fp8bs.describe_config(fp8bs.LAYOUT_K_GROUPED, p.M, p.N, p.K, p.G, 0)
        elif isinstance(q["extra"], str):
            plan = fp8bs.describe_config({"nn": fp8bs.LAYOUT_DENSE_NN, "tn": fp8bs.LAYOUT_DENSE_TN,
                                          "tt": fp8bs.LAYOUT_DENSE_TT}[q["extra"]], p.M, p.N, p.K)
        else:
            plan = fp8bs.describe_config({"dense": 0, "contiguous": 1, "masked": 2}[p.kind],
                                         p.max_m if p.kind == "masked" else p.M, p.N, p.K, p.G,
                                         p.expected_m)
        per_shape.append(dict(
            name=q["desc"]["name"], kind=p.kind, M=p.M, N=p.N, K=p.K, G=p.G,
            valid_rows=p.M if p.kind == "k_grouped" else p.valid_rows, gflop=p.flops() / 1e9, mbytes=p.algorithmic_bytes() / 1e6,
            avg_us=avg_ms * 1e3, median_us=med_ms * 1e3, p10_us=times[len(times) // 10] * 1e3,
            p90_us=times[(9 * len(times)) // 10] * 1e3, tflops=tflops, gbs=gbs, bound=bound,
            roofline_frac=max(t_mfma, t_hbm) / (avg_ms * 1e-3), plan=plan))

    dom = max(range(len(problems)), key=lambda i: per_shape[i]["avg_us"])
    d = per_shape[dom]
    if d["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": d["tflops"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": d["tflops"] / PEAK_FP8_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": d["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": d["gbs"] / PEAK_HBM_GBS}
    roof["traffic"] = load_traffic(d["name"])
    roof["kernel"] = d["name"]
    roof["algorithmic_per_launch"] = {"gflop": d["gflop"], "mbytes": d["mbytes"]}
    roof["avg_launch_us"] = d["avg_us"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(problems, args.cpu_rows)

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": FAMILY_NAMES[args.family], "family": args.family,
                   "shapes": [q["desc"]["name"] for q in problems],
                   "gflop_per_step": flops_step / 1e9,
                   "timing": ("step: one graph of K steps, replayed once; per launch: event "
                              "pairs around each launch in a second pass of K steps, enqueued "
                              "behind a spin kernel so that they run back to back"
                              if not args.eager else "eager launches")},
        "roofline": roof, "cpu_baseline": cpu,
        "per_shape": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()}
                      for s in per_shape],
        "wall_s": round(wall, 4), "input_gen_s": round(gen_s, 2),
        "device": torch.cuda.get_device_name(dev),
    }
    if args.per_shape_out:
        with open(args.per_shape_out, "w") as fh:
            json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


COPY_PROBE_BYTES = 512 << 20


def _pmc_per_dispatch(d, counter):
    """{kernel name: [per-dispatch counter value summed over dimensions]} from a rocprofv3
    --pmc csv output directory."""
    import csv
    import glob
    import collections
    vals = collections.defaultdict(float)
    names = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            vals[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key in sorted(vals, key=lambda k: int(k[0])):
        out[names[key]].append(vals[key])
    return out


def ingest_traffic(fetch_dir, write_dir, name):
    """profiles/traffic.json: HBM bytes per launch of the GEMM kernel in a traffic probe,
    FETCH_SIZE and WRITE_SIZE (KiB) scaled so that the plain copy of COPY_PROBE_BYTES
    reads and writes exactly that many bytes."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    def pick(tab, pred):
        ks = [k for k in tab if pred(k)]
        if len(ks) != 1:
            raise SystemExit(f"expected one matching kernel, found {ks}")
        return ks[0], tab[ks[0]]
    gk, gf = pick(fetch, lambda k: "fp8bs_gemm_kernel" in k)
    ck, cf = pick(fetch, lambda k: "fp8bs" not in k and "copy" in k.lower())
    _, gw = pick(write, lambda k: "fp8bs_gemm_kernel" in k)
    _, cw = pick(write, lambda k: "fp8bs" not in k and "copy" in k.lower())
    # the copy kernel also moved the (small) inputs to the device: keep the three largest
    # dispatches, the COPY_PROBE_BYTES copies
    cf, cw = sorted(cf)[-3:], sorted(cw)[-3:]
    med = lambda v: sorted(v)[len(v) // 2]
    fscale = COPY_PROBE_BYTES / (med(cf) * 1024.0)
    wscale = COPY_PROBE_BYTES / (med(cw) * 1024.0)
    fetch_b = med(gf) * 1024.0 * fscale
    write_b = med(gw) * 1024.0 * wscale
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    if data.get("source_sha256") != kernel_source_hash():
        data = {"source_sha256": kernel_source_hash(), "shapes": {}}
    data["shapes"][name] = {"kernel": gk, "fetch_bytes": fetch_b, "write_bytes": write_b,
                            "bytes_per_launch": fetch_b + write_b,
                            "copy_kernel": ck, "fetch_scale": fscale, "write_scale": wscale}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    json.dump(data, open(path, "w"), indent=1)
    print(json.dumps(data["shapes"][name]))


def summarize_trace(d, family):
    """Average duration per workload shape from a kernel trace of `bench.py --family F`.
    Each call is one GEMM dispatch (staged or B-streaming kernel), followed by a split-K
    reduction when its plan splits K; the calls cycle through the family's shapes in
    order, so a GEMM dispatch starts the next shape and a reduction belongs to the GEMM
    before it."""
    import csv
    import glob
    from moe_grouped_gemm_block_amd import synth
    names = [x["name"] for x in synth.workload_shapes(family)]
    kinds = ("fp8bs_gemm_kernel", "fp8bs_stream_kernel", "fp8bs_splitk_reduce")
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        rows += [r for r in csv.DictReader(open(path))
                 if any(k in r["Kernel_Name"] for k in kinds)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    gemm = {n: [] for n in names}
    red = {n: [] for n in names}
    call = -1
    for r in rows:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "fp8bs_splitk_reduce" in r["Kernel_Name"]:
            if call >= 0:
                red[names[call % len(names)]].append(us)
        else:
            call += 1
            gemm[names[call % len(names)]].append(us)
    out = {}
    for n in names:
        v, w = gemm[n], red[n]
        avg = sum(v) / max(1, len(v))
        ravg = sum(w) / len(w) if w else 0.0
        out[n] = {"dispatches": len(v), "avg_us": avg,
                  "min_us": min(v) if v else None, "max_us": max(v) if v else None,
                  "reduce_dispatches": len(w), "reduce_avg_us": ravg,
                  "call_avg_us": avg + (ravg * len(w) / len(v) if v else 0.0)}
    print(json.dumps(out, indent=1))


def cpu_baseline(problems, rows_per_shape: int):
    """The oracle, untuned, on the host cores: the first `rows_per_shape` valid rows of D
    (all N columns) of every shape of the step, timed; reported in TFLOP/s."""
    import numpy as np

    import oracle
    from moe_grouped_gemm_block_amd import synth  # noqa: F401  (inputs already drawn)

    flop = 0.0
    t = 0.0
    sample = f"first {rows_per_shape} valid rows of D (all columns) of each shape in the step"
    for q in problems:
        p = q["p"]
        if p.kind == "k_grouped":
            # the first R features of A (all N columns, every group): the oracle on that
            # slice of the operands
            R = max(1, rows_per_shape // 64)
            sample = (f"the first {R} rows (all columns, every group) of each K-grouped "
                      f"shape's D")
            A_s = np.ascontiguousarray(p.A[:, :R])
            SA_s = np.ascontiguousarray(p.SA[:R])
            t0 = time.perf_counter()
            oracle.k_grouped(A_s, SA_s, p.B, p.SB, p.ks)
            t += time.perf_counter() - t0
            flop += 2.0 * R * p.N * p.K
            continue
        valid = np.nonzero(_valid_rows(p))[0][:rows_per_shape]
        rows = np.repeat(valid, p.N)
        cols = np.tile(np.arange(p.N), valid.size)
        grp = _row_groups(p)[rows]
        B = p.B if p.kind != "dense" else p.B[0]
        SB = p.SB if p.kind != "dense" else p.SB[0]
        t0 = time.perf_counter()
        oracle.points(p.A.reshape(-1, p.K), p.SA.reshape(-1, p.K // 128), B, SB, rows, grp, cols)
        t += time.perf_counter() - t0
        flop += 2.0 * rows.size * p.K
    return {"value": flop / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(t, 3),
            "sample": f"{sample}, {flop / 1e9:.1f} GFLOP"}


def _valid_rows(p):
    import numpy as np
    if p.kind == "dense":
        return np.ones(p.M, bool)
    if p.kind == "contiguous":
        return (p.layout >= 0) & (p.layout < p.G)
    v = np.clip(p.masked_m, 0, p.max_m)
    return (np.arange(p.max_m)[None, :] < v[:, None]).reshape(-1)


def _row_groups(p):
    import numpy as np
    if p.kind == "dense":
        return np.zeros(p.M, np.int64)
    if p.kind == "contiguous":
        g = p.layout.astype(np.int64)
        g[g < 0] = 0
        return g
    return np.repeat(np.arange(p.G), p.max_m)


if __name__ == "__main__":
    main()
