#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 GEMM on one MI355X.

A step is one pass over a workload family: every GEMM shape of the family run once.  The
headline family (default 3: the MoE contiguous layout, G = 8 experts, about 33k rows, two
(N, K) shapes) gives the JSON line's value and roofline; the other families (default
0, 1, 2, 4) are measured the same way, with fewer steps, and reported under "families".
Inputs are synthetic, seeded, and resident in HBM before timing starts.  Prints one JSON
line.

    python bench.py [--steps K] [--warmup W] [--family F] [--families 0,1,2,4|none]
                    [--flush-mib 512] [--warm] [--no-cpu-baseline]

Timing (cold, the default): before every timed GEMM launch a fill kernel writes
--flush-mib MiB (twice the 256 MB last-level cache), outside the event pair that times
the launch, so that the GEMM's operands come from HBM; the launches and flushes of the K
steps are enqueued behind a spin kernel so that they then run back to back.  The step time
is the sum over the family's shapes of their mean launch time.  The headline family is
also timed warm: the K steps (no flush) captured in one HIP graph and replayed once.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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
DEFAULT_FAMILY = 3
DEFAULT_OTHERS = "0,1,2,4"
OTHER_STEPS = 10                  # timed steps of each non-headline family (at most --steps)
CPU_SAMPLE_GFLOP = 1000.0         # oracle work of the CPU baseline (about 13 s on 16 cores)
COPY_PROBE_BYTES = 512 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_entry(fname: str, name: str):
    """The record for shape `name` in profiles/<fname>, when it was taken on this kernel
    source; None when absent, unreadable or stale."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    if data.get("source_sha256") != kernel_source_hash():
        return None
    return data.get("shapes", {}).get(name)


def load_traffic(name: str):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE + WRITE_SIZE, scaled
    by a plain copy kernel) for this kernel source; None when absent or stale."""
    entry = _profile_entry("traffic.json", name)
    return None if entry is None else entry.get("bytes_per_launch")


def load_mfma_busy(name: str):
    """MFMA busy fraction and shader clock of the kernel from rocprofv3 --pmc
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE) for this kernel source; None when
    absent or stale."""
    entry = _profile_entry("mfma.json", name)
    if entry is None:
        return None
    return {"busy_frac": entry.get("mfma_busy_frac"), "sclk_ghz": entry.get("sclk_ghz")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def parse_families(text: str, headline: int):
    if text.strip().lower() in ("", "none"):
        return []
    out = []
    for tok in text.split(","):
        f = int(tok)
        if f not in FAMILY_NAMES:
            raise SystemExit(f"unknown family {f}")
        if f != headline and f not in out:
            out.append(f)
    return out


def input_sha256(p) -> str:
    """SHA-256 of the generated input bytes of one problem (operands, scales, group data)."""
    import numpy as np
    h = hashlib.sha256()
    arrs = [p.A, p.SA, p.B, p.SB]
    if getattr(p, "layout", None) is not None:
        arrs.append(p.layout)
    if getattr(p, "masked_m", None) is not None:
        arrs.append(p.masked_m)
    if getattr(p, "ks", None) is not None:
        arrs.append(np.asarray(p.ks, dtype=np.int64))
    for a in arrs:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ---- problems on the device --------------------------------------------------------

def build_problems(family: int, dev):
    import numpy as np
    import torch

    import moe_grouped_gemm_block_amd as fp8bs
    from moe_grouped_gemm_block_amd import synth

    problems = []
    for desc in synth.workload_shapes(family):
        p = synth.make(desc)
        sha = input_sha256(p)
        if p.kind == "k_grouped":
            ws = torch.empty(max(fp8bs.workspace_size(fp8bs.LAYOUT_K_GROUPED, p.M, p.N, p.K, p.G),
                                 16), dtype=torch.uint8, device=dev)
            problems.append(dict(
                desc=desc, p=p, sha=sha, a=torch.from_numpy(p.A).to(dev),
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
                desc=desc, p=p, sha=sha, a=torch.from_numpy(A_st).to(dev),
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
        problems.append(dict(desc=desc, p=p, sha=sha, a=a, sfa=sfa, b=b, sfb=sfb, d=d,
                             extra=extra, ws=ws))
    torch.cuda.synchronize()
    return problems


def launch(q):
    import moe_grouped_gemm_block_amd as fp8bs
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


def plan_text(q):
    import moe_grouped_gemm_block_amd as fp8bs
    p = q["p"]
    if p.kind == "k_grouped":
        return fp8bs.describe_config(fp8bs.LAYOUT_K_GROUPED, p.M, p.N, p.K, p.G, 0)
    if isinstance(q["extra"], str):
        return fp8bs.describe_config({"nn": fp8bs.LAYOUT_DENSE_NN, "tn": fp8bs.LAYOUT_DENSE_TN,
                                      "tt": fp8bs.LAYOUT_DENSE_TT}[q["extra"]], p.M, p.N, p.K)
    return fp8bs.describe_config({"dense": 0, "contiguous": 1, "masked": 2}[p.kind],
                                 p.max_m if p.kind == "masked" else p.M, p.N, p.K, p.G,
                                 p.expected_m)


def timed_launches(problems, steps, flush, stream):
    """K steps launched one call at a time with an event pair around every GEMM launch (on
    the launch stream) and, when `flush` is a tensor, a fill of it before each launch,
    outside the pair.  Everything is enqueued while the stream is held by a spin kernel, so
    that the GPU then runs it back to back and each pair brackets its kernel alone.
    Returns the per-launch times (ms) per shape and the wall time of the K steps between
    two synchronizations."""
    import torch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in problems] for _ in range(steps)]
    torch.cuda.synchronize()
    sleep = getattr(torch.cuda, "_sleep", None)          # torch's spin kernel
    if sleep is not None:
        # ~80 us of host time per launch (and flush), at a 2.4 GHz shader clock
        sleep(int(80e-6 * 2.4e9 * steps * len(problems)))
    w0 = time.perf_counter()
    for s_ in range(steps):
        for i, q in enumerate(problems):
            if flush is not None:
                flush.fill_(s_ * len(problems) + i)
            ev[s_][i][0].record(stream)
            launch(q)
            ev[s_][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return [[ev[s_][i][0].elapsed_time(ev[s_][i][1]) for s_ in range(steps)]
            for i in range(len(problems))], wall


def graph_replay_ms(problems, steps, warmup, stream, dev):
    """Warm step time: the K steps captured in one HIP graph and replayed once."""
    import torch
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for q in problems:
            launch(q)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            for q in problems:
                launch(q)
    torch.cuda.synchronize()
    for _ in range(warmup):
        for q in problems:
            launch(q)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return ms


def shape_stats(q, times_ms):
    p = q["p"]
    times = sorted(times_ms)
    avg_ms = sum(times) / len(times)
    med_ms = times[len(times) // 2]
    t_mfma = p.flops() / (PEAK_FP8_TFLOPS * 1e12)
    t_hbm = p.algorithmic_bytes() / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    valid = p.M if p.kind == "k_grouped" else p.valid_rows
    return dict(
        name=q["desc"]["name"], kind=p.kind, M=p.M, N=p.N, K=p.K, G=p.G, valid_rows=valid,
        gflop=p.flops() / 1e9, mbytes=p.algorithmic_bytes() / 1e6, avg_us=avg_ms * 1e3,
        median_us=med_ms * 1e3, p10_us=times[len(times) // 10] * 1e3,
        p90_us=times[(9 * len(times)) // 10] * 1e3, tflops=p.flops() / (avg_ms * 1e-3) / 1e12,
        gbs=p.algorithmic_bytes() / (avg_ms * 1e-3) / 1e9, bound=bound,
        roofline_frac=max(t_mfma, t_hbm) / (avg_ms * 1e-3), plan=plan_text(q),
        input_sha256=q["sha"])


def roofline_of(d):
    if d["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": d["tflops"], "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": d["tflops"] / PEAK_FP8_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": d["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": d["gbs"] / PEAK_HBM_GBS}
    roof["traffic"] = load_traffic(d["name"])
    roof["mfma_busy"] = load_mfma_busy(d["name"])
    roof["kernel"] = d["name"]
    roof["algorithmic_per_launch"] = {"gflop": d["gflop"], "mbytes": d["mbytes"]}
    roof["avg_launch_us"] = d["avg_us"]
    return roof


def measure_family(family, steps, warmup, flush, stream, dev, cpu_gflop=0.0, warm=True):
    """Builds the family's problems, warms up, times K cold steps (and the warm graph
    replay); returns the summary dict (the device buffers are released with it)."""
    import torch
    t0 = time.time()
    print(f"[bench] family {family}: generating inputs", file=sys.stderr, flush=True)
    problems = build_problems(family, dev)
    gen_s = time.time() - t0
    print(f"[bench] family {family}: inputs ready ({gen_s:.1f} s), timing", file=sys.stderr,
          flush=True)
    for _ in range(warmup):
        for q in problems:
            if flush is not None:
                flush.fill_(0)
            launch(q)
    torch.cuda.synchronize()
    shape_ms, wall = timed_launches(problems, steps, flush, stream)
    per_shape = [shape_stats(q, shape_ms[i]) for i, q in enumerate(problems)]
    step_ms = sum(s["avg_us"] for s in per_shape) / 1e3
    flops = sum(q["p"].flops() for q in problems)
    out = {
        "family": family, "workload": FAMILY_NAMES[family], "steps": steps,
        "ms_per_step": step_ms, "tflops": flops / (step_ms * 1e-3) / 1e12,
        "gflop_per_step": flops / 1e9, "cold": flush is not None,
        "wall_s": round(wall, 4), "input_gen_s": round(gen_s, 2),
        "per_shape": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()}
                      for s in per_shape],
    }
    dom = max(range(len(per_shape)), key=lambda i: per_shape[i]["avg_us"])
    out["roofline"] = roofline_of(per_shape[dom])
    if warm:
        wms = graph_replay_ms(problems, steps, warmup, stream, dev)
        out["warm"] = {"ms_per_step": wms, "tflops": flops / (wms * 1e-3) / 1e12,
                       "timing": "K steps without flushes captured in one HIP graph, "
                                 "replayed once"}
    if cpu_gflop > 0:
        print(f"[bench] family {family}: CPU baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(problems, cpu_gflop)
    print(f"[bench] family {family}: done, {out['tflops']:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--family", type=int, default=DEFAULT_FAMILY, choices=sorted(FAMILY_NAMES),
                    help="the headline family (value, roofline, CPU baseline)")
    ap.add_argument("--families", default=DEFAULT_OTHERS,
                    help="other families measured in the same run (comma list, or none)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written before every timed launch (0: warm, no flush)")
    ap.add_argument("--warm", action="store_true", help="no flush before the timed launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", default="",
                    help="run only this shape of --family (3 launches) and a 512 MiB device copy "
                         "(3 launches), for rocprofv3 --pmc passes")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two rocprofv3 --pmc output directories of a traffic probe into "
                         "profiles/traffic.json")
    ap.add_argument("--ingest-mfma", default="", metavar="PMC_DIR",
                    help="MFMA busy cycles, GPU-active cycles and kernel time of a traffic probe's "
                         "rocprofv3 --pmc --kernel-trace run, into profiles/mfma.json")
    ap.add_argument("--summarize-trace", default="",
                    help="per-shape kernel durations from a rocprofv3 --kernel-trace output "
                         "directory of a bench.py run of --family with --families none")
    ap.add_argument("--cpu-gflop", type=float, default=CPU_SAMPLE_GFLOP,
                    help="oracle work (GFLOP) of the CPU baseline sample")
    ap.add_argument("--per-shape-out", default="", help="also write the result here (indented)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.family)
        return
    if args.ingest_traffic:
        if not args.traffic_probe:
            raise SystemExit("--ingest-traffic needs --traffic-probe NAME (the probed shape)")
        ingest_traffic(args.ingest_traffic[0], args.ingest_traffic[1], args.traffic_probe)
        return
    if args.ingest_mfma:
        if not args.traffic_probe:
            raise SystemExit("--ingest-mfma needs --traffic-probe NAME (the probed shape)")
        ingest_mfma(args.ingest_mfma, args.traffic_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); there is "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    others = parse_families(args.families, args.family)

    import torch

    import moe_grouped_gemm_block_amd as fp8bs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fp8bs._load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.traffic_probe:
        problems = build_problems(args.family, dev)
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

    flush_mib = 0 if args.warm else args.flush_mib
    flush = (torch.empty((flush_mib << 20) // 4, dtype=torch.int32, device=dev)
             if flush_mib > 0 else None)

    head = measure_family(args.family, args.steps, args.warmup, flush, stream, dev,
                          0.0 if args.no_cpu_baseline else args.cpu_gflop)
    torch.cuda.empty_cache()
    fams = {}
    for f in others:
        fams[str(f)] = measure_family(f, min(args.steps, OTHER_STEPS), min(args.warmup, 2),
                                      flush, stream, dev, warm=False)
        torch.cuda.empty_cache()

    ms_per_step = head["ms_per_step"]
    timing = (f"cold: each GEMM launch preceded by a {flush_mib} MiB fill outside the event "
              "pair that times it; step time = sum over the family's shapes of the mean "
              "launch time over K steps, enqueued back to back behind a spin kernel"
              if flush is not None else
              "warm: step time = sum over the family's shapes of the mean launch time over K "
              "steps, enqueued back to back behind a spin kernel, no flush")
    out = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": FAMILY_NAMES[args.family], "family": args.family,
                   "shapes": [s["name"] for s in head["per_shape"]],
                   "gflop_per_step": head["gflop_per_step"], "timing": timing,
                   "flush_mib": flush_mib,
                   "input_sha256": {s["name"]: s["input_sha256"] for s in head["per_shape"]}},
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "warm": head.get("warm"),
        "per_shape": head["per_shape"],
        "families": {k: {kk: vv for kk, vv in v.items()} for k, v in fams.items()},
        "wall_s": head["wall_s"], "input_gen_s": head["input_gen_s"],
        "device": torch.cuda.get_device_name(dev),
    }
    if args.per_shape_out:
        with open(args.per_shape_out, "w") as fh:
            json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


# ---- profiler ingestion -------------------------------------------------------------

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


def _gemm_kernel(name: str) -> bool:
    return "fp8bs_gemm_kernel" in name or "fp8bs_stream_kernel" in name


def _pick(tab, pred):
    ks = [k for k in tab if pred(k)]
    if len(ks) != 1:
        raise SystemExit(f"expected one matching kernel, found {ks}")
    return ks[0], tab[ks[0]]


def ingest_traffic(fetch_dir, write_dir, name):
    """profiles/traffic.json: HBM bytes per launch of the GEMM kernel in a traffic probe,
    FETCH_SIZE and WRITE_SIZE (KiB) scaled so that the plain copy of COPY_PROBE_BYTES
    reads and writes exactly that many bytes."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    gk, gf = _pick(fetch, _gemm_kernel)
    ck, cf = _pick(fetch, lambda k: "fp8bs" not in k and "copy" in k.lower())
    _, gw = _pick(write, _gemm_kernel)
    _, cw = _pick(write, lambda k: "fp8bs" not in k and "copy" in k.lower())
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


def _pmc_durations(d, counter, pred):
    """Durations (ns) of the dispatches of kernels matching pred in a rocprofv3 --pmc csv
    output directory (one row per dispatch and counter carries the dispatch's stamps)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += [r for r in csv.DictReader(open(path))
                 if r["Counter_Name"] == counter and pred(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def ingest_mfma(pmc_dir, name, simds=1024, xcds=8):
    """profiles/mfma.json: for the GEMM dispatches of a traffic probe run under
    `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE`:
    MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES summed over every SIMD / (GRBM_GUI_ACTIVE
    of one XCD x SIMDs) -- rocprofv3's own MfmaUtil metric, 256 CUs x 4 SIMDs; the csv sums
    GRBM_GUI_ACTIVE over the eight XCDs, so one XCD's count is that sum / 8.  The shader
    clock the dispatch ran at is one XCD's GRBM_GUI_ACTIVE / the dispatch's duration (its
    start and end stamps in the same csv).  A 16x16x128 FP8 MFMA keeps its SIMD's matrix
    unit busy for 32 cycles, so the busy fraction is the achieved FP8 rate over the peak at
    the clock the kernel actually ran at."""
    busy = _pmc_per_dispatch(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _pmc_per_dispatch(pmc_dir, "GRBM_GUI_ACTIVE")
    gk, b = _pick(busy, _gemm_kernel)
    _, g = _pick(gui, _gemm_kernel)
    g = [v / xcds for v in g]
    durs = _pmc_durations(pmc_dir, "GRBM_GUI_ACTIVE", _gemm_kernel)
    med = lambda v: sorted(v)[len(v) // 2]
    rec = {"kernel": gk, "dispatches": len(b),
           "mfma_busy_cycles": med(b), "gui_active_cycles": med(g),
           "mfma_busy_frac": med(b) / (med(g) * simds),
           "mfma_instructions_16x16x128": med(b) / 32.0,
           "normalisation": f"sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE of one XCD x "
                            f"{simds} SIMDs)"}
    if durs:
        rec["kernel_us"] = med(durs) / 1e3
        rec["sclk_ghz"] = med(g) / med(durs)
        rec["peak_at_sclk_tflops"] = 8192 * 256 * rec["sclk_ghz"] / 1e3
    path = os.path.join(ROOT, "profiles", "mfma.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    if data.get("source_sha256") != kernel_source_hash():
        data = {"source_sha256": kernel_source_hash(), "shapes": {}}
    data["shapes"][name] = rec
    os.makedirs(os.path.dirname(path), exist_ok=True)
    json.dump(data, open(path, "w"), indent=1)
    print(json.dumps(rec))


def summarize_trace(d, family):
    """Average duration per workload shape from a kernel trace of `bench.py --family F
    --families none`.  Each call is one GEMM dispatch (staged or B-streaming kernel),
    followed by a split-K reduction when its plan splits K; the calls cycle through the
    family's shapes in order, so a GEMM dispatch starts the next shape and a reduction
    belongs to the GEMM before it.  A call whose GEMM dispatch directly follows a fill
    kernel (the cache flush) is cold; the others (warm-up before graph capture, the graph
    replay) are warm; both are reported."""
    import csv
    import glob
    from moe_grouped_gemm_block_amd import synth
    names = [x["name"] for x in synth.workload_shapes(family)]
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    acc = {n: {"cold": [], "warm": [], "red_cold": [], "red_warm": []} for n in names}
    call = -1
    prev_fill = False
    cold = False
    for r in rows:
        kn = r["Kernel_Name"]
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "fp8bs_splitk_reduce" in kn:
            if call >= 0:
                acc[names[call % len(names)]]["red_cold" if cold else "red_warm"].append(us)
        elif _gemm_kernel(kn):
            call += 1
            cold = prev_fill
            acc[names[call % len(names)]]["cold" if cold else "warm"].append(us)
        prev_fill = "FillFunctor" in kn
    out = {}
    for n in names:
        a = acc[n]
        rec = {}
        for kind in ("cold", "warm"):
            v, w = a[kind], a["red_" + kind]
            if not v:
                continue
            avg = sum(v) / len(v)
            ravg = sum(w) / len(w) if w else 0.0
            rec[kind] = {"dispatches": len(v), "avg_us": avg, "min_us": min(v),
                         "max_us": max(v), "reduce_dispatches": len(w), "reduce_avg_us": ravg,
                         "call_avg_us": avg + ravg * len(w) / len(v)}
        out[n] = rec
    print(json.dumps(out, indent=1))


def cpu_baseline(problems, gflop_target: float):
    """The oracle, untuned, on the host cores: the first R valid rows of D (all N columns)
    of every shape of the step, R chosen so that the sample is about `gflop_target` GFLOP;
    timed, reported in TFLOP/s."""
    import numpy as np

    import oracle

    per_row = 0.0
    for q in problems:
        p = q["p"]
        per_row += 2.0 * p.N * p.K * (1 if p.kind != "k_grouped" else 1.0 / 64)
    rows_per_shape = max(1, int(gflop_target * 1e9 / per_row))
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
            "kind": "oracle", "seconds": round(t, 3), "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
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
