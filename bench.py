#!/usr/bin/env python3
"""Benchmark of the group-wise 4-bit linear layer on one MI355X.

One step = the quantized linears of one Llama-3-8B decode token: 32 layers x
(q, k, v, o, gate, up, down) = 224 linear_int4_groups calls at M=1, group 128,
bf16 activations, f32 bias on every q projection.  Every layer has its own
weights (3.76 GB packed + scales + zeros per step), so each step streams the
weights from HBM rather than from the 256 MB last-level cache.  The step is
captured once in a HIP graph and replayed.

Printed JSON line (rank 0):
  value        effective weight GB/s over the whole step (packed + scale + zero
               bytes / wall time of the replayed graph, launch gaps included)
  roofline     the decode kernel alone (gemv_kernel, every launch of the step):
               algorithmic bytes per launch / its average launch duration
               (HIP events around the replayed step graph)
  grouped      the same step with q/k/v and gate/up each run as one grouped
               call (woq_linear_int4_groups_grouped: one launch per group)
  prepared     the same step over prepared (fragment-ordered) weights, made
               once before timing by woq_prepare_int4 (also grouped)
  prefill      TFLOP/s of the M=2048 GEMM path on both prefill shapes
  cpu_baseline the CPU oracle's linear on a bounded sample of the same layer
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = "int4-g128 linear: effective weight GB/s (% HBM peak) at M=1; TFLOP/s at M=2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
GROUP = 128
TRAFFIC_SUMMARY = ROOT / "profiles" / "traffic_gemv_decode_m1_g128.txt"
KERNEL_SOURCES = ["linear_gemv.hip", "mfma_common.h"]


def weight_bytes(n: int, k: int, group: int = GROUP, sym16: bool = False, mx: bool = False,
                 zp4: bool = False) -> int:
    """Packed codes + float32 scale + uint8 zero of an [n, k] weight (for signed
    codes: packed codes + float16 scale; for MXFP4: codes + one byte per 32;
    with packed zero points: two zero points a byte)."""
    if mx:
        return n * k // 2 + n * k // 32
    if zp4:
        return n * k // 2 + (n * k // group) * 4 + n * ((k // group + 1) // 2)
    return n * k // 2 + (n * k // group) * (2 if sym16 else 5)


def algorithmic_bytes(m: int, n: int, k: int, has_bias: bool, group: int = GROUP,
                      sym16: bool = False, mx: bool = False, zp4: bool = False) -> int:
    """Bytes a linear call must move at least once: weights, x, y (bf16), bias."""
    return weight_bytes(n, k, group, sym16, mx, zp4) + m * k * 2 + m * n * 2 + (n * 4 if has_bias else 0)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "weight_only_quantization_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary.

    Returns None unless the summary was taken on the current kernel sources.
    """
    if not TRAFFIC_SUMMARY.exists():
        return None
    fields = {}
    for line in TRAFFIC_SUMMARY.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def build_decode_step(torch, woq, layers: int, seed: int = 2024):
    """Seeded weights and activations of `layers` Llama-3-8B layers on the GPU."""
    from workloads import LLAMA3_8B_LAYER

    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    calls = []
    for layer in range(layers):
        for idx, (role, n, k, has_bias) in enumerate(LLAMA3_8B_LAYER):
            gen.manual_seed(seed + 100 * layer + idx)
            w = torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32).mul_(0.02)
            q, s, z = woq.quantize_groups(w, GROUP)
            packed = woq.pack_uint4(q)
            del w, q
            x = torch.randn((1, k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            b = (torch.randn((n,), generator=gen, device=dev, dtype=torch.float32).mul_(0.01)
                 if has_bias else None)
            y = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
            calls.append(dict(role=role, n=n, k=k, x=x, packed=packed, scale=s, zero=z, bias=b, y=y))
    torch.cuda.synchronize()
    return calls


def run_calls(woq, calls):
    for c in calls:
        woq.linear_int4_groups(c["x"], c["packed"], c["scale"], c["zero"], bias=c["bias"],
                               group=GROUP, out=c["y"], out_dtype=c["y"].dtype)


def grouped_plan(calls, layers: int):
    """The decode step with the projections that share an input in one call:
    per layer (q, k, v) on q's activations, o, (gate, up) on gate's, down."""
    per = len(calls) // layers
    groups = []
    for layer in range(layers):
        c = calls[layer * per:(layer + 1) * per]
        roles = {cc["role"]: cc for cc in c}
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            groups.append([roles[nm] for nm in names])
    return groups


def run_groups(woq, groups, prepared: bool = False):
    key = "prepared" if prepared else "packed"
    for g in groups:
        woq.linear_int4_groups_grouped(g[0]["x"], [(c[key], c["scale"], c["zero"], c["bias"]) for c in g],
                                       prepared=prepared, out_dtype=g[0]["y"].dtype, outs=[c["y"] for c in g])


def run_calls_prepared(woq, calls):
    for c in calls:
        woq.linear_int4_groups_prepared(c["x"], c["prepared"], c["scale"], c["zero"], bias=c["bias"],
                                        out=c["y"], out_dtype=c["y"].dtype)


def time_step(torch, run, steps: int, warmup: int, use_graph: bool):
    """Seconds for `steps` replays of one step (a HIP graph of run(), or run()
    launched eagerly), after `warmup` untimed ones; events bracket the replays."""
    run()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()           # warm-up on a side stream, as graph capture requires
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
    step = graph.replay if graph is not None else run
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = e0.elapsed_time(e1) * 1e-3
    del graph
    return elapsed


def measure_prefill(torch, woq, reps: int = 5, calls: int = 20):
    """Per-call time of each prefill shape: `calls` back-to-back launches (pre-pass
    included) between two events, median of `reps` repetitions, after warm-up."""
    from workloads import PREFILL

    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    out = []
    for case in PREFILL:
        gen.manual_seed(case.seed_w)
        w = torch.randn((case.n, case.k), generator=gen, device=dev).mul_(0.02)
        q, s, z = woq.quantize_groups(w, case.group)
        packed = woq.pack_uint4(q)
        del w, q
        x = torch.randn((case.m, case.k), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((case.m, case.n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(woq.linear_workspace_bytes(case.m, case.n, case.k, case.group, False),
                         dtype=torch.uint8, device=dev)
        for _ in range(5):
            woq.linear_int4_groups(x, packed, s, z, group=case.group, out=y, workspace=ws)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                woq.linear_int4_groups(x, packed, s, z, group=case.group, out=y, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / calls)
        t = statistics.median(times)
        flops = 2.0 * case.m * case.n * case.k
        out.append(dict(shape=f"{case.m}x{case.n}x{case.k}", ms=round(t * 1e3, 4),
                        tflops=round(flops / t / 1e12, 1)))
    tot_flops = sum(2.0 * c.m * c.n * c.k for c in PREFILL)
    tot_t = sum(o["ms"] for o in out) * 1e-3
    tf = tot_flops / tot_t / 1e12
    return dict(metric="TFLOP/s at M=2048 (both prefill shapes, pre-pass included, back-to-back calls)",
                value=round(tf, 1), peak=BF16_PEAK_TFLOPS, frac=round(tf / BF16_PEAK_TFLOPS, 4),
                per_shape=out, plan=woq.linear_plan(2048, 14336, 4096, GROUP))


def measure_configs(torch, woq, reps: int = 40, pool_bytes: int = 1 << 30, cases=None,
                    sym16: bool = False, mx: bool = False, zp4: bool = False):
    """Per-launch time of every small-M sweep and act-order configuration (or of
    `cases`; with sym16, over signed codes with float16 scales; with mx, over
    MXFP4 weights).

    Weights are random bytes in the Int4GroupLinear layout (timing does not
    depend on the values); each configuration rotates over enough copies
    (>= 1 GB in all) that every launch reads its weights from HBM, not from
    the 256 MB last-level cache.  Launches are replayed from one HIP graph and
    timed with events around it.
    """
    from workloads import ACTORDER, SWEEP

    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    out = []
    pools = {}
    for case in (cases if cases is not None else (*SWEEP, *ACTORDER)):
        key = (case.n, case.k, case.group)
        wb = weight_bytes(case.n, case.k, case.group, sym16, mx, zp4)
        if key not in pools:
            pools.clear()
            torch.cuda.empty_cache()
            copies = max(2, -(-pool_bytes // wb))
            ng = case.k // case.group
            if mx:
                pools[key] = [
                    (torch.randint(0, 256, (case.n, case.k // 2), generator=gen, device=dev, dtype=torch.uint8),
                     torch.randint(118, 124, (case.n, case.k // 32), generator=gen, device=dev, dtype=torch.uint8),
                     None)
                    for _ in range(copies)]
            elif sym16:
                pools[key] = [
                    (torch.randint(0, 256, (case.n, case.k // 2), generator=gen, device=dev, dtype=torch.uint8),
                     torch.rand((case.n, ng), generator=gen, device=dev).mul_(0.01).add_(1e-3).half(), None)
                    for _ in range(copies)]
            else:
                pools[key] = [
                    (torch.randint(0, 256, (case.n, case.k // 2), generator=gen, device=dev, dtype=torch.uint8),
                     torch.rand((case.n, ng), generator=gen, device=dev).mul_(0.01).add_(1e-3),
                     torch.randint(0, 256 if zp4 else 16, (case.n, (ng + 1) // 2 if zp4 else ng), generator=gen,
                                   device=dev, dtype=torch.uint8))
                    for _ in range(copies)]
        pool = pools[key]
        x = torch.randn((case.m, case.k), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((case.m, case.n), dtype=torch.bfloat16, device=dev)
        bias = torch.randn((case.n,), generator=gen, device=dev).mul_(0.01) if case.has_bias else None
        order = (torch.randperm(case.k, generator=gen, device=dev).to(torch.int32)
                 if case.act_order else None)
        ws_bytes = (woq.linear_int4_groups_zp4_workspace_bytes if zp4 else woq.linear_workspace_bytes)(
            case.m, case.n, case.k, case.group, order is not None)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def call(i):
            p, sc, z = pool[i % len(pool)]
            if mx:
                woq.linear_mxfp4(x, p, sc, bias=bias, out=y, workspace=ws if ws_bytes else None)
            elif sym16:
                woq.linear_int4_sym(x, p, sc, bias=bias, order=order, group=case.group, out=y,
                                    workspace=ws if ws_bytes else None)
            elif zp4:
                woq.linear_int4_groups_zp4(x, p, sc, z, bias=bias, order=order, group=case.group, out=y,
                                           workspace=ws)
            else:
                woq.linear_int4_groups(x, p, sc, z, bias=bias, order=order, group=case.group, out=y,
                                       workspace=ws if ws_bytes else None)

        for i in range(len(pool)):
            call(i)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(0)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                call(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        flops = 2.0 * case.m * case.n * case.k
        ab = algorithmic_bytes(case.m, case.n, case.k, case.has_bias, case.group, sym16, mx, zp4) + (
            case.k * 4 if case.act_order else 0)
        out.append(dict(name=case.name, m=case.m, n=case.n, k=case.k, group=case.group,
                        us=round(t * 1e6, 2), weight_GBps=round(wb / t / 1e9, 1),
                        hbm_frac=round(ab / t / 1e9 / HBM_PEAK_GBS, 4),
                        tflops=round(flops / t / 1e12, 2),
                        mfma_frac=round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                        plan=woq.linear_plan(case.m, case.n, case.k, case.group, order is not None)))
        del g
    pools.clear()
    torch.cuda.empty_cache()
    return out


def cpu_baseline(min_seconds: float = 10.0, max_passes: int = 8):
    """The CPU oracle's linear over one Llama-3-8B layer's seven M=1 linears.

    Weights are drawn directly in the Int4GroupLinear layout (the oracle's
    quantizer is not timed); passes over the layer repeat until min_seconds.
    """
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    layer = []
    for idx, (role, n, k, has_bias) in enumerate(workloads.LLAMA3_8B_LAYER):
        p, s, z = workloads.packed_weights(n, k, GROUP, seed=900 + idx)
        x = workloads.activations_bf16(1, k, seed=950 + idx)
        b = workloads.bias(n, seed=990) if has_bias else None
        layer.append((n, k, p, s, z, x, b))
    bytes_done, passes = 0, 0
    t0 = time.perf_counter()
    while passes < max_passes:
        for (n, k, p, s, z, x, b) in layer:
            oracle.linear_int4_groups(x, p, s, z, n, k, GROUP, bias=b)
            bytes_done += weight_bytes(n, k)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(bytes_done / dt / 1e9, 4), unit="GB/s", cores=int(blas_threads),
                kind="oracle",
                sample=f"{passes} pass(es) of one Llama-3-8B layer's 7 linears at M=1, group 128 "
                       f"({bytes_done / 1e9:.2f} GB of weights, {dt:.1f} s; numpy float64; "
                       f"BLAS threads={blas_threads}, affinity cores={len(os.sched_getaffinity(0))})")


DECODE_TAG = "gemv_kernel"
COPY_TAG = "copyBuffer"            # the runtime's device-to-device copy kernel


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirpath: Path, suffix: str) -> Path:
    hits = sorted(dirpath.rglob(f"*{suffix}"))
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirpath}")
    return hits[0]


def summarize_profiles(root: Path, copy_mib: int) -> None:
    """Print the text summaries kept under profiles/ from three rocprofv3 runs.

    root/ktrace: --kernel-trace --stats of the bench; root/fetch and root/write:
    --pmc FETCH_SIZE and --pmc WRITE_SIZE of a short eager bench that also runs a
    plain device copy of copy_mib MiB, whose counter reading calibrates the
    counters to bytes (factor = copied bytes / counted bytes).
    """
    trace = _csv_rows(_find(root / "ktrace", "_kernel_trace.csv"))
    by_kernel = {}
    for r in trace:
        name = r["Kernel_Name"]
        if "woq::" not in name:
            continue
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by_kernel.setdefault(name, []).append((int(r["Grid_Size_X"]), dur))
    out = ["# rocprofv3 kernel trace of bench.py, woq kernels only (durations in microseconds)"]
    for name, rows in sorted(by_kernel.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        durs = [d for _, d in rows]
        out.append(f"kernel: {name}")
        out.append(f"  launches: {len(rows)}  average_us: {statistics.mean(durs) / 1e3:.3f}  "
                   f"min_us: {min(durs) / 1e3:.3f}  max_us: {max(durs) / 1e3:.3f}")
        grids = {}
        for g, d in rows:
            grids.setdefault(g, []).append(d)
        for g, ds in sorted(grids.items()):
            out.append(f"  grid_threads {g}: launches {len(ds)}  average_us {statistics.mean(ds) / 1e3:.3f}")
    for cand in sorted((root / "ktrace").rglob("*.json")):
        for line in cand.read_text().splitlines():
            try:
                rl = json.loads(line)["roofline"]
            except (ValueError, KeyError, TypeError):
                continue
            out.append(f"bench_avg_launch_us (HIP events around the replayed step graph): {rl['avg_launch_us']}")
    print("\n".join(out))

    def counter(sub, cname):
        rows = _csv_rows(_find(root / sub, "_counter_collection.csv"))
        sk = [float(r["Counter_Value"]) for r in rows
              if r["Counter_Name"] == cname and DECODE_TAG in r["Kernel_Name"]]
        cp = [float(r["Counter_Value"]) for r in rows
              if r["Counter_Name"] == cname and COPY_TAG in r["Kernel_Name"]]
        return sk, cp

    f_sk, f_cp = counter("fetch", "FETCH_SIZE")
    w_sk, w_cp = counter("write", "WRITE_SIZE")
    copy_bytes = copy_mib << 20
    if not f_cp or not w_cp:
        raise SystemExit("the calibration copy is missing from the counter runs")
    # the largest copy of the run is the calibration copy
    f_factor = copy_bytes / (max(f_cp) * 1024.0)
    w_factor = copy_bytes / (max(w_cp) * 1024.0)
    fetch = statistics.mean(f_sk) * 1024.0 * f_factor
    write = statistics.mean(w_sk) * 1024.0 * w_factor
    print()
    print("# HBM traffic of the decode GEMV kernel per launch (rocprofv3 --pmc, copy-calibrated)")
    # the sources the counted kernel was built from, as the profiled bench printed them
    src_hash = None
    for cand in sorted((root / "fetch").rglob("*.json")):
        for line in cand.read_text().splitlines():
            try:
                src_hash = json.loads(line)["roofline"]["kernel_source_sha256_16"]
            except (ValueError, KeyError, TypeError):
                continue
    if src_hash is None:
        raise SystemExit("the profiled bench's JSON line (fetch/*.json) is missing")
    print(f"kernel_source_sha256_16: {src_hash}")
    print(f"launches_counted: {len(f_sk)}")
    print(f"fetch_KiB_raw_avg: {statistics.mean(f_sk):.1f}")
    print(f"write_KiB_raw_avg: {statistics.mean(w_sk):.1f}")
    print(f"copy_calibration_MiB: {copy_mib}")
    print(f"fetch_factor: {f_factor:.4f}")
    print(f"write_factor: {w_factor:.4f}")
    print(f"hbm_bytes_per_launch: {fetch + write:.0f}")



def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the small-M sweep and act-order per-launch timings")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a graph")
    ap.add_argument("--no-grouped", action="store_true", help="skip the grouped-call step")
    ap.add_argument("--no-prepared", action="store_true",
                    help="skip the decode step over prepared weights")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="print the profiles/ summaries from rocprofv3 output under DIR and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(Path(args.summarize_profiles), args.copy_calibration_mib or 512)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import weight_only_quantization_amd as woq

    woq.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    calls = build_decode_step(torch, woq, args.layers)
    wbytes = sum(weight_bytes(c["n"], c["k"]) for c in calls)
    abytes = [algorithmic_bytes(1, c["n"], c["k"], c["bias"] is not None) for c in calls]

    elapsed = time_step(torch, lambda: run_calls(woq, calls), args.steps, args.warmup,
                        not args.no_graph)
    ms_per_step = elapsed / args.steps * 1e3
    value = wbytes * args.steps / elapsed / 1e9

    # The step is one graph of back-to-back launches of the decode kernel, so the
    # kernel's average launch duration is the timed region over the launches in it
    # (inter-launch gaps included, which makes the figure conservative).
    avg_launch = elapsed / (args.steps * len(calls))
    achieved = sum(abytes) / len(abytes) / avg_launch / 1e9
    traffic = read_traffic()
    roofline = dict(
        bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
        frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
        kernel="woq::gemv_kernel<GB=4,FR=1,CC,PF=4> (every launch of the step)",
        launches=len(calls), avg_launch_us=round(avg_launch * 1e6, 3),
        algorithmic_bytes_per_launch=round(sum(abytes) / len(abytes)),
        traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
        kernel_source_sha256_16=kernel_source_hash(),
        plans={f"{c['n']}x{c['k']}": woq.linear_plan(1, c["n"], c["k"], GROUP)
               for c in calls[:len(calls) // args.layers]},
    )

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)          # a device-to-device copy: the runtime's copyBuffer kernel
        torch.cuda.synchronize()
        del src, dst

    # The same step with the projections that share their input grouped into one
    # call each (q, k, v; gate, up): one decode launch per group.
    groups = grouped_plan(calls, args.layers)
    grouped = None
    if not args.no_grouped:
        el_g = time_step(torch, lambda: run_groups(woq, groups), args.steps, args.warmup, not args.no_graph)
        avg_g = el_g / (args.steps * len(groups))
        grouped = dict(
            metric="effective weight GB/s at M=1, projections sharing an input grouped (same linears, same bytes)",
            value=round(wbytes * args.steps / el_g / 1e9, 1), unit="GB/s",
            ms_per_step=round(el_g / args.steps * 1e3, 4), launches_per_step=len(groups),
            hbm_peak_frac=round(wbytes * args.steps / el_g / 1e9 / HBM_PEAK_GBS, 4),
            avg_launch_us=round(avg_g * 1e6, 3),
            roofline_achieved=round(sum(abytes) / len(groups) / avg_g / 1e9, 1),
            roofline_frac=round(sum(abytes) / len(groups) / avg_g / 1e9 / HBM_PEAK_GBS, 4),
            note="woq_linear_int4_groups_grouped: per layer (q,k,v) and (gate,up) share one launch each")

    prepared = None
    if not args.no_prepared:
        for c in calls:
            c["prepared"] = woq.prepare_int4(c["packed"])
        torch.cuda.synchronize()
        el_p = time_step(torch, lambda: run_calls_prepared(woq, calls), args.steps, args.warmup,
                         not args.no_graph)
        val_p = wbytes * args.steps / el_p / 1e9
        avg_p = el_p / (args.steps * len(calls))
        el_pg = None if args.no_grouped else time_step(
            torch, lambda: run_groups(woq, groups, prepared=True), args.steps, args.warmup, not args.no_graph)
        prepared = dict(
            metric="effective weight GB/s at M=1 over prepared weights (same step, same bytes)",
            grouped_value=None if el_pg is None else round(wbytes * args.steps / el_pg / 1e9, 1),
            grouped_ms_per_step=None if el_pg is None else round(el_pg / args.steps * 1e3, 4),
            value=round(val_p, 1), unit="GB/s", ms_per_step=round(el_p / args.steps * 1e3, 4),
            hbm_peak_frac=round(val_p / HBM_PEAK_GBS, 4), avg_launch_us=round(avg_p * 1e6, 3),
            roofline_achieved=round(sum(abytes) / len(abytes) / avg_p / 1e9, 1),
            roofline_frac=round(sum(abytes) / len(abytes) / avg_p / 1e9 / HBM_PEAK_GBS, 4),
            note="woq_prepare_int4 re-orders each weight once before timing (load time)")
        for c in calls:
            del c["prepared"]

    prefill = None if args.no_prefill else measure_prefill(torch, woq)
    configs = None if args.no_configs else measure_configs(torch, woq)
    sym16 = mxfp4 = zp4 = None
    if not args.no_configs:
        from workloads import ZP4
        zp4 = dict(
            note="packed 4-bit zero points, unpacked into the workspace by each call (woq_linear_int4_groups_zp4)",
            configs=measure_configs(torch, woq, cases=ZP4, zp4=True))
        from workloads import SYM16
        sym16 = dict(
            note="signed int4 codes with float16 scales, no zero point (woq_linear_int4_sym_f16)",
            configs=measure_configs(torch, woq, cases=SYM16, sym16=True))
        from workloads import MXFP4
        mxfp4 = dict(
            note="MXFP4: E2M1 codes, one E8M0 scale per block of 32 (woq_linear_mxfp4); plan strings are "
                 "woq_linear_plan's for the same sizes at group 32, except that the MXFP4 pre-pass copies the "
                 "activations in natural order and forms no group sums",
            configs=measure_configs(torch, woq, cases=MXFP4, mx=True))
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    line = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(ms_per_step, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="Llama-3-8B decode linears at M=1: 32 layers x (q,k,v,o,gate,up,down), "
                             "int4 group 128, bf16 x, f32 bias on q, bf16 y",
                    m=1, group=GROUP, layers=args.layers, launches_per_step=len(calls),
                    weight_bytes_per_step=wbytes, hbm_peak_frac=round(value / HBM_PEAK_GBS, 4),
                    graph=not args.no_graph, accumulate="f32",
                    tokens_per_s_linears_only=round(1.0 / (ms_per_step * 1e-3), 1) if args.layers == 32 else None),
        roofline=roofline, grouped=grouped, prepared=prepared, prefill=prefill, configs=configs,
        sym16=sym16, mxfp4=mxfp4, zp4=zp4,
        cpu_baseline=cpu,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
