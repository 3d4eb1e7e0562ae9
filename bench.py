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
  roofline     the step's dominant kernel on its own: the row-streaming decode
               kernel on the gate/up projections (14336x4096, 2 of the 7 linears
               of a layer and 54 % of the step's bytes with the down projection),
               algorithmic bytes per launch / average launch duration of a graph
               of back-to-back launches over >= 1 GB of rotating weight copies
               (HIP events); the down projection and the whole-step average beside it
  grouped      the same step with q/k/v and gate/up each run as one grouped
               call (woq_linear_int4_groups_grouped: one launch per group)
  prepared     the same step over prepared (fragment-ordered) weights, made
               once before timing by woq_prepare_int4 (also grouped)
  prefill      TFLOP/s of the M=2048 GEMM path on both prefill shapes
  cpu_baseline the CPU oracle (dequantize + float64 matmul) on bounded samples of
               every configuration, with its core count and a single-thread run
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
TRAFFIC_SUMMARY = ROOT / "profiles" / "traffic_rows_decode_m1_g128.txt"
KERNEL_SOURCES = ["linear_rows.hip"]


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
    included) between two events, median of `reps` repetitions, after warm-up;
    once over the canonical weights and once over prepared ones."""
    from workloads import PREFILL

    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    out = []

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / calls)
        return statistics.median(times)

    for case in PREFILL:
        gen.manual_seed(case.seed_w)
        w = torch.randn((case.n, case.k), generator=gen, device=dev).mul_(0.02)
        q, s, z = woq.quantize_groups(w, case.group)
        packed = woq.pack_uint4(q)
        del w, q
        prep = woq.prepare_int4(packed)
        x = torch.randn((case.m, case.k), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((case.m, case.n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(woq.linear_workspace_bytes(case.m, case.n, case.k, case.group, False),
                         dtype=torch.uint8, device=dev)
        t = timed(lambda: woq.linear_int4_groups(x, packed, s, z, group=case.group, out=y, workspace=ws))
        tp = timed(lambda: woq.linear_int4_groups_prepared(x, prep, s, z, out=y, workspace=ws))
        flops = 2.0 * case.m * case.n * case.k
        out.append(dict(shape=f"{case.m}x{case.n}x{case.k}", ms=round(t * 1e3, 4),
                        tflops=round(flops / t / 1e12, 1), prepared_ms=round(tp * 1e3, 4),
                        prepared_tflops=round(flops / tp / 1e12, 1)))
        del packed, prep, s, z, x, y, ws
    tot_flops = sum(2.0 * c.m * c.n * c.k for c in PREFILL)
    tot_t = sum(o["ms"] for o in out) * 1e-3
    tot_tp = sum(o["prepared_ms"] for o in out) * 1e-3
    tf = tot_flops / tot_t / 1e12
    return dict(metric="TFLOP/s at M=2048 (both prefill shapes, pre-pass included, back-to-back calls)",
                value=round(tf, 1), peak=BF16_PEAK_TFLOPS, frac=round(tf / BF16_PEAK_TFLOPS, 4),
                prepared_value=round(tot_flops / tot_tp / 1e12, 1),
                prepared_frac=round(tot_flops / tot_tp / 1e12 / BF16_PEAK_TFLOPS, 4),
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
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / reps)
        t = statistics.median(ts)
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


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        return 1


def cpu_baseline():
    """The CPU oracle (dequantize to exact float64, then a float64 matmul) timed
    on the host cores, on bounded samples of every configuration.

    Weights are drawn directly in the Int4GroupLinear layout (the quantizer is
    not timed).  Each configuration computes a sample of its output columns
    (all of them for the decode shapes), best of three; GB/s counts the sampled
    rows' weight bytes, GFLOP/s their 2*M*rows*K.  The decode shapes are also
    run with one BLAS thread.  Dequantization is NumPy element-wise work on one
    thread; the matmul runs on the BLAS threads.
    """
    import numpy as np

    import oracle
    import workloads

    threads = _blas_threads()

    def run(case, rows):
        p, s_, z = workloads.packed_weights(case.n, case.k, case.group, seed=900 + case.seed_w)
        x = workloads.activations_bf16(case.m, case.k, seed=950 + case.seed_x)
        b = workloads.bias(case.n, seed=990) if case.has_bias else None
        o = workloads.order(case.k, seed=case.seed_order) if case.act_order else None
        sel = np.arange(case.n) if rows >= case.n else np.linspace(0, case.n - 1, rows).astype(np.int64)
        best = None
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.linear_int4_groups(x, p, s_, z, case.n, case.k, case.group, bias=b, order=o, rows=sel)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        wbytes = sel.size * (case.k // 2 + case.k // case.group * 5)
        return dict(name=case.name, rows=int(sel.size), of_rows=case.n, s=round(best, 4),
                    weight_GBps=round(wbytes / best / 1e9, 4),
                    gflops=round(2.0 * case.m * sel.size * case.k / best / 1e9, 3))

    per = []
    t_all = time.perf_counter()
    single = []
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            single = [run(c, c.n) for c in workloads.DECODE]
    except Exception:  # noqa: BLE001
        single = []
    decode = [run(c, c.n) for c in workloads.DECODE]
    per += decode
    per += [run(c, 4096) for c in workloads.SWEEP if c.group == 128 or c.m == 1]
    per += [run(c, 1024) for c in workloads.PREFILL]
    per += [run(c, 4096) for c in workloads.ACTORDER]
    total = time.perf_counter() - t_all
    # value: the seven M=1 linears of one layer, weight bytes over summed oracle
    # time, on one thread (the BLAS threads are limited to one; the dequantization
    # is single-threaded NumPy work either way)
    base = single if single else decode
    step_bytes = step_s = 0.0
    for _, n, k, _ in workloads.LLAMA3_8B_LAYER:
        hit = [d for d, c in zip(base, workloads.DECODE) if c.n == n and c.k == k][0]
        step_bytes += weight_bytes(n, k)
        step_s += hit["s"]
    return dict(value=round(step_bytes / step_s / 1e9, 4), unit="GB/s", cores=1 if single else int(threads),
                kind="oracle",
                sample=(f"value: one Llama-3-8B layer's seven M=1 group-128 linears computed in full on one "
                        f"thread (weight bytes / summed oracle time, best of 3); per_config: every decode shape in "
                        f"full and 4096 (act-order, sweep) or 1024 (prefill) evenly spaced output columns of the "
                        f"other configurations with {threads} BLAS threads; {total:.1f} s in all; NumPy float64"),
                blas_threads=int(threads), host_cpus=len(os.sched_getaffinity(0)),
                per_config=per, single_thread_decode=single)


DOMINANT_TAG = "rows_kernel<4, 1, 0, false, 128>"    # 14336x4096 at M=1 (gate, up projections)
DOMINANT_GRID = 3584 * 128                           # 3584 workgroups of 2 waves
DOWN_TAG = "rows_kernel<16, 1, 0, false, 128>"      # 4096x14336 at M=1 (down projection)
DOWN_GRID = 256 * 7 * 64                             # 256 workgroups of 7 waves
COPY_TAG = "copyBuffer"                              # the runtime's device-to-device copy kernel


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirpath: Path, suffix: str) -> Path:
    hits = sorted(dirpath.rglob(f"*{suffix}"))
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirpath}")
    return hits[0]


def _bench_line(dirpath: Path):
    for cand in sorted(dirpath.rglob("*.json")):
        for line in cand.read_text().splitlines():
            try:
                return json.loads(line)
            except ValueError:
                continue
    raise SystemExit(f"no bench JSON line under {dirpath}")


def summarize_trace(root: Path) -> None:
    """Kernel trace summary: every woq kernel, per launch grid, from the
    --kernel-trace --stats run under root, and the bench's own figures."""
    trace = _csv_rows(_find(root, "_kernel_trace.csv"))
    by_kernel = {}
    for r in trace:
        name = r["Kernel_Name"]
        if "woq::" not in name:
            continue
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        by_kernel.setdefault(name, []).append((grid, dur))
    out = ["# rocprofv3 kernel trace, woq kernels only (durations in microseconds)"]
    for name, rows in sorted(by_kernel.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        durs = [d for _, d in rows]
        out.append(f"kernel: {name}")
        out.append(f"  launches: {len(rows)}  average_us: {statistics.mean(durs) / 1e3:.3f}  "
                   f"median_us: {statistics.median(durs) / 1e3:.3f}  min_us: {min(durs) / 1e3:.3f}  "
                   f"max_us: {max(durs) / 1e3:.3f}")
        grids = {}
        for g, d in rows:
            grids.setdefault(g, []).append(d)
        for g, ds in sorted(grids.items()):
            out.append(f"  grid_threads {g}: launches {len(ds)}  average_us {statistics.mean(ds) / 1e3:.3f}  "
                       f"median_us {statistics.median(ds) / 1e3:.3f}")
    line = _bench_line(root)
    rl = line.get("roofline")
    if rl:
        out.append(f"bench roofline kernel: {rl['kernel']}")
        out.append(f"bench avg_launch_us (HIP events around a graph of back-to-back launches): "
                   f"{rl['avg_launch_us']}  achieved_GBps: {rl['achieved']}  frac: {rl['frac']}")
        d = rl.get("down")
        if d:
            out.append(f"bench down projection ({d['kernel']}): avg_launch_us {d['avg_launch_us']}  "
                       f"frac {d['frac']}")
    for c in (line.get("smallbatch") or []) + (line.get("fewrows") or []):
        out.append(f"bench {c['name']}: {c['us']} us per call (HIP events, graph of back-to-back calls)  "
                   f"plan: {c['plan']}")
    pf = line.get("prefill")
    if pf:
        for shp in pf["per_shape"]:
            out.append(f"bench prefill {shp['shape']}: {shp['ms']} ms per call  {shp['tflops']} TFLOP/s")
    print("\n".join(out))


def summarize_traffic(root: Path, copy_mib: int) -> None:
    """HBM bytes per launch of the dominant decode kernel (and of the down
    projection's) from --pmc FETCH_SIZE (root/fetch) and --pmc WRITE_SIZE
    (root/write) runs of the eager 32-layer step, each calibrated by a plain
    device copy of copy_mib MiB in the same run (factor = copied bytes /
    counted bytes)."""

    def counter(sub, cname, tag, grid):
        rows = _csv_rows(_find(root / sub, "_counter_collection.csv"))
        return [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == cname and tag in r["Kernel_Name"] and int(r["Grid_Size"]) == grid]

    def copies(sub, cname):
        rows = _csv_rows(_find(root / sub, "_counter_collection.csv"))
        return [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == cname and COPY_TAG in r["Kernel_Name"]]

    f_cp, w_cp = copies("fetch", "FETCH_SIZE"), copies("write", "WRITE_SIZE")
    if not f_cp or not w_cp:
        raise SystemExit("the calibration copy is missing from the counter runs")
    copy_bytes = copy_mib << 20
    f_factor = copy_bytes / (max(f_cp) * 1024.0)     # the largest copy of the run is the calibration copy
    w_factor = copy_bytes / (max(w_cp) * 1024.0)
    src_hash = _bench_line(root / "fetch")["kernel_source_sha256_16"]
    print(f"kernel_source_sha256_16: {src_hash}")
    print(f"copy_calibration_MiB: {copy_mib}")
    print(f"fetch_factor: {f_factor:.4f}")
    print(f"write_factor: {w_factor:.4f}")
    for label, tag, grid, (n, k) in (("dominant", DOMINANT_TAG, DOMINANT_GRID, (14336, 4096)),
                                     ("down", DOWN_TAG, DOWN_GRID, (4096, 14336))):
        f_sk = counter("fetch", "FETCH_SIZE", tag, grid)
        w_sk = counter("write", "WRITE_SIZE", tag, grid)
        if not f_sk or not w_sk:
            raise SystemExit(f"no {tag} launches with grid {grid} in the counter runs")
        fetch = statistics.mean(f_sk) * 1024.0 * f_factor
        write = statistics.mean(w_sk) * 1024.0 * w_factor
        alg = algorithmic_bytes(1, n, k, False)
        pre = "" if label == "dominant" else f"{label}_"
        print(f"{pre}kernel: woq::{tag} grid_threads {grid} ({n}x{k}, M=1, group {GROUP})")
        print(f"{pre}launches_counted: {len(f_sk)}")
        print(f"{pre}fetch_KiB_raw_avg: {statistics.mean(f_sk):.1f}")
        print(f"{pre}write_KiB_raw_avg: {statistics.mean(w_sk):.1f}")
        print(f"{pre}algorithmic_bytes_per_launch: {alg}")
        print(f"{pre}hbm_bytes_per_launch: {fetch + write:.0f}")
        print(f"{pre}traffic_over_algorithmic: {(fetch + write) / alg:.4f}")


def summarize_mfma(root: Path) -> None:
    """MFMA counters of the prefill GEMM launches (root/pmc: --pmc MfmaUtil
    MfmaFlopsBF16 MfmaFlopsF32) with their durations from the kernel trace of
    the same command (root/ktrace)."""
    rows = _csv_rows(_find(root / "pmc", "_counter_collection.csv"))
    per = {}
    for r in rows:
        if "woq::" not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        per.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    trace = _csv_rows(_find(root / "ktrace", "_kernel_trace.csv"))
    durs = {}
    for r in trace:
        if "woq::" in r["Kernel_Name"]:
            key = (r["Kernel_Name"], int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0))
            durs.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("# MFMA counters per woq kernel and launch grid (averages over the launches counted)")
    for (name, grid), cs in sorted(per.items(), key=lambda kv: -statistics.mean(durs.get(kv[0], [0]))):
        util = statistics.mean(cs.get("MfmaUtil", [float("nan")]))
        fb = statistics.mean(cs.get("MfmaFlopsBF16", [0.0]))
        ff = statistics.mean(cs.get("MfmaFlopsF32", [0.0]))
        d = durs.get((name, grid))
        print(f"kernel: {name}")
        print(f"  grid_threads {grid}: launches_counted {len(cs.get('MfmaUtil', []))}  MfmaUtil_pct {util:.2f}  "
              f"MfmaFlopsBF16 {fb:.4e}  MfmaFlopsF32 {ff:.4e}")
        if d:
            us = statistics.mean(d) / 1e3
            print(f"  kernel_trace: launches {len(d)}  average_us {us:.3f}  "
                  f"bf16_TFLOPs {fb / (us * 1e-6) / 1e12:.1f}  frac_of_bf16_peak "
                  f"{fb / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS:.4f}")


def measure_dominant(torch, woq, reps: int = 100):
    """Per-launch time of the decode kernel on the step's two largest shapes
    (14336x4096: gate and up; 4096x14336: down) at M=1, group 128: `reps`
    back-to-back launches in one HIP graph over >= 1 GB of rotating weight
    copies, HIP events around the replay, median of five replays."""
    from workloads import DECODE

    cases = [c for c in DECODE if (c.n, c.k) in ((14336, 4096), (4096, 14336))]
    res = {(r["n"], r["k"]): r for r in measure_configs(torch, woq, reps=reps, cases=cases)}
    out = {}
    for (n, k), tag in (((14336, 4096), DOMINANT_TAG), ((4096, 14336), DOWN_TAG)):
        r = res[(n, k)]
        ab = algorithmic_bytes(1, n, k, False)
        achieved = ab / (r["us"] * 1e-6) / 1e9
        out[(n, k)] = dict(kernel=f"woq::{tag} on {n}x{k}, M=1, group {GROUP}", avg_launch_us=r["us"],
                           algorithmic_bytes_per_launch=ab, achieved=round(achieved, 1),
                           frac=round(achieved / HBM_PEAK_GBS, 4), plan=r["plan"])
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--only", choices=["all", "step", "dominant", "prefill", "smallbatch", "fewrows"],
                    default="all",
                    help="step: the decode step alone; dominant: the dominant-kernel timing alone; "
                         "prefill: the M=2048 timing alone; smallbatch: M = 16 and 64 on the decode "
                         "shapes alone; fewrows: M = 2 to 4 on the decode shapes alone (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the small-M sweep and act-order per-launch timings")
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of replaying a graph")
    ap.add_argument("--no-grouped", action="store_true", help="skip the grouped-call step")
    ap.add_argument("--no-prepared", action="store_true",
                    help="skip the decode step over prepared weights")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize", nargs=2, metavar=("KIND", "DIR"),
                    help="print a profiles/ summary (KIND: trace, traffic or mfma) from rocprofv3 output "
                         "under DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        kind, where = args.summarize
        if kind == "trace":
            summarize_trace(Path(where))
        elif kind == "traffic":
            summarize_traffic(Path(where), args.copy_calibration_mib or 512)
        elif kind == "mfma":
            summarize_mfma(Path(where))
        else:
            raise SystemExit("--summarize KIND is one of trace, traffic, mfma")
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

    if args.only == "prefill":
        print(json.dumps(dict(prefill=measure_prefill(torch, woq),
                              kernel_source_sha256_16=kernel_source_hash())), flush=True)
        return
    if args.only == "smallbatch":
        from workloads import SMALLBATCH
        print(json.dumps(dict(smallbatch=measure_configs(torch, woq, cases=SMALLBATCH),
                              kernel_source_sha256_16=kernel_source_hash())), flush=True)
        return
    if args.only == "fewrows":
        from workloads import FEWROWS
        print(json.dumps(dict(fewrows=measure_configs(torch, woq, cases=FEWROWS),
                              kernel_source_sha256_16=kernel_source_hash())), flush=True)
        return
    if args.only == "dominant":
        dom = measure_dominant(torch, woq)
        print(json.dumps(dict(roofline=dict(dom[(14336, 4096)], down=dom[(4096, 14336)]),
                              kernel_source_sha256_16=kernel_source_hash())), flush=True)
        return

    # The dominant kernel first, on a GPU that has run nothing else yet: the
    # same conditions as the standalone profiling run (--only dominant).
    dom = measure_dominant(torch, woq) if args.only == "all" else None
    torch.cuda.empty_cache()

    calls = build_decode_step(torch, woq, args.layers)
    wbytes = sum(weight_bytes(c["n"], c["k"]) for c in calls)
    abytes = [algorithmic_bytes(1, c["n"], c["k"], c["bias"] is not None) for c in calls]

    elapsed = time_step(torch, lambda: run_calls(woq, calls), args.steps, args.warmup,
                        not args.no_graph)
    ms_per_step = elapsed / args.steps * 1e3
    value = wbytes * args.steps / elapsed / 1e9
    # the step's launches on average (one graph of back-to-back launches, gaps included)
    avg_launch = elapsed / (args.steps * len(calls))
    step_avg = dict(avg_launch_us=round(avg_launch * 1e6, 3), launches=len(calls),
                    algorithmic_bytes_per_launch=round(sum(abytes) / len(abytes)),
                    achieved=round(sum(abytes) / len(abytes) / avg_launch / 1e9, 1),
                    frac=round(sum(abytes) / len(abytes) / avg_launch / 1e9 / HBM_PEAK_GBS, 4),
                    plans={f"{c['n']}x{c['k']}": woq.linear_plan(1, c["n"], c["k"], GROUP)
                           for c in calls[:len(calls) // args.layers]})

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)          # a device-to-device copy: the runtime's copyBuffer kernel
        torch.cuda.synchronize()
        del src, dst

    if args.only == "step":
        print(json.dumps(dict(metric=METRIC, value=round(value, 1), unit="GB/s", ms_per_step=round(ms_per_step, 4),
                              step_average=step_avg, kernel_source_sha256_16=kernel_source_hash())), flush=True)
        return

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
            note="woq_linear_int4_groups_grouped: per layer (q,k,v) and (gate,up) share one launch each")

    prepared = None
    if not args.no_prepared:
        for c in calls:
            c["prepared"] = woq.prepare_int4(c["packed"])
        torch.cuda.synchronize()
        el_p = time_step(torch, lambda: run_calls_prepared(woq, calls), args.steps, args.warmup,
                         not args.no_graph)
        val_p = wbytes * args.steps / el_p / 1e9
        el_pg = None if args.no_grouped else time_step(
            torch, lambda: run_groups(woq, groups, prepared=True), args.steps, args.warmup, not args.no_graph)
        prepared = dict(
            metric="effective weight GB/s at M=1 over prepared weights (same step, same bytes)",
            grouped_value=None if el_pg is None else round(wbytes * args.steps / el_pg / 1e9, 1),
            grouped_ms_per_step=None if el_pg is None else round(el_pg / args.steps * 1e3, 4),
            value=round(val_p, 1), unit="GB/s", ms_per_step=round(el_p / args.steps * 1e3, 4),
            hbm_peak_frac=round(val_p / HBM_PEAK_GBS, 4),
            note="woq_prepare_int4 re-orders each weight once before timing (load time); the prepared "
                 "weights run on the tile GEMV")
        for c in calls:
            del c["prepared"]
    del calls, groups
    torch.cuda.empty_cache()

    gate = dom[(14336, 4096)]
    roofline = dict(bound="hbm", achieved=gate["achieved"], peak=HBM_PEAK_GBS, unit="GB/s", frac=gate["frac"],
                    traffic=read_traffic(), kernel=gate["kernel"], avg_launch_us=gate["avg_launch_us"],
                    algorithmic_bytes_per_launch=gate["algorithmic_bytes_per_launch"],
                    timing="100 back-to-back launches in one HIP graph over >= 1 GB of rotating weight copies, "
                           "HIP events around the replay, median of 5, measured first in the run",
                    traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE on the eager 32-layer "
                                 "step, copy-calibrated)",
                    kernel_source_sha256_16=kernel_source_hash(), plan=gate["plan"],
                    down=dom[(4096, 14336)], step_average=step_avg)

    prefill = None if args.no_prefill else measure_prefill(torch, woq)
    configs = None if args.no_configs else measure_configs(torch, woq)
    sym16 = mxfp4 = zp4 = midsize = smallbatch = fewrows = None
    if not args.no_configs:
        from workloads import FEWROWS
        fewrows = dict(
            note="M = 2 to 4 on the decode shapes and 8192x28672: the row-streaming kernel, or the tile GEMV "
                 "on layers of at least 2^25 weights with K >= 8192",
            configs=measure_configs(torch, woq, cases=FEWROWS))
        from workloads import SMALLBATCH
        smallbatch = dict(
            note="M = 16 and 64 on the decode shapes: layers under 800 tiles of 16 rows run on the small-M path "
                 "with the activation slice in LDS (K split over workgroups, partials summed in order), "
                 "14336x4096 on the small-M kernel",
            configs=measure_configs(torch, woq, cases=SMALLBATCH))
        from workloads import MIDSIZE
        midsize = dict(
            note="M = 128 and 256 on the decode shapes: the tiled GEMM, its K split over workgroups where the "
                 "tiles alone would not fill the chip (k_splits in the plan), or the small-M kernel",
            configs=measure_configs(torch, woq, cases=MIDSIZE))
        from workloads import ZP4
        zp4 = dict(
            note="packed 4-bit zero points (woq_linear_int4_groups_zp4)",
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
                    m=1, group=GROUP, layers=args.layers, launches_per_step=len(abytes),
                    weight_bytes_per_step=wbytes, hbm_peak_frac=round(value / HBM_PEAK_GBS, 4),
                    graph=not args.no_graph, accumulate="f32",
                    tokens_per_s_linears_only=round(1.0 / (ms_per_step * 1e-3), 1) if args.layers == 32 else None),
        roofline=roofline, grouped=grouped, prepared=prepared, prefill=prefill, configs=configs,
        sym16=sym16, mxfp4=mxfp4, zp4=zp4, fewrows=fewrows, smallbatch=smallbatch, midsize=midsize,
        cpu_baseline=cpu,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
