"""Benchmark: Dion / Orth-Dion optimizer steps per second on the 3B-parameter
Llama-shaped stack (28 layers, 196 matrices: Q/O 3072x3072, K/V 3072x1024,
gate/up 3072x8192, down 8192x3072; float32 X, R, V; bfloat16 G) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--variant orth]
                    [--rank-div 4] [--extra] [--no-configs] [--no-cpu]

One step = one grouped libdion step over all 196 matrices (every phase of
the method).  Inputs are synthetic, drawn on the device before timing.
Prints one JSON line.  The per-phase durations come from HIP events the
library records on its own stream during the timed steps; the dominant
phase (one kernel launch) is reported against the MI355X roofline.  The
line also carries the same stack with the other arithmetic of the products
and at the other rank fraction, and both variants on the other workloads
(with the oracle beside each).  The CPU baseline is the float64 oracle on
a bounded sample of the same workload (four layers), scaled to the whole
stack.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12             # MI355X HBM3E bytes/s
MFMA_F32_PEAK = 157.3e12      # MI355X dense float32 matrix flop/s
MFMA_BF16_PEAK = 2516.6e12    # MI355X dense bfloat16 matrix flop/s
# Matrix-core operations per algorithmic flop of the three m x n x r
# products: 1 for float32 MFMA, 3 bfloat16 products for split-bfloat16.
MATH = {"f32": (MFMA_F32_PEAK, 1), "bf16x3": (MFMA_BF16_PEAK, 3)}
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "rank_orthonormalized_optimizer_dion_amd", "csrc")


def phase_model(mats, variant: str, eg: int):
    """Algorithmic flops and bytes of each phase, summed over the matrices.

    Per m x n matrix of rank r (eg = bytes per element of G):
      mv      2mnr flops;  reads G, R, V, writes P: (eg+4)mn + 4nr + 4mr
      orth_p  CholeskyQR of m x r (Gram, Cholesky and inverse, Q T^-1):
              4mr^2 + (4/3)r^3; reads P twice, writes U: 12mr bytes
      mtu     2mnr;  reads G, R, U, writes W: (eg+4)mn + 4mr + 4nr
      right   orth: 4nr^2 + (4/3)r^3, 12nr bytes; dion: 3nr flops, 12nr bytes
      update  4mnr;  reads X, G, R, U, Vbar, W, writes X, R: (16+eg)mn + 4mr + 8nr
    """
    f = dict.fromkeys(("mv", "orth_p", "mtu", "right", "update"), 0.0)
    b = dict.fromkeys(f, 0.0)
    for (m, n, r) in mats:
        mn = m * n
        f["mv"] += 2.0 * mn * r
        b["mv"] += (eg + 4) * mn + 4.0 * n * r + 4.0 * m * r
        f["orth_p"] += 4.0 * m * r * r + 4.0 / 3.0 * r ** 3
        b["orth_p"] += 12.0 * m * r
        f["mtu"] += 2.0 * mn * r
        b["mtu"] += (eg + 4) * mn + 4.0 * m * r + 4.0 * n * r
        if variant == "orth":
            f["right"] += 4.0 * n * r * r + 4.0 / 3.0 * r ** 3
            b["right"] += 12.0 * n * r
        else:
            f["right"] += 3.0 * n * r
            b["right"] += 12.0 * n * r
        f["update"] += 4.0 * mn * r
        b["update"] += (16 + eg) * mn + 4.0 * m * r + 8.0 * n * r
    return f, b


def step_model(mats, variant: str, eg: int):
    """Whole-step algorithmic flops and compulsory bytes (read X, G, R, V;
    write X, R, V)."""
    flops = 0.0
    bmin = 0.0
    for (m, n, r) in mats:
        flops += 8.0 * m * n * r + 4.0 * m * r * r + (4.0 * n * r * r if variant == "orth" else 3.0 * n * r)
        bmin += (16 + eg) * m * n + 8.0 * n * r
    return flops, bmin


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources that define and launch `kernel`: the headers, the
    host API and the kernel's own translation unit (the other kernel files
    do not change its code or its launches)."""
    files = sorted(os.listdir(KERNEL_SRC))
    units = [f for f in files if f.startswith("k_") and f.endswith(".hip")]
    own = [f for f in units
           if re.search(r"\bvoid\s+%s\s*\(" % re.escape(kernel),
                        open(os.path.join(KERNEL_SRC, f)).read())]
    h = hashlib.sha256()
    for f in files:
        if f.endswith((".hip", ".h")) and (f not in units or f in own):
            with open(os.path.join(KERNEL_SRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter runs (profiles/traffic_<kernel>_llama3b.json), or None
    when missing or taken on other kernel sources."""
    try:
        with open(os.path.join(PROFILES, f"traffic_{kernel}_llama3b.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("workload") != workload:
        return None
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def make_stack(wl, device):
    from workloads.device import DeviceMatrix
    out = []
    for s in wl.mats:
        out.append(DeviceMatrix(wl, s, device))
        if s.index % 28 == 27:
            print(f"[bench]   {s.index + 1} matrices ready", file=sys.stderr, flush=True)
    return out


def time_plan(dion, torch, mats, variant, steps, warmup, eta, beta, math="f32", phases=True):
    """Seconds per step over `steps` timed steps, and the per-phase HIP-event
    times of those same steps (phases=False: no phase events, for steps so
    short that recording them would be a visible part of the step)."""
    plan = dion.Plan([(d.X, d.G, d.R, d.V) for d in mats], variant, math=math)
    ws = plan.new_workspace()
    for _ in range(warmup):
        plan.step(eta, beta, ws)
    torch.cuda.synchronize()
    if phases:
        plan.timing_enable(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.step(eta, beta, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ph, n = plan.timing_read() if phases else ({}, 1)
    rc, per = dion.status(ws, plan.count)
    plan.close()
    del ws
    if rc != 0:
        raise RuntimeError(f"breakdown during the benchmark: {per}")
    return (t1 - t0) / steps, {k: v / n for k, v in ph.items()}


def time_sharded(dion, torch, whole, shards, variant, steps, warmup, eta, beta, math):
    """Seconds per step of a DION_SHARDED plan over `shards` (one GPU's row
    shards of the matrices `whole`), run as its three stages.  The two
    exchanges deliver what an all-reduce over all shards would: the global
    Gram matrix and W, taken once from stages 0 and 1 on the whole matrices
    (which do not touch X, R or V) and copied into every shard's buffers
    inside the timed step."""
    full = dion.Plan(whole, variant, math=math, sharded=True)
    wsf = full.new_workspace()
    full.shard_stage(0, eta, beta, wsf)
    gram = [full.shard_buffer(wsf, dion.SHARD_GRAM, i).clone() for i in range(full.count)]
    full.shard_stage(1, eta, beta, wsf)
    wsum = [full.shard_buffer(wsf, dion.SHARD_W, i).clone() for i in range(full.count)]
    full.close()
    del wsf
    plan = dion.Plan(shards, variant, math=math, sharded=True)
    ws = plan.new_workspace()
    gbuf = [plan.shard_buffer(ws, dion.SHARD_GRAM, i) for i in range(plan.count)]
    wbuf = [plan.shard_buffer(ws, dion.SHARD_W, i) for i in range(plan.count)]

    def one():
        plan.shard_stage(0, eta, beta, ws)
        for dst, src in zip(gbuf, gram):
            dst.copy_(src)
        plan.shard_stage(1, eta, beta, ws)
        for dst, src in zip(wbuf, wsum):
            dst.copy_(src)
        plan.shard_stage(2, eta, beta, ws)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rc, per = dion.status(ws, plan.count)
    plan.close()
    del ws
    if rc != 0:
        raise RuntimeError(f"breakdown during the sharded benchmark: {per}")
    return (t1 - t0) / steps


def roofline_of(phase: str, ms: float, f: dict, b: dict, traffic, math: str):
    """Roofline of one phase (one kernel launch on the 3B stack).

    achieved = algorithmic flops (or bytes) / duration, against the
    published peak of the arithmetic the kernel runs on: float32 MFMA, or
    bfloat16 MFMA for split-bfloat16 (which issues 3 bfloat16 products per
    algorithmic flop; the bound is decided on the executed intensity)."""
    t = ms * 1e-3
    peak, ops = MATH[math] if phase in ("mv", "mtu", "update") else (MFMA_F32_PEAK, 1)
    intensity = ops * f[phase] / b[phase]
    out = {}
    if intensity >= peak / HBM_PEAK:
        achieved = f[phase] / t / 1e12
        out = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak / 1e12, 1),
               "unit": "TFLOP/s", "frac": round(achieved / (peak / 1e12), 4), "traffic": traffic}
    else:
        achieved = b[phase] / t / 1e9
        out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
               "frac": round(achieved / 8000.0, 4), "traffic": traffic}
    out["mfma_ops_per_flop"] = ops
    return out


def _blas_info():
    blas, threads = "unknown BLAS", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads", 1) for i in libs), default=threads)
        if libs:
            blas = f"{libs[0].get('internal_api', 'blas')} {libs[0].get('version', '')}".strip()
    except Exception:
        pass
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return blas, int(threads), cpu


def oracle_seconds(wl, variant: str, indices, steps: int = 1, threads=None) -> float:
    """Seconds the float64 oracle takes for `steps` steps of the matrices
    `indices` of workload `wl` (inputs from the seeded numpy streams, drawn
    outside the timing); threads = None uses every BLAS thread."""
    import contextlib
    import numpy as np
    from oracle import dion_step
    from workloads import MatrixStream
    limit = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads, user_api="blas")
    eta, beta = float(np.float32(wl.eta)), float(np.float32(wl.beta))
    total = 0.0
    with limit:
        for i in indices:
            st = MatrixStream(wl, wl.mats[i])
            x, r, v = (a.astype(np.float64) for a in st.init())
            for t in range(steps):
                g = st.grad_f64(t)
                t0 = time.perf_counter()
                res = dion_step(x, g, r, v, eta, beta, variant)
                total += time.perf_counter() - t0
                x, r, v = res.X, res.R, res.V
    return total


def cpu_baseline(wl, variant: str, layers: int):
    """The float64 oracle on the first `layers` layer(s) of the stack (one
    step per matrix, inputs from the seeded numpy streams), scaled to the
    whole stack."""
    blas, threads, cpu = _blas_info()
    per_layer = sum(1 for s in wl.mats if s.layer == 0)
    sample = [s.index for s in wl.mats if s.layer < layers]
    total = oracle_seconds(wl, variant, sample)
    scale = len(wl.mats) / len(sample)
    return {"value": round(1.0 / (total * scale), 6), "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(sample)} of {len(wl.mats)} matrices (layers 0-{layers - 1}, "
                      f"{per_layer} roles each), one {variant} step each in numpy float64 "
                      f"({blas}, {cpu}), {total:.1f} s, scaled x{scale:g}"}


def step_roofline(shapes, variant: str, eg: int, math: str):
    """Whole-step roofline time: T_roof = max(B_min / HBM peak, F_alg /
    P_used), with every algorithmic flop at the matrix peak of the
    arithmetic the products run in (P_used = the float32 matrix peak, or a
    third of the bfloat16 peak for split-bfloat16, three bfloat16 products
    per float32 product).  Returns (T_roof, T_mfma, flops, compulsory bytes)."""
    flops, bmin = step_model(shapes, variant, eg)
    peak, ops = MATH[math]
    t_mfma = ops * flops / peak
    return max(bmin / HBM_PEAK, t_mfma), t_mfma, flops, bmin


def step_roofline_entry(shapes, variant: str, eg: int, math: str, sec: float) -> dict:
    t_roof, t_mfma, flops, bmin = step_roofline(shapes, variant, eg, math)
    peak, ops = MATH[math]
    return {"bound": "mfma" if t_mfma > bmin / HBM_PEAK else "hbm",
            "p_used_tflops": round(peak / ops / 1e12, 1),
            "algorithmic_tflop": round(flops / 1e12, 3),
            "compulsory_gb": round(bmin / 1e9, 3),
            "effective_gbps": round(bmin / sec / 1e9, 1),
            "effective_tflops": round(flops / sec / 1e12, 2),
            "frac": round(t_roof / sec, 4)}


# the other workloads: (label, config number, rank for config 5, timed steps,
# oracle sample: (matrix indices, steps), single-threaded oracle too)
OTHER_CONFIGS = (("single-256x128", 1, None, 1000, ((0,), 10), True),
                 ("planted-2048", 2, None, 40, ((0,), 3), True),
                 ("gpt160m-stack", 3, None, 30, (tuple(range(72)), 1), False),
                 ("mlp70b-r512", 5, 512, 10, ((0,), 1), False),
                 ("mlp70b-r2048", 5, 2048, 10, ((0,), 1), False))


def time_configs(dion, torch, dev, math: str, cpu: bool = True, only=None, variants=("orth", "dion")):
    """steps/s of both variants on every other workload, with the fraction
    of the whole-step roofline each reaches, and the float64 oracle's
    steps/s on the same workload (all BLAS threads; also one thread for the
    single matrices).  only: one workload's label."""
    from workloads import config
    from workloads.device import DeviceMatrix
    out = {}
    blas, threads, cpu_name = _blas_info()
    for label, num, r, steps, (sample, osteps), single in OTHER_CONFIGS:
        if only is not None and label != only:
            continue
        wl = config(num, r=r) if r else config(num)
        print(f"[bench] {wl.name}", file=sys.stderr, flush=True)
        mats = [DeviceMatrix(wl, s, dev) for s in wl.mats]
        torch.cuda.synchronize()
        shapes = [(s.m, s.n, s.r) for s in wl.mats]
        eg = 2 if wl.g_dtype == "bf16" else 4
        for var in variants:
            sec, _ = time_plan(dion, torch, mats, var, steps, 3, wl.eta, wl.beta, math,
                               phases=False)
            entry = {"workload": wl.name, "steps_per_s": round(1 / sec, 2),
                     "ms_per_step": round(sec * 1e3, 4),
                     "step_roofline": step_roofline_entry(shapes, var, eg, math, sec)}
            if cpu and var == "orth":
                scale = len(wl.mats) / len(sample)
                t = oracle_seconds(wl, var, sample, osteps) * scale / osteps
                entry["cpu_baseline"] = {"value": round(1.0 / t, 4), "unit": "steps/s",
                                         "cores": threads, "kind": "oracle",
                                         "sample": f"{len(sample)} of {len(wl.mats)} matrices, "
                                                   f"{osteps} step(s), numpy float64 ({blas}, "
                                                   f"{cpu_name})"}
                if single:
                    t1 = oracle_seconds(wl, var, sample, osteps, threads=1) * scale / osteps
                    entry["cpu_baseline_1thread"] = {"value": round(1.0 / t1, 4),
                                                     "unit": "steps/s", "cores": 1}
            out[f"{label}_{var}"] = entry
        del mats
        torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--variant", choices=("orth", "dion"), default="orth")
    ap.add_argument("--math", choices=("f32", "bf16x3"), default="bf16x3",
                    help="arithmetic of the three m x n x r products: split-bfloat16 "
                         "(default) or float32 MFMA")
    ap.add_argument("--rank-div", type=int, choices=(4, 16), default=4)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--extra", action="store_true",
                    help="also time the other variant at both rank fractions and one GPU's "
                         "share of a row-sharded stack")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the main setting (no other arithmetic or rank fraction; "
                         "for profiling runs)")
    ap.add_argument("--only", choices=[c[0] for c in OTHER_CONFIGS], default=None,
                    help="time only this workload of --configs (variant --variant), without "
                         "the 3B stack: for profiling one workload")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the other workloads (single matrices, the 160M stack, the 70B "
                         "MLP matrix), which the line otherwise carries under \"configs\" "
                         "with both variants and their oracle baselines")
    ap.add_argument("--cpu-layers", type=int, default=4)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (a known byte "
                         "count for scaling hardware traffic counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the Dion step here runs on a single MI355X and "
              "has no multi-GPU path (a row-sharded step's per-shard stages are the "
              "DION_SHARDED plans, with the Gram matrix and W as the exchange points).",
              file=sys.stderr)
        return 2

    import torch
    import rank_orthonormalized_optimizer_dion_amd as dion
    from workloads import config
    dion.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        res = time_configs(dion, torch, dev, args.math, cpu=not args.no_cpu, only=args.only,
                           variants=(args.variant,))
        print(json.dumps({"configs": res}))
        return 0

    wl = config(4, args.rank_div, layers=args.layers)
    print(f"[bench] generating {wl.name}: {wl.count} matrices on the device", file=sys.stderr,
          flush=True)
    mats = make_stack(wl, dev)
    torch.cuda.synchronize()
    print("[bench] inputs ready; timing", file=sys.stderr, flush=True)
    shapes = [(s.m, s.n, s.r) for s in wl.mats]
    eg = 2
    sec, phases = time_plan(dion, torch, mats, args.variant, args.steps, args.warmup,
                            wl.eta, wl.beta, args.math)
    f, b = phase_model(shapes, args.variant, eg)
    dom = max(phases, key=phases.get)
    # kernels of each phase on this stack (split-bfloat16: the 256 x 256
    # product tiles at r = 1/4, where rows and ranks are multiples of 256;
    # at r = 1/16 the 256 x 192 tiles of its r = 192 classes, which carry
    # nearly all of the products)
    names = {"mv": "k_mv", "orth_p": "orth(P)", "mtu": "k_mtu", "right": "right factor",
             "update": "k_epi"}
    if args.math == "bf16x3":
        wide = args.rank_div == 16
        names.update(mv="k_mv3s" if wide else "k_mv3b", mtu="k_mtu3s" if wide else "k_mtu3b",
                     update="k_epi3b")
    kernel = names[dom]
    traffic = measured_traffic(kernel, wl.name) if kernel.startswith("k_") else None
    roof = roofline_of(dom, phases[dom], f, b, traffic, args.math)
    roof["kernel"] = kernel
    out = {
        "metric": "Dion/Orth-Dion steps/sec + effective HBM GB/s (% roofline), 3B-shaped stack",
        "value": round(1.0 / sec, 4),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "bf16x3" if args.math == "bf16x3" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": wl.count, "variant": args.variant,
                   "math": args.math,
                   "g_dtype": "bf16", "state_dtype": "f32", "layers": args.layers,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "step_roofline": step_roofline_entry(shapes, args.variant, eg, args.math, sec),
        "phase_ms": {k: round(v, 3) for k, v in phases.items()},
    }
    if args.main_only:
        print(json.dumps(out), flush=True)
        return 0
    # the same stack with the other arithmetic and at the other rank
    # fraction, in the default line too (fewer timed steps)
    other_math = "f32" if args.math == "bf16x3" else "bf16x3"
    sec_m, ph_m = time_plan(dion, torch, mats, args.variant, max(3, args.steps // 2), 1,
                            wl.eta, wl.beta, other_math)
    out[f"{other_math}_products"] = {
        "steps_per_s": round(1 / sec_m, 4),
        "step_roofline_frac": step_roofline_entry(shapes, args.variant, eg, other_math, sec_m)["frac"],
        "p_used_tflops": round(MATH[other_math][0] / MATH[other_math][1] / 1e12, 1),
        "phase_ms": {k: round(v, 3) for k, v in ph_m.items()}}
    extra = {}
    if args.extra:
        other = "dion" if args.variant == "orth" else "orth"
        sec2, ph2 = time_plan(dion, torch, mats, other, max(3, args.steps // 2), 1, wl.eta,
                              wl.beta, args.math)
        extra[f"{other}_r1/{args.rank_div}"] = {
            "steps_per_s": round(1 / sec2, 4),
            "step_roofline_frac": step_roofline_entry(shapes, other, eg, args.math, sec2)["frac"],
            "phase_ms": {k: round(v, 3) for k, v in ph2.items()}}
        # one GPU's share of an 8-way row-sharded (FSDP) stack: rows
        # [0, m/8) of every matrix, stepped in the three DION_SHARDED stages
        whole = [(d.X, d.G, d.R, d.V) for d in mats]
        shard = [(d.X[: d.X.shape[0] // 8], d.G[: d.G.shape[0] // 8], d.R[: d.R.shape[0] // 8],
                  d.V) for d in mats]
        sec4 = time_sharded(dion, torch, whole, shard, args.variant, max(3, args.steps // 2), 1,
                            wl.eta, wl.beta, args.math)
        extra[f"{args.variant}_r1/{args.rank_div}_shard1of8"] = {
            "steps_per_s": round(1 / sec4, 4), "rows": "m/8 of every matrix",
            "exchange": "the all-reduced Gram matrix and W landed by device copies"}
        del shard, whole
    # the other rank fraction, in the default line too
    div2 = 16 if args.rank_div == 4 else 4
    wl2 = config(4, div2, layers=args.layers)
    for d, s2 in zip(mats, wl2.mats):
        d.reset_rank(s2.r)
    torch.cuda.synchronize()
    shapes2 = [(s2.m, s2.n, s2.r) for s2 in wl2.mats]
    sec_r, ph_r = time_plan(dion, torch, mats, args.variant, args.steps, 1, wl.eta, wl.beta,
                            args.math)
    out[f"{args.variant}_r1/{div2}"] = {
        "steps_per_s": round(1 / sec_r, 4),
        "step_roofline": step_roofline_entry(shapes2, args.variant, eg, args.math, sec_r),
        "phase_ms": {k: round(v, 3) for k, v in ph_r.items()}}
    if args.extra:
        other = "dion" if args.variant == "orth" else "orth"
        sec3, ph3 = time_plan(dion, torch, mats, other, max(3, args.steps // 2), 1, wl.eta,
                              wl.beta, args.math)
        extra[f"{other}_r1/{div2}"] = {
            "steps_per_s": round(1 / sec3, 4),
            "step_roofline_frac": step_roofline_entry(shapes2, other, eg, args.math, sec3)["frac"],
            "phase_ms": {k: round(v, 3) for k, v in ph3.items()}}
        out["extra"] = extra
    del mats
    torch.cuda.empty_cache()
    if args.configs:
        out["configs"] = time_configs(dion, torch, dev, args.math, cpu=not args.no_cpu)
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.variant, args.cpu_layers)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
