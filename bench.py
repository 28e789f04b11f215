"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--no-cpu-baseline]

A step is one pass of the whole path -- forward (attn_fwd) and backward
(attn_bwd's three stages) -- over one batch of seeded synthetic input, once
without and once with the causal mask, on the hidden-size-2048 attention layer
with head dimension 128: B=4, N=4096, H=16, d=128, bf16, scale 1/sqrt(128).
Throughput counts 4*B*H*N^2*d FLOPs per forward (halved when causal) and 2.5x
that per backward.  Inputs are resident in HBM before the timed region.

Prints one JSON line.  Besides the throughput it carries
  roofline      for the dominant kernel (the non-causal backward main kernel):
                its algorithmic FLOPs / its mean duration from HIP events on its
                own stream, against the dense bf16 MFMA peak; `traffic` is the HBM
                bytes per launch measured with rocprofv3 counters for the current
                kernel source (null when the source changed since);
  targets       forward and backward TFLOP/s at the points the forward target
                is stated for (d = 128, N = 4096 and 16384) and at d = 64
                (N = 4096 and 16384), causal and not, each after its own
                warm-up (HIP events, median of 10);
  cpu_baseline  the CPU fp64 oracle timed on a bounded sample of the same
                workload on this host: whole (batch, head) slices, one per
                worker process over the host's cores, with the core count,
                CPU model and BLAS threads recorded;
  blocksparse   block-sparse attention (attn_fwd_blocksparse /
                attn_bwd_blocksparse) on its own workload -- hidden 2048,
                d = 128, B = 1, N = 16384, one block mask with every diagonal
                block and a seeded 25% of the others -- timed outside the step:
                TFLOP/s over the computed blocks and the speed-up over the
                dense kernels on the same shape;
  shard         rectangular attention (attn_fwd_rect / attn_bwd_rect) on one
                device's share of a causal 65536-token sequence split 8 ways:
                the last 8192 queries against all 65536 keys, B = 1, H = 8,
                d = 128 (FLOPs over the allowed query-key pairs); and the
                split-KV forward (attn_fwd_splitkv) on a short-query shape,
                128 queries against 65536 keys, B = 1, H = 32, d = 128,
                against the unsplit kernel;
  secondary_ceilings  exponential and LDS-read throughput measured by
                libattn_probe.so, beside what the non-causal forward needs;
  mfma_ceiling  the sustained MFMA rate measured on this part by
                libattn_probe.so (random and constant bf16 operands); the
                roofline entry also gives the dominant kernel's fraction of it;
  standard      standard attention (attn_fwd_standard / attn_bwd_standard),
                which writes the N x N scores and probabilities to HBM, against
                the tiled kernels on the step's shape: times, speed-ups, extra
                device memory and algorithmic HBM bytes of each; `by_N`: the
                speed-ups over the hidden-2048, d = 128 sequence-length sweep
                (B * N = 16384).
--sweep also prints per-workload forward/backward TFLOP/s for every full-size
configuration to stderr; --oracle-sweep times the CPU oracle (fwd, fwd+bwd)
on every full-size configuration and exits.
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

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
WORKLOAD = dict(name="hidden2048_d128", b=4, n=4096, h=16, d=128)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_dkdv_traffic_B4_N4096_H16_d128.json")
KERNEL_SOURCES = ("exact_io_aware_75_amd/csrc/attn_bwd.hip", "exact_io_aware_75_amd/csrc/attn_common.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def fwd_flops(b, n, h, d, causal):
    f = 4.0 * b * h * n * n * d
    return f / 2 if causal else f


def load_traffic():
    """HBM bytes per launch of the backward main kernel, if measured for this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return 0


def _pool_workers() -> int:
    """Worker processes for the oracle: the host cores this process may use,
    capped by OMP_NUM_THREADS when it is set (the CPU share of the machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _oracle_slice(task):
    """One whole (batch, head) slice of the oracle, fwd then bwd (a worker
    process with one BLAS thread).  Returns (fwd seconds, fwd+bwd seconds).
    ``rows`` < N times only the first ``rows`` queries against all keys
    (non-causal: the oracle forms the full score rows either way)."""
    import numpy as np

    import oracle
    from exact_io_aware_75_amd import inputs as gen

    n, d, causal, seed, rows = task
    x = gen.make_inputs(1, n, 1, 1, d, "bf16", cfg_id=3, seed=seed)
    q, k, v, do = (x[t][0, :, 0] for t in ("q", "k", "v", "do"))
    if rows < n:
        q, do, causal = q[:rows], do[:rows], False
    scale = 1.0 / np.sqrt(d)
    t0 = time.perf_counter()
    oracle.attention_head_fwd(q, k, v, causal, scale)
    t1 = time.perf_counter()
    oracle.attention_head_bwd(q, k, v, do, causal, scale)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t0


def _oracle_pool(workers):
    import multiprocessing as mp

    # one BLAS thread per worker process; set before the children start
    saved = {k_: os.environ.get(k_) for k_ in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k_ in saved:
        os.environ[k_] = "1"
    try:
        pool = mp.get_context("spawn").Pool(workers)
    finally:
        for k_, v_ in saved.items():
            if v_ is None:
                os.environ.pop(k_, None)
            else:
                os.environ[k_] = v_
    return pool


def cpu_baseline(seconds: float):
    """Time the fp64 oracle on whole (batch, head) slices of the workload, one
    slice per worker process over the host's cores, for about ``seconds`` of
    wall clock."""
    w = WORKLOAD
    n, d = w["n"], w["d"]
    workers = _pool_workers()
    pool = _oracle_pool(workers)
    try:
        pool.map(_oracle_slice, [(256, d, False, 0, 256)] * workers)  # start-up and imports, untimed
        flops = 0.0
        slices = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            tasks = [(n, d, (slices + i) % 2 == 1, 1000 + slices + i, n) for i in range(workers)]
            pool.map(_oracle_slice, tasks)
            flops += sum(3.5 * fwd_flops(1, n, 1, d, t[2]) for t in tasks)
            slices += len(tasks)
        elapsed = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{slices} (batch, head) slices of N={n}, d={d} (alternately non-causal and causal), "
                  f"fwd+bwd in fp64, {workers} worker processes x 1 BLAS thread, {elapsed:.1f} s wall; "
                  f"FLOPs counted as for the GPU (causal halved, although the oracle forms every score)",
        "host": {"os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(),
                 "blas_threads_in_parent": _blas_threads(), "workers": workers},
    }


def oracle_sweep(max_rows: int = 4096):
    """Wall clock of the fp64 oracle per full-size workload, fwd and fwd+bwd,
    on the host's cores (one (batch, head) slice per worker).  Slices of more
    than ``max_rows`` queries are timed on their first ``max_rows`` rows
    against all keys and scaled by N / max_rows (the oracle's cost is linear
    in the rows); those points are marked extrapolated."""
    from exact_io_aware_75_amd import configs

    workers = _pool_workers()
    pool = _oracle_pool(workers)
    out = []
    try:
        pool.map(_oracle_slice, [(256, 64, False, 0, 256)] * workers)
        for s in configs.all_shapes()[1:]:
            slices = s.b * s.hq
            rows = min(s.n, max_rows)
            tasks = [(s.n, s.d, s.causal, 7 + i, rows) for i in range(min(workers, slices))]
            t0 = time.perf_counter()
            res = pool.map(_oracle_slice, tasks)
            wall = time.perf_counter() - t0
            rounds = -(-slices // workers)
            scale_rows = s.n / rows
            fwd_share = sum(r[0] for r in res) / max(sum(r[1] for r in res), 1e-30)
            total = wall * rounds * scale_rows
            rec = {"workload": s.name, "B": s.b, "N": s.n, "Hq": s.hq, "Hkv": s.hkv, "d": s.d,
                   "causal": s.causal, "fwd_s": round(total * fwd_share, 2), "fwd_bwd_s": round(total, 2),
                   "workers": workers, "extrapolated": rows < s.n or rounds > 1,
                   "how": f"{len(tasks)} slices of {rows}/{s.n} rows in parallel took {wall:.2f} s; "
                          f"x {rounds} rounds of {workers} slices" + (f" x {scale_rows:g} rows" if rows < s.n else "")}
            print("oracle " + json.dumps(rec), file=sys.stderr, flush=True)
            out.append(rec)
    finally:
        pool.close()
        pool.join()
    return out


def run(args):
    import numpy as np
    import torch

    import exact_io_aware_75_amd as ea
    from exact_io_aware_75_amd import inputs as gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOAD
    b, n, h, d = w["b"], w["n"], w["h"], w["d"]
    scale = 1.0 / float(np.sqrt(d))
    x = gen.make_inputs(b, n, h, h, d, "bf16", cfg_id=3)
    q, k, v, do = (gen.to_torch(x[t], "bf16", dev) for t in ("q", "k", "v", "do"))
    del x
    o = torch.empty_like(q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(b, n, h, h, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    stages = ("attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq")
    ops = []  # (label, callable)
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        ops.append((f"fwd_{tag}", lambda c=causal: ea.attn_fwd(q, k, v, o, lse, c, scale, stream)))
        for st in stages:
            ops.append((f"{st}_{tag}", lambda c=causal, s=st: ea.attn_bwd(
                q, k, v, o, do, lse, dq, dk, dv, ws, c, scale, stream, stage=s)))

    def step(events=None):
        for i, (_, fn) in enumerate(ops):
            if events is not None:
                events[i].record(stream)
            fn()
        if events is not None:
            events[len(ops)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dur = {label: [] for label, _ in ops}
    for s in range(args.steps):
        for i, (label, _) in enumerate(ops):
            dur[label].append(evs[s][i].elapsed_time(evs[s][i + 1]))
    mean = {k_: float(np.mean(v_)) for k_, v_ in dur.items()}

    flops_step = sum(3.5 * fwd_flops(b, n, h, d, c) for c in (False, True))
    ms_per_step = wall / args.steps * 1e3
    value = flops_step / (ms_per_step / 1e3) / 1e12
    fwd_tf = {c: fwd_flops(b, n, h, d, c) / (mean[f"fwd_{'causal' if c else 'noncausal'}"] / 1e3) / 1e12
              for c in (False, True)}
    bwd_tf = {}
    for c in (False, True):
        tag = "causal" if c else "noncausal"
        t_ms = sum(mean[f"{st}_{tag}"] for st in stages)
        bwd_tf[c] = 2.5 * fwd_flops(b, n, h, d, c) / (t_ms / 1e3) / 1e12

    # Dominant kernel: the non-causal dK/dV kernel.  Its algorithmic work is
    # four N x N x d products per (batch, head): S, dP, dV, dK = 8 B H N^2 d FLOP.
    main_ms = mean["attn_bwd_dkdv_noncausal"]
    achieved = 8.0 * b * h * n * n * d / (main_ms / 1e3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": "attn_bwd_dkdv_kernel<bf16, d=128, non-causal>",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": load_traffic(),
        "mean_ms": round(main_ms, 4),
    }
    line = {
        "metric": "attention fwd/bwd TFLOP/s (bf16, causal/non, d=64/128) and % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1), rounded to bf16)",
        "config": {"workload": "attention layer, hidden size 2048, head dim 128: fwd+bwd, non-causal and causal",
                   "B": b, "N": n, "H": h, "d": d, "scale": "1/sqrt(d)"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": {"noncausal": round(fwd_tf[False], 2), "causal": round(fwd_tf[True], 2)},
        "bwd_tflops": {"noncausal": round(bwd_tf[False], 2), "causal": round(bwd_tf[True], 2)},
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in mean.items()},
        "roofline": roofline,
    }
    if args.targets:
        line["targets"] = targets_measure()
    if args.sparse:
        line["blocksparse"] = blocksparse_measure()
        line["shard"] = shard_measure()
    if args.standard:
        line["standard"] = standard_measure()
    ceil = mfma_ceiling()
    line["mfma_ceiling"] = ceil
    line["secondary_ceilings"] = secondary_ceilings(fwd_tf[False], d)
    roofline["frac_of_measured_ceiling"] = round(achieved / ceil["random_bf16_tflops"], 4)
    if args.targets:
        # the same points against the sustained MFMA rate this part showed in
        # this run (boxes differ in clock by more than 10%)
        for pt in line["targets"]["points"].values():
            pt["fwd_frac_of_measured_ceiling"] = round(pt["fwd_tflops"] / ceil["random_bf16_tflops"], 4)
            pt["bwd_frac_of_measured_ceiling"] = round(pt["bwd_tflops"] / ceil["random_bf16_tflops"], 4)
    if args.sweep:
        sweep()
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def measure_shape(s, reps=10, seed=0):
    """Forward and backward of one workload (torch.randn inputs rounded to
    bf16): HIP events on the launch stream, median of ``reps`` launches after
    at least 100 ms of warm-up launches of the same workload, so that the
    clock state left by the previous workload has passed.  Returns
    {"fwd": (ms, TFLOP/s), "bwd": (ms, TFLOP/s)}."""
    import numpy as np
    import torch

    import exact_io_aware_75_amd as ea

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    mk = lambda hh: torch.randn(s.b, s.n, hh, s.d, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
    q, k, v, do = mk(s.hq), mk(s.hkv), mk(s.hkv), mk(s.hq)
    o, lse = torch.empty_like(q), torch.empty((s.b, s.hq, s.n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(s.b, s.n, s.hq, s.hkv, s.d), dtype=torch.uint8, device=dev)
    sc = 1.0 / float(np.sqrt(s.d))
    res = {}
    for name, fn in (("fwd", lambda: ea.attn_fwd(q, k, v, o, lse, s.causal, sc, stream)),
                     ("bwd", lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, s.causal, sc, stream))):
        t0 = time.perf_counter()
        n_warm = 0
        while n_warm < 3 or time.perf_counter() - t0 < 0.1:
            fn()
            n_warm += 1
            if n_warm % 8 == 0:
                stream.synchronize()
        stream.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        t = float(np.median(ts))
        fl = s.fwd_flops() * (2.5 if name == "bwd" else 1.0)
        res[name] = (t, fl / (t / 1e3) / 1e12)
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


# The points the forward target is stated for (d = 128, N >= 4k) and the
# d = 64 half of the metric, on the hidden-2048 layer (B * N = 16384).
TARGET_POINTS = ((128, 4096), (128, 16384), (64, 4096), (64, 16384))


def targets_measure():
    from exact_io_aware_75_amd import configs

    out = {}
    for d, n in TARGET_POINTS:
        for c in (False, True):
            s = configs.hidden2048(d, n, c)
            r = measure_shape(s)
            out[f"d{d}_n{n}_{'causal' if c else 'noncausal'}"] = {
                "B": s.b, "N": s.n, "H": s.hq, "d": s.d, "causal": c,
                "fwd_ms": round(r["fwd"][0], 4), "fwd_tflops": round(r["fwd"][1], 1),
                "fwd_frac_of_peak": round(r["fwd"][1] / PEAK_BF16_TFLOPS, 4),
                "bwd_ms": round(r["bwd"][0], 4), "bwd_tflops": round(r["bwd"][1], 1),
                "bwd_frac_of_peak": round(r["bwd"][1] / PEAK_BF16_TFLOPS, 4)}
    return {"what": "hidden-2048 layer (B * N = 16384, H = 2048 / d), bf16, scale 1/sqrt(d); HIP events on the "
                    "launch stream, median of 10 after >= 100 ms of warm-up launches of the same workload; "
                    "backward = 2.5 x forward FLOPs, causal halved",
            "points": out}


def sweep():
    """Per-configuration forward / backward throughput for every full-size
    workload (``measure_shape``), printed to stderr."""
    from exact_io_aware_75_amd import configs

    for s in configs.all_shapes()[1:]:
        res = measure_shape(s)
        print(f"sweep {s.name:16s} B={s.b:2d} N={s.n:6d} Hq={s.hq:2d} Hkv={s.hkv:2d} d={s.d:3d} causal={int(s.causal)}  "
              f"fwd {res['fwd'][0]:8.3f} ms {res['fwd'][1]:7.1f} TFLOP/s ({100 * res['fwd'][1] / PEAK_BF16_TFLOPS:4.1f}%)  "
              f"bwd {res['bwd'][0]:8.3f} ms {res['bwd'][1]:7.1f} TFLOP/s ({100 * res['bwd'][1] / PEAK_BF16_TFLOPS:4.1f}%)",
              file=sys.stderr, flush=True)


def _median_ms(fn, stream, reps=10):
    import numpy as np
    import torch

    for _ in range(3):
        fn()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def blocksparse_measure():
    """Block-sparse forward / backward on the block-sparse workload, against
    the dense kernels on the same shape (HIP events, median of 10)."""
    import numpy as np
    import torch

    import exact_io_aware_75_amd as ea
    from exact_io_aware_75_amd import configs
    from exact_io_aware_75_amd import inputs as gen

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s0 = configs.blocksparse(False)
    mask_np = gen.make_block_mask(1, s0.n, configs.BLOCKSPARSE_DENSITY, cfg_id=s0.cfg_id)
    mask = torch.from_numpy(mask_np).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    mk = lambda hh: torch.randn(s0.b, s0.n, hh, s0.d, device=dev, generator=g).to(torch.bfloat16)  # noqa: E731
    q, k, v, do = mk(s0.hq), mk(s0.hkv), mk(s0.hkv), mk(s0.hq)
    o, lse = torch.empty_like(q), torch.empty((s0.b, s0.hq, s0.n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(s0.b, s0.n, s0.hq, s0.hkv, s0.d), dtype=torch.uint8, device=dev)
    sc = 1.0 / float(np.sqrt(s0.d))
    out = {"workload": f"{s0.name}: B={s0.b} N={s0.n} H={s0.hq} d={s0.d} bf16, 128x128 blocks",
           "mask": f"diagonal + seeded {configs.BLOCKSPARSE_DENSITY:.0%} of the other blocks, shared by all heads",
           "density": round(float(mask_np.mean()), 4), "unit": "TFLOP/s (computed blocks only)"}
    for causal in (False, True):
        s = configs.blocksparse(causal)
        fl = configs.masked_fwd_flops(s, mask_np)
        t = {}
        for kind, bm in (("sparse", mask), ("dense", None)):
            t[f"fwd_{kind}"] = _median_ms(lambda: ea.attn_fwd(q, k, v, o, lse, causal, sc, stream, block_mask=bm), stream)
            t[f"bwd_{kind}"] = _median_ms(lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal, sc,
                                                              stream, block_mask=bm), stream)
        tag = "causal" if causal else "noncausal"
        out[tag] = {
            "flop_fraction": round(fl / s.fwd_flops(), 4),
            "fwd_ms": round(t["fwd_sparse"], 4), "bwd_ms": round(t["bwd_sparse"], 4),
            "fwd_tflops": round(fl / (t["fwd_sparse"] / 1e3) / 1e12, 1),
            "bwd_tflops": round(2.5 * fl / (t["bwd_sparse"] / 1e3) / 1e12, 1),
            "dense_fwd_ms": round(t["fwd_dense"], 4), "dense_bwd_ms": round(t["bwd_dense"], 4),
            "speedup_fwd": round(t["fwd_dense"] / t["fwd_sparse"], 2),
            "speedup_bwd": round(t["bwd_dense"] / t["bwd_sparse"], 2),
        }
    del q, k, v, do, o, lse, dq, dk, dv, ws, mask
    torch.cuda.empty_cache()
    return out


def shard_measure():
    """Rectangular forward / backward on the context-parallel shard shape."""
    import numpy as np
    import torch

    import exact_io_aware_75_amd as ea

    b, nq, nk, h, d = 1, 8192, 65536, 8, 128
    off = nk - nq
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    mk = lambda n: torch.randn(b, n, h, d, device=dev, generator=g).to(torch.bfloat16)  # noqa: E731
    q, do, k, v = mk(nq), mk(nq), mk(nk), mk(nk)
    o, lse = torch.empty_like(q), torch.empty((b, h, nq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(b, nq, h, h, d), dtype=torch.uint8, device=dev)
    sc = 1.0 / float(np.sqrt(d))
    pairs = float(np.minimum(nk, np.maximum(0, np.arange(nq) + off + 1)).sum())
    fl = 4.0 * d * b * h * pairs
    t_f = _median_ms(lambda: ea.attn_fwd(q, k, v, o, lse, True, sc, stream, causal_offset=off), stream)
    t_b = _median_ms(lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, True, sc, stream,
                                         causal_offset=off), stream)
    del q, do, k, v, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    out = {"workload": f"last of 8 causal shards of a 65536-token sequence: B={b} Nq={nq} Nk={nk} H={h} d={d} "
                       f"bf16, causal offset {off}",
           "unit": "TFLOP/s (allowed query-key pairs)",
           "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
           "fwd_tflops": round(fl / (t_f / 1e3) / 1e12, 1),
           "bwd_tflops": round(2.5 * fl / (t_b / 1e3) / 1e12, 1)}
    # split-KV on a short-query shape (one 128-row block per head)
    b, nq, nk, h, splits = 1, 128, 65536, 32, 16
    q, k, v = mk_shape(g, dev, b, nq, h, d), mk_shape(g, dev, b, nk, h, d), mk_shape(g, dev, b, nk, h, d)
    o, lse = torch.empty_like(q), torch.empty((b, h, nq), dtype=torch.float32, device=dev)
    ws = torch.empty(ea.attn_fwd_splitkv_workspace_bytes(b, nq, h, d, splits), dtype=torch.uint8, device=dev)
    fl = 4.0 * d * b * h * nq * nk
    t_1 = _median_ms(lambda: ea.attn_fwd(q, k, v, o, lse, False, sc, stream), stream)
    t_s = _median_ms(lambda: ea.attn_fwd_splitkv(q, k, v, o, lse, ws, False, sc, splits, stream), stream)
    out["splitkv"] = {"workload": f"B={b} Nq={nq} Nk={nk} H={h} d={d} bf16, non-causal, {splits} splits",
                      "fwd_ms": round(t_s, 4), "fwd_tflops": round(fl / (t_s / 1e3) / 1e12, 1),
                      "unsplit_fwd_ms": round(t_1, 4), "speedup": round(t_1 / t_s, 2)}
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return out


def standard_measure():
    """Standard (materialising) attention against the tiled kernels on the
    benchmark workload: time (HIP events, median of 10), device memory beyond
    the inputs and outputs, and the algorithmic HBM bytes of each."""
    import numpy as np
    import torch

    import exact_io_aware_75_amd as ea

    w = WORKLOAD
    b, n, h, d = w["b"], w["n"], w["h"], w["d"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    q, k, v, do = (mk_shape(g, dev, b, n, h, d) for _ in range(4))
    o, lse = torch.empty_like(q), torch.empty((b, h, n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    std_ws = ea.attn_standard_workspace_bytes(b, n, h, h, d)
    ws_s = torch.empty(std_ws, dtype=torch.uint8, device=dev)
    ws_t = torch.empty(ea.attn_bwd_workspace_bytes(b, n, h, h, d), dtype=torch.uint8, device=dev)
    sc = 1.0 / float(np.sqrt(d))
    bh, nd, nn = b * h, n * d, n * n
    out = {"workload": f"B={b} N={n} H={h} d={d} bf16 (the step's shape)",
           "what": "standard attention: S = scale QK^T (fp32) and P = softmax(S) written to HBM in full, "
                   "O = PV; backward reads the stored P (dV = P^T dO, dP = dO V^T, dS, dQ, dK)",
           "extra_memory_bytes": {"standard": std_ws, "tiled": int(ws_t.numel()) + 4 * bh * n,
                                  "ratio": round(std_ws / (ws_t.numel() + 4 * bh * n), 1)},
           # S write + read, P write + read (fwd); P read twice, dP write + read, dS write + 2 reads (bwd)
           "algorithmic_hbm_bytes": {"standard_fwd": bh * (12 * nn + 8 * nd + 4 * n),
                                     "standard_bwd": bh * (18 * nn + 14 * nd),
                                     "tiled_fwd": bh * (8 * nd + 4 * n), "tiled_bwd": bh * (16 * nd + 8 * n)}}
    for causal in (False, True):
        t_sf = _median_ms(lambda: ea.attn_fwd_standard(q, k, v, o, lse, ws_s, causal, sc, stream), stream)
        t_sb = _median_ms(lambda: ea.attn_bwd_standard(q, k, v, do, dq, dk, dv, ws_s, causal, sc, stream), stream)
        t_tf = _median_ms(lambda: ea.attn_fwd(q, k, v, o, lse, causal, sc, stream), stream)
        t_tb = _median_ms(lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws_t, causal, sc, stream), stream)
        hb = out["algorithmic_hbm_bytes"]
        out["causal" if causal else "noncausal"] = {
            "standard_fwd_ms": round(t_sf, 4), "standard_bwd_ms": round(t_sb, 4),
            "tiled_fwd_ms": round(t_tf, 4), "tiled_bwd_ms": round(t_tb, 4),
            "speedup_fwd": round(t_sf / t_tf, 2), "speedup_bwd": round(t_sb / t_tb, 2),
            "speedup_fwd_bwd": round((t_sf + t_sb) / (t_tf + t_tb), 2),
            "standard_fwd_hbm_GBps": round(hb["standard_fwd"] / (t_sf / 1e3) / 1e9, 1),
            "standard_bwd_hbm_GBps": round(hb["standard_bwd"] / (t_sb / 1e3) / 1e9, 1)}
    del q, k, v, do, o, lse, dq, dk, dv, ws_s, ws_t
    torch.cuda.empty_cache()
    # the same comparison over the sequence lengths of the hidden-2048, d = 128
    # sweep (B * N = 16384 tokens, H = 16), median of 5 launches each
    out["by_N"] = []
    for n2 in (1024, 2048, 8192, 16384):
        b2 = 16384 // n2
        q, k, v, do = (mk_shape(g, dev, b2, n2, h, d) for _ in range(4))
        o, lse = torch.empty_like(q), torch.empty((b2, h, n2), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        sw = ea.attn_standard_workspace_bytes(b2, n2, h, h, d)
        ws_s = torch.empty(sw, dtype=torch.uint8, device=dev)
        ws_t = torch.empty(ea.attn_bwd_workspace_bytes(b2, n2, h, h, d), dtype=torch.uint8, device=dev)
        row = {"N": n2, "B": b2, "standard_workspace_GB": round(sw / 1e9, 2)}
        for causal in (False, True):
            t_sf = _median_ms(lambda: ea.attn_fwd_standard(q, k, v, o, lse, ws_s, causal, sc, stream), stream, reps=5)
            t_sb = _median_ms(lambda: ea.attn_bwd_standard(q, k, v, do, dq, dk, dv, ws_s, causal, sc, stream), stream,
                              reps=5)
            t_tf = _median_ms(lambda: ea.attn_fwd(q, k, v, o, lse, causal, sc, stream), stream, reps=5)
            t_tb = _median_ms(lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws_t, causal, sc, stream), stream,
                              reps=5)
            row["causal" if causal else "noncausal"] = {
                "speedup_fwd": round(t_sf / t_tf, 2), "speedup_bwd": round(t_sb / t_tb, 2),
                "speedup_fwd_bwd": round((t_sf + t_sb) / (t_tf + t_tb), 2)}
        out["by_N"].append(row)
        del q, k, v, do, o, lse, dq, dk, dv, ws_s, ws_t
        torch.cuda.empty_cache()
    return out


def mfma_ceiling():
    """Sustained MFMA rate of this part (libattn_probe.so): back-to-back
    32x32x16 bf16 products at two wavefronts per SIMD on every CU, once on
    random bf16 operands (the realistic ceiling: the power-limited clock
    depends on operand bit toggling) and once on constant operands."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_75_amd", "libattn_probe.so"))
    lib.attn_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_probe_mfma.restype = ctypes.c_int
    lib.attn_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.attn_probe_mfma_flops.restype = ctypes.c_double
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wgs, iters = 256 * 2, 20000  # two four-wavefront workgroups per CU: two wavefronts per SIMD
    out = torch.empty(wgs * 256 * 16, dtype=torch.float32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    res = {}
    for kind in ("random", "constant"):
        if kind == "random":
            ops = torch.randn(wgs * 256 * 64, device=dev, generator=g).to(torch.bfloat16)
        else:
            ops = torch.full((wgs * 256 * 64,), 0.5, device=dev, dtype=torch.bfloat16)

        def call():
            st = lib.attn_probe_mfma(ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(out.data_ptr()), wgs, iters,
                                     ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"attn_probe_mfma failed with status {st}")

        t = _median_ms(call, stream, reps=5)
        res[kind] = lib.attn_probe_mfma_flops(wgs, iters) / (t / 1e3) / 1e12
    del out, ops
    torch.cuda.empty_cache()
    return {"what": "v_mfma_f32_32x32x16_bf16 back to back, 2 wavefronts per SIMD on all 256 CUs",
            "random_bf16_tflops": round(res["random"], 1), "constant_tflops": round(res["constant"], 1),
            "frac_of_spec_random": round(res["random"] / PEAK_BF16_TFLOPS, 4)}


def secondary_ceilings(fwd_tflops, d):
    """Exponential and LDS-read throughput of this part (libattn_probe.so),
    beside what the non-causal forward at `fwd_tflops` needs: one exponential
    per score (FLOPs / 4d) and, per wavefront and 32 MFMAs (2^20 FLOP), 16 KiB
    of K and 16 KiB of V^T read from LDS (0.03125 B/FLOP at d = 128)."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_75_amd", "libattn_probe.so"))
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_exp.argtypes = [vp, vp, i, i, vp]
    lib.attn_probe_lds.argtypes = [vp, vp, i, i, vp]
    lib.attn_probe_exp.restype = lib.attn_probe_lds.restype = i
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    wgs, iters = 256 * 8, 20000
    seed = torch.rand(wgs * 256 * 8, device=dev)
    res = torch.empty(wgs * 256, device=dev)

    def run_exp():
        if lib.attn_probe_exp(ctypes.c_void_p(seed.data_ptr()), ctypes.c_void_p(res.data_ptr()), wgs, iters, sp) != 0:
            raise RuntimeError("attn_probe_exp failed")

    t = _median_ms(run_exp, stream, reps=5)
    exp_rate = wgs * 256.0 * iters * 8 / (t / 1e3)
    need = fwd_tflops * 1e12 / (4 * d)
    out["exp"] = {"what": "v_exp_f32, 8 independent chains per lane, 8 workgroups of 4 wavefronts per CU",
                  "measured_per_s": float(f"{exp_rate:.4g}"), "forward_needs_per_s": float(f"{need:.4g}"),
                  "fraction_used": round(need / exp_rate, 3)}
    wgs, iters = 256 * 4, 20000
    res = torch.empty(wgs * 256, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)

    def run_lds():
        if lib.attn_probe_lds(ctypes.c_void_p(res.data_ptr()), ctypes.c_void_p(clk.data_ptr()), wgs, iters, sp) != 0:
            raise RuntimeError("attn_probe_lds failed")

    t = _median_ms(run_lds, stream, reps=5)
    lds_bps = wgs * 256.0 * iters * 8 * 16 / (t / 1e3)
    c = clk.cpu().numpy().astype(np.float64)
    ghz = c[0] / c[1] * 0.1 if c[1] > 0 else float("nan")  # shader cycles per 10 ns tick
    # 32 KiB per 32 MFMAs of 32 x 32 x 16 (2 FLOP per multiply-add): 2^15 B / 2^20 FLOP
    need_lds = fwd_tflops * 1e12 * (32768.0 / (32 * 32 * 32 * 16 * 2)) if d == 128 else float("nan")
    out["lds"] = {"what": "ds_read_b128, conflict-free, 4 workgroups of 4 wavefronts per CU",
                  "measured_TBps": round(lds_bps / 1e12, 1),
                  "per_CU_bytes_per_clock": round(lds_bps / 256 / (ghz * 1e9), 1),
                  "probe_clock_GHz": round(ghz, 2),
                  "forward_needs_TBps": round(need_lds / 1e12, 1),
                  "fraction_used": round(need_lds / lds_bps, 3)}
    del seed, res, clk
    torch.cuda.empty_cache()
    return out


def mk_shape(g, dev, b, n, h, d):
    import torch

    return torch.randn(b, n, h, d, device=dev, generator=g).to(torch.bfloat16)


COPY_BYTES = 512 << 20  # calibration copy: reads and writes this many bytes per launch


def copy_calibration():
    """A plain device copy of known size, launched before the timed steps so the
    same rocprofv3 counter run measures it: FETCH_SIZE / WRITE_SIZE of this
    kernel against COPY_BYTES gives the scale from counter units to bytes."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)  # one elementwise kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize()


def _read_csv(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


PROFILE_TAG = "B4_N4096_H16_d128"  # the benchmark workload, for profile file names


EVIDENCE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT",
                     "SQ_LDS_IDX_ACTIVE", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_TRANS_F32",
                     "GRBM_GUI_ACTIVE")


def _profile_table(trace_dir, fetch_dir, write_dir, evidence_dir):
    """Per-kernel rows from rocprofv3 CSV output: (header lines, rows, raw).

    trace_dir: a --kernel-trace --stats run; fetch_dir / write_dir: --pmc
    FETCH_SIZE and --pmc WRITE_SIZE runs whose program ran copy_calibration()
    first; evidence_dir: a --pmc run of EVIDENCE_COUNTERS (any subset), or
    None.  HBM bytes are the counters scaled by what they read for the copy.
    """
    import glob

    def find(d, pattern):
        hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
        if not hits:
            raise SystemExit(f"no {pattern} under {d}")
        return hits[0]

    def per_kernel(d, counters):
        rows = _read_csv(find(d, "*counter_collection.csv"))
        acc = {}
        for r in rows:
            if r.get("Counter_Name") not in counters:
                continue
            acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        return {k_: {c_: sum(v_) / len(v_) for c_, v_ in cs.items()} for k_, cs in acc.items()}

    stats = _read_csv(find(trace_dir, "*kernel_stats.csv"))
    fetch = per_kernel(fetch_dir, {"FETCH_SIZE"})
    write = per_kernel(write_dir, {"WRITE_SIZE"})
    evid = per_kernel(evidence_dir, set(EVIDENCE_COUNTERS)) if evidence_dir else {}
    is_copy = lambda nm: "elementwise" in nm.lower() and "neg" in nm.lower()  # noqa: E731
    cname = next(k_ for k_ in fetch if is_copy(k_))
    cf, cw = fetch[cname]["FETCH_SIZE"], write[cname]["WRITE_SIZE"]
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)

    def short(nm):
        nm = nm.replace("(anonymous namespace)::", "").replace("attn::", "")
        return nm[nm.find("attn_"):nm.find("(")] if "attn_" in nm else nm[:60]

    head = [f"HBM counter calibration: plain copy of {COPY_BYTES} B reads FETCH_SIZE {cf:.0f} KiB, "
            f"WRITE_SIZE {cw:.0f} KiB -> byte scale {f_scale:.4f} (fetch) / {w_scale:.4f} (write)",
            "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
            "MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; co-exec = SQ_VALU_MFMA_COEXEC_CYCLES / "
            "SQ_VALU_MFMA_BUSY_CYCLES (share of MFMA-busy cycles in which a VALU instruction also issued); "
            "exp = SQ_INSTS_VALU_TRANS_F32 x 64 lanes",
            "",
            f"{'kernel':52s} {'calls':>5s} {'avg_us':>9s} {'pct':>6s} {'HBM_rd_MB':>10s} {'HBM_wr_MB':>10s} "
            f"{'HBM_GB/s':>9s} {'MFMA_busy':>9s} {'MFMA_TFLOP':>10s} {'LDS_confl':>9s} {'co-exec':>8s} {'exp_G':>8s}"]
    rows, raw = [], []
    for r in stats:
        nm = r["Name"]
        if "attn_" not in nm:
            continue
        avg_us = float(r["AverageNs"]) / 1e3
        fk = fetch.get(nm, {})
        wk = write.get(nm, {})
        ek = evid.get(nm, {})
        rd = fk.get("FETCH_SIZE", float("nan")) * 1024.0 * f_scale
        wr = wk.get("WRITE_SIZE", float("nan")) * 1024.0 * w_scale
        gbs = (rd + wr) / (avg_us * 1e-6) / 1e9
        nan = float("nan")
        busy = ek["SQ_VALU_MFMA_BUSY_CYCLES"] * 8 / (ek["GRBM_GUI_ACTIVE"] * 1024.0) \
            if "SQ_VALU_MFMA_BUSY_CYCLES" in ek and "GRBM_GUI_ACTIVE" in ek else nan
        tf = ek["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e12 if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in ek else nan
        conf = ek["SQ_LDS_BANK_CONFLICT"] / max(1.0, ek["SQ_LDS_IDX_ACTIVE"]) \
            if "SQ_LDS_BANK_CONFLICT" in ek and "SQ_LDS_IDX_ACTIVE" in ek else nan
        coex = ek["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(1.0, ek["SQ_VALU_MFMA_BUSY_CYCLES"]) \
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in ek and "SQ_VALU_MFMA_BUSY_CYCLES" in ek else nan
        exps = ek["SQ_INSTS_VALU_TRANS_F32"] * 64 / 1e9 if "SQ_INSTS_VALU_TRANS_F32" in ek else nan
        rows.append(f"{short(nm)[:52]:52s} {r['Calls']:>5s} {avg_us:9.2f} {float(r['Percentage']):6.2f} "
                    f"{rd / 1e6:10.1f} {wr / 1e6:10.1f} {gbs:9.1f} {busy:9.3f} {tf:10.4f} {conf:9.4f} "
                    f"{coex:8.3f} {exps:8.2f}")
        raw.append((nm, rd, wr, fk.get("FETCH_SIZE"), wk.get("WRITE_SIZE"), avg_us, cf, cw))
    return head, rows, raw


def summarize_workload(trace_dir, fetch_dir, write_dir, evidence_dir, out_name, title, cmd):
    """profiles/OUT_NAME from the four rocprofv3 runs of `bench.py
    --profile-workload SPEC` (one workload per run)."""
    head, rows, _ = _profile_table(trace_dir, fetch_dir, write_dir, evidence_dir)
    lines = [title, ""] + [f"{k_ + ':':9s} {cmd.get(k_, '')}" for k_ in ("trace", "fetch", "write", "evidence")]
    lines += ["($R: the repository root; $O: an output directory; each command run from /tmp)", ""] + head + rows
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def profile_workload(spec: str, reps: int):
    """Run one workload's forward and backward ``reps`` times each (after one
    untimed call of each), for rocprofv3 counter passes."""
    import numpy as np
    import torch

    import exact_io_aware_75_amd as ea

    s = shape_of(spec)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    mk = lambda hh: torch.randn(s.b, s.n, hh, s.d, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
    q, k, v, do = mk(s.hq), mk(s.hkv), mk(s.hkv), mk(s.hq)
    o, lse = torch.empty_like(q), torch.empty((s.b, s.hq, s.n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(s.b, s.n, s.hq, s.hkv, s.d), dtype=torch.uint8, device=dev)
    sc = 1.0 / float(np.sqrt(s.d))
    for _ in range(1 + reps):
        ea.attn_fwd(q, k, v, o, lse, s.causal, sc, stream)
    for _ in range(1 + reps):
        ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, s.causal, sc, stream)
    torch.cuda.synchronize()
    print(f"profiled {spec}: {s}", flush=True)


def shape_of(spec: str):
    """A full-size workload by name: 'd:n:causal' (hidden-2048 layer), 'w256'
    (MHA d = 256), 'gqa8' / 'gqa1' (GQA / MQA) or 'long32768' / 'long65536'."""
    from exact_io_aware_75_amd import configs

    if spec == "w256":
        return configs.wide_head()
    if spec.startswith("gqa"):
        return configs.gqa(int(spec[3:]))
    if spec.startswith("long"):
        return configs.long_seq(int(spec[4:]))
    d, n, c = spec.split(":")
    return configs.hidden2048(int(d), int(n), c == "1")


def summarize_profiles(trace_dir, fetch_dir, write_dir, evidence_dir, cmd):
    """Turn rocprofv3 CSV output of `bench.py` runs into profiles/ summaries.

    trace_dir: a --kernel-trace --stats run (kernel_stats.csv); fetch_dir /
    write_dir: --pmc FETCH_SIZE and --pmc WRITE_SIZE runs; evidence_dir: a
    --pmc run of SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
    SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE (or None).
    Writes profiles/step_kernels_<workload>.txt (per-kernel time, HBM bytes,
    MFMA busy, LDS conflicts) and profiles/bwd_dkdv_traffic_<workload>.json
    (the dominant kernel's HBM bytes per launch, read back by the benchmark).
    """
    head, rows, raw = _profile_table(trace_dir, fetch_dir, write_dir, evidence_dir)
    lines = [f"Kernels of one benchmark step (workload {PROFILE_TAG}, bf16; fwd + bwd, non-causal and causal)",
             "",
             f"trace:    {cmd.get('trace', '')}",
             f"fetch:    {cmd.get('fetch', '')}",
             f"write:    {cmd.get('write', '')}",
             f"evidence: {cmd.get('evidence', '')}",
             "($R: the repository root; $O: an output directory; each command run from /tmp)",
             ""] + head + rows
    # <dtype, d, causal, block-sparse, paired>
    dom = next((x for x in raw if re.search(r"attn_bwd_dkdv_kernel<[^,<>]+, 128, false, false(, false)?>", x[0])), None)
    if dom is None:
        raise SystemExit("dK/dV kernel (d=128, non-causal) not found in the trace")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"step_kernels_{PROFILE_TAG}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    nm, rd, wr, fkib, wkib, avg_us, cf, cw = dom
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"kernel": nm, "source_sha256": kernel_source_hash(), "avg_us_rocprof": avg_us,
                   "fetch_kib": fkib, "write_kib": wkib, "copy_fetch_kib": cf, "copy_write_kib": cw,
                   "copy_bytes": COPY_BYTES, "read_bytes": rd, "write_bytes": wr,
                   "bytes_per_launch": rd + wr, "commands": cmd}, f, indent=1)
    print("\n".join(lines))


def summarize_hbm(trace_dir, fetch_dir, write_dir, out_name, title, cmds, name_filter):
    """Write profiles/<out_name>: mean duration (kernel trace), HBM bytes read
    and written per launch (FETCH_SIZE / WRITE_SIZE runs, scaled by the same
    counters' reading for the calibration copy) and the resulting GB/s for the
    kernels whose name holds `name_filter`."""
    import glob

    def find(d, pattern):
        hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
        if not hits:
            raise SystemExit(f"no {pattern} under {d}")
        return hits[0]

    def per_kernel(d, counter):
        acc = {}
        for r in _read_csv(find(d, "*counter_collection.csv")):
            if r.get("Counter_Name") == counter:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k_: sum(v_) / len(v_) for k_, v_ in acc.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    cname = next(k_ for k_ in fetch if "elementwise" in k_.lower() and "neg" in k_.lower())
    f_scale = COPY_BYTES / (fetch[cname] * 1024.0)
    w_scale = COPY_BYTES / (write[cname] * 1024.0)
    lines = [title, ""] + [f"{k_}: {v_}" for k_, v_ in cmds.items()] + [
        "", f"HBM counter calibration: plain copy of {COPY_BYTES} B -> byte scale {f_scale:.4f} (fetch) / "
            f"{w_scale:.4f} (write)", "",
        f"{'kernel':58s} {'calls':>5s} {'avg_us':>9s} {'HBM_rd_MB':>10s} {'HBM_wr_MB':>10s} {'HBM_GB/s':>9s}"]
    for r in _read_csv(find(trace_dir, "*kernel_stats.csv")):
        nm = r["Name"]
        if name_filter not in nm:
            continue
        avg_us = float(r["AverageNs"]) / 1e3
        rd = fetch.get(nm, float("nan")) * 1024.0 * f_scale
        wr = write.get(nm, float("nan")) * 1024.0 * w_scale
        short = nm.replace("(anonymous namespace)::", "").replace("attn::", "").replace("void ", "")
        short = short[:short.find("(")]
        lines.append(f"{short[:58]:58s} {r['Calls']:>5s} {avg_us:9.2f} {rd / 1e6:10.1f} {wr / 1e6:10.1f} "
                     f"{(rd + wr) / (avg_us * 1e-6) / 1e9:9.1f}")
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir, out_name, title, cmd, name_filter=""):
    """Write profiles/<out_name>: calls and durations per kernel and grid shape
    of a rocprofv3 --kernel-trace run (its kernel_trace.csv), for the kernels
    whose name holds `name_filter` and "attn_"."""
    import glob

    hits = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not hits:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    durs = {}  # (kernel, grid in workgroups) -> durations
    for r in _read_csv(hits[0]):
        nm = r["Kernel_Name"]
        if "attn_" not in nm or name_filter not in nm:
            continue
        wg = [int(r[f"Grid_Size_{a}"]) // max(1, int(r[f"Workgroup_Size_{a}"])) for a in "XYZ"]
        key = (nm, "x".join(str(v_) for v_ in wg))
        durs.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def short(nm):
        nm = nm.replace("(anonymous namespace)::", "").replace("attn::", "")
        return nm[nm.find("attn_"):nm.find("(")] if "attn_" in nm else nm[:60]

    lines = [title, "", f"trace: {cmd}", "",
             f"{'kernel':52s} {'grid (WGs)':>12s} {'calls':>5s} {'avg_us':>9s} {'median_us':>9s} "
             f"{'min_us':>9s} {'max_us':>9s}"]
    for (nm, grid), ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        s = sorted(ds)
        lines.append(f"{short(nm)[:52]:52s} {grid:>12s} {len(s):5d} {sum(s) / len(s):9.2f} "
                     f"{s[len(s) // 2]:9.2f} {s[0]:9.2f} {s[-1]:9.2f}")
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps before the timed ones (40 steps, about 0.14 s, let the clock settle)")
    ap.add_argument("--sweep", action="store_true", help="also time every full-size configuration")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle baseline budget in seconds (0 disables it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-workload", metavar="SPEC",
                    help="run one workload's fwd and bwd --steps times each for rocprofv3 counter passes and exit "
                         "(SPEC: d:n:causal for the hidden-2048 layer, w256, gqa8, gqa1, long32768, long65536)")
    ap.add_argument("--summarize-workload", nargs=6,
                    metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "EVIDENCE_DIR", "OUT_NAME", "TITLE"),
                    help="write per-kernel time, HBM bytes and counters of a --profile-workload run to "
                         "profiles/OUT_NAME and exit")
    ap.add_argument("--oracle-sweep", action="store_true",
                    help="time the CPU fp64 oracle on every full-size workload (fwd, fwd+bwd) and exit")
    ap.add_argument("--no-targets", dest="targets", action="store_false",
                    help="skip the per-workload target points in the JSON line")
    ap.add_argument("--no-sparse", dest="sparse", action="store_false",
                    help="skip the block-sparse and shard measurements")
    ap.add_argument("--no-standard", dest="standard", action="store_false",
                    help="skip the standard (materialising) attention comparison")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain copy of known size first (for counter calibration)")
    ap.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "EVIDENCE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV output and exit")
    ap.add_argument("--summarize-cmds", default="{}", help="JSON dict of the commands that made them")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "OUT_NAME", "TITLE", "CMD"),
                    help="write a per-kernel duration table of a kernel-trace run to profiles/OUT_NAME and exit")
    ap.add_argument("--trace-filter", default="", help="only kernels whose name contains this")
    ap.add_argument("--summarize-hbm", nargs=6, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "OUT_NAME", "TITLE",
                                                        "FILTER"),
                    help="write per-kernel time and HBM bytes of matching kernels to profiles/OUT_NAME and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(*args.summarize, json.loads(args.summarize_cmds))
        return
    if args.summarize_workload:
        summarize_workload(*args.summarize_workload, json.loads(args.summarize_cmds))
        return
    if args.summarize_hbm:
        summarize_hbm(*args.summarize_hbm[:5], json.loads(args.summarize_cmds), args.summarize_hbm[5])
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, name_filter=args.trace_filter)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the kernels shard trivially over batch and heads; this benchmark measures one GPU).",
              file=sys.stderr)
        sys.exit(2)
    if args.oracle_sweep:
        print(json.dumps({"oracle_sweep": oracle_sweep()}), flush=True)
        return
    if args.profile_workload:
        if args.copy_calibration:
            copy_calibration()
        profile_workload(args.profile_workload, args.steps)
        return
    if args.no_cpu_baseline:
        args.cpu_seconds = 0.0
    if args.copy_calibration:
        copy_calibration()
    run(args)


if __name__ == "__main__":
    main()
