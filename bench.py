#!/usr/bin/env python3
"""Benchmark of the plan/run attention hot path on one MI355X.

A step is one xattn_run over one batch of a seeded synthetic workload: every kernel
of the run (attention, and the log-sum-exp merge when contexts are split). Plan is
host work, done once before the timed region (its time is printed separately).

Default workload: Whisper-large-style decode cross-attention (64 requests x 1 query,
context 1500, 20 heads, head_dim 64, bf16, page_size 16, shuffled pages), metric:
effective KV GB/s = algorithmic K+V bytes (sum of kv_len x Hkv x D x 2 x 2 B) per
step time. Prefill workloads report TFLOP/s = 4 x D x (visible query-key pairs x Hq)
per step time.

Prints ONE JSON line. With --all, a "sweep" object carries the other workloads'
numbers (same definitions) as well.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (prefill) and effective KV GB/s (decode) vs MI355X roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3      # MI355X fp32 vector, published
KERNEL_SOURCES = {
    "decode": "ragged_attention_serving_amd/csrc/attn_decode.hip",
    "mfma": "ragged_attention_serving_amd/csrc/attn_mma.hip",
    "fp32": "ragged_attention_serving_amd/csrc/attn_f32.hip",
    "merge": "ragged_attention_serving_amd/csrc/merge.hip",
    "write": "ragged_attention_serving_amd/csrc/write_kv.hip",
}
TIMING_EVERY = 5  # kernel start/end events on every 5th timed run
# Without --warmup, warm-up runs continue until this much time has passed: the GPU leaves
# its idle clocks only after some tens of milliseconds of load (a short prefill timed at
# once reads about 25% slow).
WARMUP_SECONDS = 0.5
MAX_AUTO_WARMUP = 4000


def warm_up(run, warmup):
    """Runs `run` `warmup` times, or (warmup None) until WARMUP_SECONDS have passed (at least
    5 runs); returns the number of runs."""
    import torch
    if warmup is not None:
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        return warmup
    n = 0
    t0 = time.perf_counter()
    while n < 5 or (time.perf_counter() - t0 < WARMUP_SECONDS and n < MAX_AUTO_WARMUP):
        for _ in range(5):
            run()
        n += 5
        torch.cuda.synchronize()
    return n
KERNEL_NAMES = {"decode": "attn_decode_kernel", "mfma": "attn_mma_kernel", "fp32": "attn_f32_kernel",
                "merge": "merge_kernel"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """The source without comments and blank lines: edits to comments keep the hash."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", l).rstrip() for l in text.splitlines())
    return "\n".join(l for l in lines if l.strip())


def source_sha(stage: str) -> str:
    """Hash of the code (comments stripped) of a kernel stage's source and device.h."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[stage], "ragged_attention_serving_amd/csrc/device.h"):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def workload_numbers(w, info):
    """Algorithmic bytes and FLOPs of one step (the method's own work only)."""
    elt = 2 if w.dtype == "bf16" else 4
    kv_bytes = int(w.kv_lens().sum()) * w.num_kv_heads * w.head_dim * 2 * elt
    flops = 4 * w.head_dim * int(info["visible_pairs"])
    g = w.num_qo_heads // w.num_kv_heads
    decode = bool(np.all(w.qo_lens() * g <= 8)) and w.dtype == "bf16"
    return kv_bytes, flops, decode


def to_dev(a, dtype, dev):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def measure(w, steps, warmup, dev, cold_steps=5):
    """Plans, then times `steps` back-to-back runs (wall clock and per-kernel events)."""
    import torch
    import ragged_attention_serving_amd as xa

    q, k, v = (to_dev(w.q, w.dtype, dev), to_dev(w.k_pages, w.dtype, dev), to_dev(w.v_pages, w.dtype, dev))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    plan = xa.Plan()
    t0 = time.perf_counter()
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
              w.num_kv_heads, w.head_dim, w.page_size, w.num_pages, w.mask_mode, w.block_size,
              w.sm_scale, w.dtype)
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info()
    warmed = warm_up(lambda: plan.run(q, k, v, out, lse), warmup)

    # timed region: exactly `steps` runs, synchronised on both sides; on every TIMING_EVERY-th
    # run the library launches each kernel with HIP events stamped with its start and end,
    # on the run's stream, which give the per-kernel durations
    plan.set_timing(TIMING_EVERY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.run(q, k, v, out, lse)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    stages = plan.timing()
    plan.set_timing(0)

    # cold runs: 1 GiB written between runs to evict L2 and the Infinity Cache
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(cold_steps):
        scratch.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        plan.run(q, k, v, out, lse)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del scratch
    plan.close()
    del q, k, v, out, lse
    return dict(plan_ms=plan_ms, wall_ms=wall_ms, stages=stages, info=info, warmup=warmed,
                cold_ms=float(np.median(cold)) if cold else None)


def measure_write(w, steps, warmup, dev):
    """Times the context write (xattn_write_kv) of w's contexts into fresh pools: `steps`
    back-to-back writes between two synchronisations. Bytes moved: the packed K and V
    rows read once and written once."""
    import torch
    import ragged_attention_serving_amd as xa
    from ragged_attention_serving_amd import synth

    ks, vs = synth.context_source(w, seed=1)
    ksrc, vsrc = to_dev(ks, w.dtype, dev), to_dev(vs, w.dtype, dev)
    del ks, vs
    kpool = torch.zeros(w.k_pages.shape, dtype=ksrc.dtype, device=dev)
    vpool = torch.zeros(w.v_pages.shape, dtype=ksrc.dtype, device=dev)
    plan = xa.Plan()
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
              w.num_kv_heads, w.head_dim, w.page_size, w.num_pages, w.mask_mode, w.block_size,
              w.sm_scale, w.dtype)
    warmed = warm_up(lambda: plan.write_kv(ksrc, vsrc, kpool, vpool), warmup)
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.write_kv(ksrc, vsrc, kpool, vpool)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    moved = 2 * 2 * ksrc.numel() * ksrc.element_size()
    plan.close()
    return {"workload": f"context_write:{w.name}", "ms_per_write": round(ms, 5), "warmup": warmed,
            "bytes": moved, "GBps": moved / (ms * 1e-3) / 1e9,
            "hbm_frac": moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def summarize(w, m):
    kv_bytes, flops, decode = workload_numbers(w, m["info"])
    per = {}
    for st, (ms, n) in m["stages"].items():
        if n:
            per[st] = ms / n
    dominant = max(per, key=per.get) if per else None
    res = dict(workload=w.name, decode=decode, kv_bytes=kv_bytes, flops=flops, plan_ms=round(m["plan_ms"], 3),
               ms_per_step=m["wall_ms"], cold_ms_per_step=m["cold_ms"],
               kernel_ms={k: round(v, 5) for k, v in per.items()}, dominant=dominant,
               schedule=m["info"])
    if decode:
        res["GBps"] = kv_bytes / (m["wall_ms"] * 1e-3) / 1e9
        res["GBps_cold"] = kv_bytes / (m["cold_ms"] * 1e-3) / 1e9 if m["cold_ms"] else None
        res["kernel_GBps"] = kv_bytes / (per[dominant] * 1e-3) / 1e9 if dominant else None
        res["hbm_frac"] = res["kernel_GBps"] / HBM_PEAK_GBS if dominant else None
    else:
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
        res["TFLOPs"] = flops / (m["wall_ms"] * 1e-3) / 1e12
        res["TFLOPs_cold"] = flops / (m["cold_ms"] * 1e-3) / 1e12 if m["cold_ms"] else None
        res["kernel_TFLOPs"] = flops / (per[dominant] * 1e-3) / 1e12 if dominant else None
        res["mfma_frac"] = res["kernel_TFLOPs"] / peak if dominant else None
        # compulsory HBM bytes of a prefill: K and V once, Q read and out and lse written once
        elt = 2 if w.dtype == "bf16" else 4
        rows = int(w.qo_lens().sum()) * w.num_qo_heads
        hbm_bytes = kv_bytes + rows * (2 * w.head_dim * elt + 4)
        res["hbm_bytes_compulsory"] = hbm_bytes
        res["hbm_GBps_compulsory"] = hbm_bytes / (per[dominant] * 1e-3) / 1e9 if dominant else None
        res["hbm_frac_compulsory"] = res["hbm_GBps_compulsory"] / HBM_PEAK_GBS if dominant else None
    return res


def traffic_for(stage: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{workload}:{stage}")
    except Exception:
        return None
    if not rec or rec.get("source_sha") != source_sha(stage):
        return None
    return rec.get("bytes_per_launch")


_CPU_W = None  # the workload, shared with forked workers


def _cpu_worker(args):
    """One process: oracle passes over requests start, start+step, ... for wall_s seconds."""
    start, step, wall_s = args
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)  # one BLAS thread per process
    except Exception:  # pragma: no cover
        ctx = None
    from oracle import ref
    w = _CPU_W
    elt = 2 if w.dtype == "bf16" else 4
    kv = w.kv_lens()
    done_bytes, done_req, i = 0, 0, start
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < wall_s:
        r = i % w.batch_size
        ref.run_workload(w, requests=[r])
        done_bytes += int(kv[r]) * w.num_kv_heads * w.head_dim * 2 * elt
        done_req += 1
        i += step
    el = time.perf_counter() - t0
    del ctx  # (the limit only needs to hold while this worker runs)
    return done_bytes, done_req, el


def cpu_baseline(w, cpu_seconds=24.0):
    """The fp64 oracle as it stands, on this host's cores: one process per core (at most 16),
    each taking whole requests (all heads) in turn for cpu_seconds / processes (at least 2 s)
    of wall time.
    Must run before the process touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    global _CPU_W
    _CPU_W = w
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    wall = max(2.0, cpu_seconds / n)
    ctx = mp.get_context("fork")
    with ctx.Pool(n) as pool:
        t0 = time.perf_counter()
        parts = pool.map(_cpu_worker, [(k, n, wall) for k in range(n)])
        el = time.perf_counter() - t0
    done_bytes = sum(p[0] for p in parts)
    done_req = sum(p[1] for p in parts)
    elt = 2 if w.dtype == "bf16" else 4
    kv_bytes = int(w.kv_lens().sum()) * w.num_kv_heads * w.head_dim * 2 * elt
    return {"value": done_bytes / el / 1e9, "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"{done_req} request passes (all {w.num_qo_heads} heads each, {done_req / w.batch_size:.2f} "
                      f"x the workload's {w.batch_size} requests) by {n} processes in {el:.1f} s",
            "workload_bytes": kv_bytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed runs before the timed ones (default: as many as fill %.1f s)" % WARMUP_SECONDS)
    ap.add_argument("--workload", default="whisper_decode_cross")
    ap.add_argument("--all", action="store_true", help="also measure every other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="CPU seconds (summed over the worker processes) for the oracle baseline")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="runs timed one by one after a 1 GiB cache flush (0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device to device once (the known-size kernel that scales "
                         "the FETCH_SIZE and WRITE_SIZE counters) and exit")
    ap.add_argument("--context-write", action="store_true",
                    help="only time the context write (xattn_write_kv) of the workload's contexts "
                         "and print its line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path is data-parallel per GPU; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from ragged_attention_serving_amd import synth

    cpu_line = None
    if not (args.no_cpu_baseline or args.copy_calibration or args.context_write):
        # before anything touches the GPU: the oracle's worker processes are forked
        log(f"[bench] timing the CPU oracle on {args.workload}")
        cpu_line = cpu_baseline({**synth.WORKLOADS, **synth.TP_WORKLOADS}[args.workload](0), args.cpu_seconds)
        log(f"[bench] cpu baseline {json.dumps(cpu_line)}")

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4}), flush=True)
        return
    all_workloads = {**synth.WORKLOADS, **synth.TP_WORKLOADS}
    log(f"[bench] generating {args.workload}")
    w = all_workloads[args.workload](0)
    if args.context_write:
        print(json.dumps(measure_write(w, args.steps, args.warmup, dev)), flush=True)
        return
    log(f"[bench] measuring {args.workload}: steps={args.steps} warmup={args.warmup}")
    m = measure(w, args.steps, args.warmup, dev, args.cold_steps)
    res = summarize(w, m)
    log(f"[bench] {json.dumps({k: v for k, v in res.items() if k != 'schedule'})}")

    st = res["dominant"]
    per_ms = res["kernel_ms"][st]
    if res["decode"]:
        achieved = res["kv_bytes"] / (per_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        value = res["kv_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
        unit = "GB/s"
    else:
        achieved = res["flops"] / (per_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        value = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12
        unit = "TFLOP/s"
    roof["traffic"] = traffic_for(st, w.name)
    roof["kernel"] = KERNEL_NAMES[st]
    roof["kernel_ms"] = round(per_ms, 5)
    roof["kernel_source_sha"] = source_sha(st)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": m["warmup"], "ms_per_step": round(res["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "requests": w.batch_size, "query_tokens": int(w.qo_indptr[-1]),
                   "kv_tokens": int(w.kv_lens().sum()), "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "mask_mode": w.mask_mode, "block_size": w.block_size, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cold_ms_per_step": round(res["cold_ms_per_step"], 5) if res["cold_ms_per_step"] else None,
        "plan_ms": res["plan_ms"],
        "schedule": res["schedule"],
    }
    if cpu_line is not None:
        line["cpu_baseline"] = cpu_line
    if args.all:
        sweep = {}
        for name, fn in synth.WORKLOADS.items():
            if name == w.name:
                continue
            log(f"[bench] sweep: generating {name}")
            ws = fn(0)
            log(f"[bench] sweep: measuring {name}")
            ms = measure(ws, args.steps, None, dev)
            r = summarize(ws, ms)
            r.pop("schedule", None)
            r["warmup"] = ms["warmup"]
            sweep[name] = r
            log(f"[bench] {json.dumps(r)}")
            del ws, ms
            torch.cuda.empty_cache()
        for name, fn in synth.TP_WORKLOADS.items():
            log(f"[bench] sweep: generating {name}")
            ws = fn(0)
            log(f"[bench] sweep: measuring {name}")
            ms = measure(ws, args.steps, None, dev)
            r = summarize(ws, ms)
            r.pop("schedule", None)
            r["warmup"] = ms["warmup"]
            sweep[name] = r
            log(f"[bench] {json.dumps(r)}")
            del ws, ms
            torch.cuda.empty_cache()
        log("[bench] sweep: context write")
        wr = measure_write(synth.WORKLOADS["whisper_decode_cross"](0), args.steps, None, dev)
        sweep[wr["workload"]] = wr
        log(f"[bench] {json.dumps(wr)}")
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
