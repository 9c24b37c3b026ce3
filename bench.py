#!/usr/bin/env python3
"""Benchmark of the plan/run attention hot path on one MI355X.

A step is one xattn_run over one batch of a seeded synthetic workload: every kernel of
the run (attention, and the log-sum-exp merge when contexts are split). Plan is host
work, done once before the timed runs (its time is printed separately). Inputs are
resident in HBM before any timed run.

Headline workload (the largest of the five): causal GQA paged decode, 256 requests x 1
query, 32 query / 8 KV heads, head_dim 128, bf16, page_size 16, contexts log-uniform in
[512, 32768] (9.51 GB of K and V). Metric: effective KV GB/s = algorithmic K+V bytes
(sum of kv_len x Hkv x D x 2 x 2 B) per step time. Prefill workloads report TFLOP/s =
4 x D x (visible query-key pairs x Hq) per step time.

`value` is the median over the timed runs, each run after 1 GiB is written to evict L2
and the Infinity Cache (cold); the best run and back-to-back (warm) runs are reported
beside it. The roofline object is the dominant kernel's algorithmic work over its own
mean duration in the cold runs (HIP events the runtime stamps with the kernel's start
and end, on the run's stream).

Prints ONE JSON line. A "sweep" object carries the four other workloads, each with its
own value, timing and roofline (--no-sweep: headline only; --all adds cacheless span-to-span
cross-attention, causal paged prefill, per-rank tensor-parallel shapes, graph replay of a
32-layer decode step and the context write).
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
HEADLINE = "gqa_decode_causal"
# what each workload is, by its sizes (the config objects of the JSON line)
CONFIGS = {
    "tiny_cross_f32": {"workload": "tiny_cross_f32", "requests": 2, "query_lens": [1, 3],
                       "context_lens": [16, 40], "num_qo_heads": 2, "num_kv_heads": 2, "head_dim": 16,
                       "page_size": 4, "mask": "none", "dtype": "f32"},
    "whisper_decode_cross": {"workload": "whisper_decode_cross", "requests": 64, "query_tokens": 64,
                             "context_len": 1500, "kv_tokens": 96000, "num_qo_heads": 20,
                             "num_kv_heads": 20, "head_dim": 64, "page_size": 16, "mask": "none"},
    "ragged_prefill_cross": {"workload": "ragged_prefill_cross", "requests": 32,
                             "query_lens": "uniform 1-448 (sum 7569)", "context_len": 1500,
                             "num_qo_heads": 20, "num_kv_heads": 20, "head_dim": 64, "page_size": 16,
                             "mask": "none"},
    "block_causal_ragged": {"workload": "block_causal_ragged", "spans": 64,
                            "span_lens": "uniform 256-4096 (sum 141675)", "block_size": 64,
                            "num_qo_heads": 16, "num_kv_heads": 16, "head_dim": 128,
                            "page_table": "identity (cacheless)", "mask": "block_causal"},
    "gqa_decode_causal": {"workload": "gqa_decode_causal", "requests": 256, "query_tokens": 256,
                          "context_lens": "log-uniform 512-32768 (sum 2321997)", "num_qo_heads": 32,
                          "num_kv_heads": 8, "head_dim": 128, "page_size": 16, "mask": "causal",
                          "kv_bytes": 9510899712, "parallelism": "none (1 GPU)"},
}
CONFIGS.update({
    "ragged_cross_spans": {"workload": "ragged_cross_spans", "requests": 32,
                           "query_spans": "uniform 1-448 (sum 7569)", "key_spans": "uniform 256-4096 (sum 68724)",
                           "num_qo_heads": 16, "num_kv_heads": 16, "head_dim": 128,
                           "page_table": "identity (cacheless)", "mask": "none"},
    "causal_prefill_paged": {"workload": "causal_prefill_paged", "requests": 16,
                             "query_lens": "= context lens, uniform 256-4096 (sum 35086)", "num_qo_heads": 32,
                             "num_kv_heads": 8, "head_dim": 128, "page_size": 16, "mask": "causal"},
    "gqa_decode_causal_tp8": {"workload": "gqa_decode_causal_tp8", "requests": 256, "num_qo_heads": 4,
                              "num_kv_heads": 1, "head_dim": 128, "page_size": 16, "mask": "causal",
                              "note": "one rank's heads of gqa_decode_causal at tensor parallelism 8"},
    "whisper_decode_cross_tp4": {"workload": "whisper_decode_cross_tp4", "requests": 64, "num_qo_heads": 5,
                                 "num_kv_heads": 5, "head_dim": 64, "page_size": 16, "mask": "none",
                                 "note": "one rank's heads of whisper_decode_cross at tensor parallelism 4"},
})
DTYPE_NAME = {"bf16": "bf16", "f32": "f32"}


def res_dtype(name):
    return "f32" if name == "tiny_cross_f32" else "bf16"


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


FLUSH_BYTES = 1 << 30  # written before each cold run: more than L2 and the 256 MB Infinity Cache


def _stats(xs):
    xs = sorted(xs)
    if not xs:
        return None
    return {"median_ms": round(float(np.median(xs)), 5), "best_ms": round(xs[0], 5),
            "mean_ms": round(float(np.mean(xs)), 5), "runs": len(xs)}


def measure(w, steps, warmup, dev, preroll_s=0.0, keep_rows=None):
    """Plans w once, then times it two ways, each over `steps` runs:

    * cold (the headline): before each run 1 GiB is written to evict L2 and the Infinity
      Cache; the run's own duration comes from HIP events around it on its stream, and, in
      a second set of `steps` such runs, each kernel's from events the runtime stamps with
      that kernel's start and end;
    * warm: `steps` runs back to back (labelled warm), events between consecutive runs;
      every TIMING_EVERY-th run carries the kernel events.

    `warmup` untimed runs come first (None: as many as fill WARMUP_SECONDS), then, when
    preroll_s > 0, cache flushes alone for that long (the GPU leaves its idle clocks only
    under load; a flush is not a run). keep_rows (query-row indices) returns those rows of
    the last timed run's out and lse."""
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
    run = lambda: plan.run(q, k, v, out, lse)  # noqa: E731
    warmed = warm_up(run, warmup)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flushes = 0
    if preroll_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < preroll_s:
            scratch.fill_(1.0)
            flushes += 1
            torch.cuda.synchronize()

    # cold runs, one at a time: first the runs' own durations (no per-kernel events, which
    # add a few microseconds to each run), then the same number of runs for the kernels'
    # own durations
    cold, cold_k = [], {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(steps):
        scratch.fill_(1.0)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    plan.set_timing(1)
    for _ in range(steps):
        scratch.fill_(1.0)
        run()
        torch.cuda.synchronize()
        for st, (ms, n) in plan.timing().items():
            if n:
                cold_k.setdefault(st, []).append(ms / n)
    del scratch

    # warm runs, back to back
    plan.set_timing(TIMING_EVERY)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i].record()
        run()
    ev[steps].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / max(steps, 1)
    warm = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    warm_k = {st: ms / n for st, (ms, n) in plan.timing().items() if n}
    plan.set_timing(0)
    kept = None
    if keep_rows is not None:
        idx = torch.as_tensor(np.asarray(keep_rows, np.int64), device=dev)
        kept = (out.index_select(0, idx).float().cpu().numpy().astype(np.float64),
                lse.index_select(0, idx).cpu().numpy().astype(np.float64))
    plan.close()
    del q, k, v, out, lse
    return dict(plan_ms=plan_ms, info=info, warmup=warmed, preroll_flushes=flushes,
                cold=cold, cold_kernel={st: float(np.mean(x)) for st, x in cold_k.items()},
                warm=warm, warm_kernel=warm_k, warm_wall_ms=wall_ms, kept=kept)


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


def measure_graph(w, layers, steps, dev):
    """One planned step of `layers` runs (each layer its own q, K/V cache, out and lse, the same
    schedule), issued eagerly from the host and replayed from one captured HIP graph, back to
    back; and the host time of planning the next step into the other slot while a replay runs
    (the double buffer of page "mstar.engine.resources.attn.cross", force_double_buffer)."""
    import torch
    import ragged_attention_serving_amd as xa

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q = [to_dev(w.q, w.dtype, dev) for _ in range(layers)]
        k = [to_dev(w.k_pages, w.dtype, dev) for _ in range(layers)]
        v = [to_dev(w.v_pages, w.dtype, dev) for _ in range(layers)]
        out = [torch.empty_like(x) for x in q]
        lse = [torch.empty(x.shape[:2], dtype=torch.float32, device=dev) for x in q]
        plan = xa.Plan()
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
                  w.num_kv_heads, w.head_dim, w.page_size, w.num_pages, w.mask_mode, w.block_size,
                  w.sm_scale, w.dtype, stream=s)

    def step():
        for i in range(layers):
            plan.run(q[i], k[i], v[i], out[i], lse[i], stream=s)

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        with torch.cuda.stream(s):
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < WARMUP_SECONDS:
                fn()
                s.synchronize()
            for i in range(steps):
                ev[i].record(s)
                fn()
            ev[steps].record(s)
        s.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))

    eager = timed(step)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    s.synchronize()
    graph = timed(g.replay)
    # the next step's plan goes into the other slot while a replay reads this one
    with torch.cuda.stream(s):
        g.replay()
        t0 = time.perf_counter()
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
                  w.num_kv_heads, w.head_dim, w.page_size, w.num_pages, w.mask_mode, w.block_size,
                  w.sm_scale, w.dtype, stream=s)
        plan_ms = (time.perf_counter() - t0) * 1e3
    s.synchronize()
    # the captured graph still replays the first slot's schedule: its outputs equal an eager run
    ref_out = [x.clone() for x in out]
    g.replay()
    s.synchronize()
    same = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(out, ref_out))
    del g
    plan.close()
    kv_bytes = int(w.kv_lens().sum()) * w.num_kv_heads * w.head_dim * 2 * (2 if w.dtype == "bf16" else 4)
    return {"workload": f"graph_replay:{w.name}", "layers": layers, "eager_ms_per_step": round(eager, 5),
            "graph_ms_per_step": round(graph, 5), "graph_speedup": round(eager / graph, 3),
            "GBps_eager": round(layers * kv_bytes / (eager * 1e-3) / 1e9, 1),
            "GBps_graph": round(layers * kv_bytes / (graph * 1e-3) / 1e9, 1),
            "plan_ms_during_replay": round(plan_ms, 3), "replay_after_next_plan_unchanged": same,
            "note": "warm, back to back; each layer reads its own K/V cache"}


def summarize(w, m, steps):
    """One workload's entry: value from the cold runs (median), warm beside it, and the
    roofline of the dominant kernel from its cold durations."""
    kv_bytes, flops, decode = workload_numbers(w, m["info"])
    per = m["cold_kernel"]
    dominant = max(per, key=per.get) if per else None
    cold, warm = _stats(m["cold"]), _stats(m["warm"])
    if decode:
        work, unit, scale = kv_bytes, "GB/s", 1e9
        bound, peak, runit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif w.dtype == "bf16":
        work, unit, scale = flops, "TFLOP/s", 1e12
        bound, peak, runit = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        work, unit, scale = flops, "TFLOP/s", 1e12
        bound, peak, runit = "alu", F32_PEAK_TFLOPS, "TFLOP/s"
    rate = lambda ms: work / (ms * 1e-3) / scale if ms else None  # noqa: E731
    res = {
        "workload": w.name, "value": round(rate(cold["median_ms"]), 3), "unit": unit,
        "ms_per_step": cold["median_ms"],
        "value_best": round(rate(cold["best_ms"]), 3),
        "value_warm": round(rate(warm["median_ms"]), 3),
        "timing": {"cold": cold, "warm": warm, "warm_wall_ms_per_step": round(m["warm_wall_ms"], 5),
                   "cold_protocol": "each run after writing 1 GiB (L2 and Infinity Cache evicted); "
                                    "HIP events around the run on its stream"},
        "work": {"kv_bytes": kv_bytes, "flops": flops, "visible_pairs": int(m["info"]["visible_pairs"])},
        "kernel_ms_cold": {k: round(v, 5) for k, v in per.items()},
        "kernel_ms_warm": {k: round(v, 5) for k, v in m["warm_kernel"].items()},
        "plan_ms": round(m["plan_ms"], 3), "warmup": m["warmup"], "schedule": m["info"],
    }
    if dominant:
        kms = per[dominant]
        achieved = rate(kms)
        wk = m["warm_kernel"].get(dominant)
        res["roofline"] = {
            "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
            "frac": round(achieved / peak, 4), "traffic": traffic_for(dominant, w.name),
            "kernel": KERNEL_NAMES[dominant], "kernel_ms": round(kms, 5),
            "kernel_timing": f"cold: mean of the kernel's own duration over {len(m['cold'])} runs, "
                             "each after a 1 GiB write (a second set of cold runs, after those that time "
                             "the steps)",
            "kernel_ms_warm": round(wk, 5) if wk else None,
            "frac_warm": round(rate(wk) / peak, 4) if wk else None,
            "kernel_source_sha": source_sha(dominant),
        }
    if not decode and w.dtype == "bf16" and dominant:
        # compulsory HBM bytes of a prefill: K and V once, Q read and out and lse written once
        elt = 2
        rows = int(w.qo_lens().sum()) * w.num_qo_heads
        hbm_bytes = kv_bytes + rows * (2 * w.head_dim * elt + 4)
        res["hbm_compulsory"] = {"bytes": hbm_bytes,
                                 "GBps": round(hbm_bytes / (per[dominant] * 1e-3) / 1e9, 1),
                                 "frac": round(hbm_bytes / (per[dominant] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
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


KEEP_BYTES = 64 << 20  # oracle results a CPU-baseline worker keeps for the parity check


def _cpu_worker(args):
    """One process: oracle passes over requests start, start+step, ... for wall_s seconds.
    Keeps the results of its first pass over each request (fp32, up to KEEP_BYTES) so that
    the bench can compare them with the GPU's outputs of the timed runs."""
    start, step, wall_s = args
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)  # one BLAS thread per process
    except Exception:  # pragma: no cover
        ctx = None
    from oracle import ref
    w = _CPU_W
    work = _request_work(w)
    done_work, done_req, i = 0, 0, start
    kept, kept_bytes = {}, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < wall_s:
        r = i % w.batch_size
        o, l = ref.run_workload(w, requests=[r])
        done_work += int(work[r])
        done_req += 1
        i += step
        a, b = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        nbytes = (b - a) * w.num_qo_heads * (w.head_dim + 1) * 4
        if r not in kept and kept_bytes + nbytes <= KEEP_BYTES:
            kept[r] = (o[a:b].astype(np.float32), l[a:b].astype(np.float32))
            kept_bytes += nbytes
    el = time.perf_counter() - t0
    del ctx  # (the limit only needs to hold while this worker runs)
    return done_work, done_req, el, kept


def _request_work(w):
    """Per request, the metric's algorithmic work: K+V bytes for a decode workload, visible
    pair FLOPs (4 x D per pair and query head) otherwise."""
    elt = 2 if w.dtype == "bf16" else 4
    g = w.num_qo_heads // w.num_kv_heads
    if bool(np.all(w.qo_lens() * g <= 8)) and w.dtype == "bf16":
        return w.kv_lens() * w.num_kv_heads * w.head_dim * 2 * elt
    qo, kv = w.qo_lens(), w.kv_lens()
    pairs = np.zeros(w.batch_size, np.int64)
    for r in range(w.batch_size):
        p = kv[r] - qo[r] + np.arange(qo[r])
        if w.mask_mode == 0:
            vis = np.full(qo[r], kv[r])
        elif w.mask_mode == 1:
            vis = np.minimum(p + 1, kv[r])
        else:
            vis = np.minimum((p // w.block_size + 1) * w.block_size, kv[r])
        pairs[r] = int(vis.sum())
    return pairs * 4 * w.head_dim * w.num_qo_heads


def cpu_baseline(w, cpu_seconds=24.0):
    """The fp64 oracle as it stands, on this host's cores: one process per core (at most 16),
    each taking whole requests (all heads) in turn for cpu_seconds / processes (at least 1 s)
    of wall time (a process finishes the request it is on).
    Must run before the process touches the GPU (the workers are forked).
    Returns the baseline record and the oracle's results per request it covered
    ({r: (out rows, lse rows)}, fp32), for the parity check of the timed outputs."""
    import multiprocessing as mp
    global _CPU_W
    _CPU_W = w
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    wall = max(1.0, cpu_seconds / n)
    ctx = mp.get_context("fork")
    with ctx.Pool(n) as pool:
        t0 = time.perf_counter()
        parts = pool.map(_cpu_worker, [(k, n, wall) for k in range(n)])
        el = time.perf_counter() - t0
    done_work = sum(p[0] for p in parts)
    done_req = sum(p[1] for p in parts)
    kept = {}
    for p in parts:
        kept.update(p[3])
    work = _request_work(w)
    decode = bool(np.all(w.qo_lens() * (w.num_qo_heads // w.num_kv_heads) <= 8)) and w.dtype == "bf16"
    scale, unit = (1e9, "GB/s") if decode else (1e12, "TFLOP/s")
    return {"value": done_work / el / scale, "unit": unit, "cores": n, "kind": "oracle",
            "host_cores": host_cores(),
            "sample": f"{done_req} request passes (all {w.num_qo_heads} heads each, {done_req / w.batch_size:.2f} "
                      f"x the workload's {w.batch_size} requests, taken in turn) by {n} processes in {el:.1f} s",
            "workload_work": int(work.sum())}, kept


def timed_output_parity(w, kept, rows_out):
    """Compares the GPU's out and lse of the timed runs (rows_out: the checked requests'
    rows, in request order) with the oracle results the CPU baseline kept, at the parity
    tolerance of the tests (bf16: 2e-2 on out, fp32: 1e-5; 1e-3 on lse)."""
    tol_o, tol_l = (2e-2, 1e-3) if w.dtype == "bf16" else (1e-5, 1e-3)
    reqs = sorted(kept)
    go, gl = rows_out
    ro = np.concatenate([kept[r][0] for r in reqs]).astype(np.float64)
    rl = np.concatenate([kept[r][1] for r in reqs]).astype(np.float64)
    fin = np.isfinite(rl)
    err_o = float(np.max(np.abs(go - ro))) if ro.size else 0.0
    err_l = float(np.max(np.abs(gl[fin] - rl[fin]))) if fin.any() else 0.0
    ok = bool(err_o <= tol_o and err_l <= tol_l and np.array_equal(np.isfinite(gl), fin)
              and not np.isnan(go).any())
    return {"requests": len(reqs), "of": w.batch_size, "rows": int(ro.shape[0]) if ro.size else 0,
            "max_abs_out_err": err_o, "max_abs_lse_err": err_l, "tol": [tol_o, tol_l], "pass": ok,
            "what": "out and lse of the last timed run against the fp64 oracle results computed by "
                    "the CPU-baseline leg for the same requests"}


def host_cores():
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    return {"affinity": aff, "cpu_count": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30,
                    help="timed runs per workload, cold (after a 1 GiB flush each) and again warm")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed runs before the timed ones (default: as many as fill %.1f s)" % WARMUP_SECONDS)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-sweep", action="store_true", help="measure the headline workload only")
    ap.add_argument("--all", action="store_true",
                    help="also measure cacheless span-to-span cross-attention, causal paged prefill, the "
                         "per-rank tensor-parallel shapes, graph replay of a 32-layer decode step and the "
                         "context write")
    ap.add_argument("--preroll", type=float, default=0.3,
                    help="seconds of cache flushes alone after the headline's warm-up runs, before its "
                         "timed runs (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="CPU seconds (summed over the worker processes) for the oracle baseline")
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

    all_workloads = {**synth.WORKLOADS, **synth.NEXT_WORKLOADS, **synth.TP_WORKLOADS}
    if args.copy_calibration:
        dev = torch.device("cuda:0")
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4}), flush=True)
        return
    log(f"[bench] generating {args.workload}")
    w = all_workloads[args.workload](0)
    cpu_line, kept = None, {}
    if not (args.no_cpu_baseline or args.context_write):
        # before anything touches the GPU: the oracle's worker processes are forked
        log(f"[bench] timing the CPU oracle on {args.workload}")
        cpu_line, kept = cpu_baseline(w, args.cpu_seconds)
        log(f"[bench] cpu baseline {json.dumps(cpu_line)}")
    dev = torch.device("cuda:0")
    if args.context_write:
        print(json.dumps(measure_write(w, args.steps, args.warmup, dev)), flush=True)
        return
    log(f"[bench] measuring {args.workload}: steps={args.steps} warmup={args.warmup}")
    # the headline is measured first in the process: after its `warmup` runs, --preroll
    # seconds of cache flushes alone bring the GPU out of its idle clocks before the timed runs
    keep_rows = None
    if kept:
        keep_rows = np.concatenate([np.arange(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])) for r in sorted(kept)])
    m = measure(w, args.steps, args.warmup, dev, preroll_s=args.preroll, keep_rows=keep_rows)
    res = summarize(w, m, args.steps)
    parity = timed_output_parity(w, kept, m["kept"]) if kept else None
    log(f"[bench] {json.dumps({k: v for k, v in res.items() if k != 'schedule'})}")
    del w, m
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": res["warmup"], "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[res_dtype(args.workload)],
        "data": "synthetic",
        "config": CONFIGS[args.workload] if args.workload in CONFIGS else {"workload": args.workload},
        "roofline": res.get("roofline"),
        "value_best": res["value_best"], "value_warm": res["value_warm"],
        "timing": res["timing"], "kernel_ms_cold": res["kernel_ms_cold"],
        "kernel_ms_warm": res["kernel_ms_warm"], "plan_ms": res["plan_ms"], "schedule": res["schedule"],
        "work": res["work"],
    }
    if "hbm_compulsory" in res:
        line["hbm_compulsory"] = res["hbm_compulsory"]
    if cpu_line is not None:
        line["cpu_baseline"] = cpu_line
    if parity is not None:
        line["parity"] = parity
        log(f"[bench] parity of the timed outputs: {json.dumps(parity)}")
    if not args.no_sweep:
        names = [n for n in synth.WORKLOADS if n != args.workload]
        if args.all:
            names += [n for n in {**synth.NEXT_WORKLOADS, **synth.TP_WORKLOADS} if n != args.workload]
        sweep = {}
        for name in names:
            log(f"[bench] sweep: generating {name}")
            ws = all_workloads[name](0)
            log(f"[bench] sweep: measuring {name}")
            ms = measure(ws, args.steps, None, dev)
            r = summarize(ws, ms, args.steps)
            r.pop("schedule", None)
            r["config"] = CONFIGS.get(name, {"workload": name})
            sweep[name] = r
            log(f"[bench] {json.dumps(r)}")
            del ws, ms
            torch.cuda.empty_cache()
        if args.all:
            log("[bench] sweep: graph replay")
            gr = measure_graph(synth.TP_WORKLOADS["whisper_decode_cross_tp4"](0), 32, args.steps, dev)
            sweep[gr["workload"]] = gr
            log(f"[bench] {json.dumps(gr)}")
            torch.cuda.empty_cache()
            log("[bench] sweep: context write")
            wr = measure_write(synth.WORKLOADS["whisper_decode_cross"](0), args.steps, None, dev)
            sweep[wr["workload"]] = wr
            log(f"[bench] {json.dumps(wr)}")
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
