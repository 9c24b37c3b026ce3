"""The oracle over a whole full-size workload, one request at a time on a pool of threads.

Test infrastructure: the oracle's own entry point (``ref.run_workload``) is called on a
one-request view of the workload (the request's query rows and its slice of the page
table, or of the packed spans; the pools are shared, not copied), so that requests run
in parallel and no call allocates the whole output. numpy releases the interpreter lock
inside its array kernels and BLAS calls, so the threads run concurrently; BLAS itself is
held to one thread each. The assembled result equals ``ref.run_workload(w)`` exactly
(``tests/test_oracle_threads.py``).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import ref
from ragged_attention_serving_amd import synth


def request_view(w: synth.Workload, r: int) -> synth.Workload:
    """A one-request workload for request r of w, sharing w's tensors."""
    q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
    meta = getattr(w, "meta", {}) or {}
    if "cu_seqlens" in meta and w.kv_page_indices is None and w.page_size == 1:
        cu = np.asarray(meta["cu_seqlens"], np.int64)
        cukv = np.asarray(meta.get("cu_seqlens_kv", cu), np.int64)
        a, b = int(cu[r]), int(cu[r + 1])
        ka, kb = int(cukv[r]), int(cukv[r + 1])
        sub_meta = {"cu_seqlens": np.array([0, b - a], np.int32)}
        if "cu_seqlens_kv" in meta:
            sub_meta["cu_seqlens_kv"] = np.array([0, kb - ka], np.int32)
        kv_ind = np.array([0, kb - ka if "cu_seqlens_kv" in meta else b - a], np.int32)
        return synth.Workload(name=f"{w.name}[{r}]", dtype=w.dtype, qo_indptr=np.array([0, b - a], np.int32),
                              kv_indptr=kv_ind, kv_page_indices=None, kv_last_page_len=None,
                              num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                              head_dim=w.head_dim, page_size=1, mask_mode=w.mask_mode,
                              block_size=w.block_size, sm_scale=w.sm_scale, q=w.q[a:b],
                              k_pages=w.k_pages[ka:kb], v_pages=w.v_pages[ka:kb], meta=sub_meta)
    p0, p1 = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
    pages = (np.arange(p0, p1, dtype=np.int32) if w.kv_page_indices is None
             else np.asarray(w.kv_page_indices[p0:p1], np.int32))
    last = None if w.kv_last_page_len is None else np.array([w.kv_last_page_len[r]], np.int32)
    return synth.Workload(name=f"{w.name}[{r}]", dtype=w.dtype, qo_indptr=np.array([0, q1 - q0], np.int32),
                          kv_indptr=np.array([0, p1 - p0], np.int32), kv_page_indices=pages,
                          kv_last_page_len=last, num_qo_heads=w.num_qo_heads,
                          num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                          mask_mode=w.mask_mode, block_size=w.block_size, sm_scale=w.sm_scale,
                          q=w.q[q0:q1], k_pages=w.k_pages, v_pages=w.v_pages)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_by_request(w: synth.Workload, threads: int | None = None, requests=None):
    """(out, lse) of the oracle over every request of w (or the given ones; other rows NaN),
    computed request by request on `threads` threads, longest contexts first."""
    threads = threads or default_threads()
    nq = int(w.qo_indptr[-1])
    out = np.full((nq, w.num_qo_heads, w.head_dim), np.nan)
    lse = np.full((nq, w.num_qo_heads), np.nan)
    reqs = list(range(w.batch_size)) if requests is None else list(requests)
    cost = w.qo_lens() * w.kv_lens() + w.kv_lens()
    reqs.sort(key=lambda r: -int(cost[r]))

    def work(r):
        o, s = ref.run_workload(request_view(w, r))
        q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        out[q0:q1] = o
        lse[q0:q1] = s

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, reqs))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return out, lse
