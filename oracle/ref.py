"""Plain fp64 CPU oracle for paged and ragged attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The library itself never calls it, and it
shares no code with the GPU path: it takes plain numpy arrays and nothing else.

What it computes, per request r and query head h (naive gather-then-softmax):

1. Gather the request's keys and values through its page table, in order
   (page "mstar.engine.resources.attn.cross", FlashInferCrossManager: the context is
   an ordinary paged KV stream read by later steps). Cacheless spans are sliced
   directly from the packed tensors (page "mstar.engine.resources.attn.ragged.base",
   module docstring: nothing to page).
2. Widen the stored values exactly to fp64 (bf16 bit patterns or fp32).
3. Scores S = scale * Q K^T in fp64.
4. Visibility per query row i of a request with qo_len queries and kv_len keys, with
   p_i = kv_len - qo_len + i (queries are the last qo_len positions):
   * NONE: every key (cross-attention is non-causal: FlashInferCrossManager summary);
   * CAUSAL: key j <= p_i (AttentionStep.causal, page "...attn.config");
   * BLOCK_CAUSAL(B): floor(j/B) <= floor(p_i/B) (RaggedBlockCausalAttnManager:
     block-causal self-attention within each span).
5. Softmax over the visible keys: m = max S, l = sum exp(S - m), lse = m + ln l,
   O = sum exp(S - m) V / l.
6. No visible key: O = 0 and lse = -inf.

GQA: query head h reads KV head h // (Hq / Hkv) (page "mstar.model.components.attention":
grouped-query attention when num_kv_heads < num_heads).

Every function below is pinned by tests under tests/ (closed forms, invariants,
brute force, and the library routine torch.nn.functional.scaled_dot_product_attention).
"""
from __future__ import annotations

import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BLOCK_CAUSAL = 2


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values: bf16 bit patterns (uint16) or fp32 to fp64."""
    if dtype == "bf16":
        return (np.asarray(x).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def request_lengths(qo_indptr, kv_indptr, kv_last_page_len, page_size):
    """Query and context lengths per request from the packed and paged index arrays.

    qo_len[r] = qo_indptr[r+1] - qo_indptr[r] (QueryPacking: cumulative query lengths);
    kv_len[r] = (npages - 1) * page_size + last_page_len, or 0 when the request has no page.
    """
    qo_indptr = np.asarray(qo_indptr, np.int64)
    kv_indptr = np.asarray(kv_indptr, np.int64)
    qo_len = qo_indptr[1:] - qo_indptr[:-1]
    npages = kv_indptr[1:] - kv_indptr[:-1]
    if kv_last_page_len is None:
        last = np.full(len(npages), page_size, np.int64)
    else:
        last = np.asarray(kv_last_page_len, np.int64)
    kv_len = np.where(npages > 0, (npages - 1) * page_size + last, 0)
    return qo_len, kv_len


def gather_pages(pool, kv_indptr, kv_page_indices, r, kv_len, page_size, kv_head):
    """Keys (or values) of request r for one KV head, in logical order: [kv_len, D].

    pool is [num_pages, page_size, Hkv, D]; kv_page_indices None means the identity table.
    """
    lo, hi = int(kv_indptr[r]), int(kv_indptr[r + 1])
    if kv_page_indices is None:
        pages = np.arange(lo, hi)
    else:
        pages = np.asarray(kv_page_indices[lo:hi], np.int64)
    rows = pool[pages, :, kv_head, :]  # [npages, page_size, D]
    return rows.reshape(-1, rows.shape[-1])[:kv_len]


def visible(mask_mode, qo_len, kv_len, block_size):
    """Boolean [qo_len, kv_len]: which keys each query row of a request may attend to."""
    j = np.arange(kv_len)[None, :]
    p = (kv_len - qo_len + np.arange(qo_len))[:, None]
    if mask_mode == MASK_NONE:
        return np.ones((qo_len, kv_len), bool)
    if mask_mode == MASK_CAUSAL:
        return j <= p
    if mask_mode == MASK_BLOCK_CAUSAL:
        return (j // block_size) <= (p // block_size)
    raise ValueError(f"unknown mask mode {mask_mode}")


def attend(Q, K, V, vis, scale):
    """Softmax attention of Q [n, D] over K, V [m, D] with visibility vis [n, m], in fp64.

    Returns (O [n, D], lse [n]); rows with no visible key give O = 0, lse = -inf.
    """
    n, d = Q.shape
    O = np.zeros((n, V.shape[1] if V.ndim == 2 else d), np.float64)
    lse = np.full(n, -np.inf, np.float64)
    if K.shape[0] == 0 or n == 0:
        return O, lse
    S = scale * (Q @ K.T)
    S = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, S.max(axis=1), 0.0)
    P = np.where(vis, np.exp(S - m[:, None]), 0.0)
    l = P.sum(axis=1)
    ok = l > 0
    O[ok] = (P[ok] @ V) / l[ok, None]
    lse[ok] = m[ok] + np.log(l[ok])
    return O, lse


def paged_attention(q, k_pages, v_pages, qo_indptr, kv_indptr, kv_page_indices,
                    kv_last_page_len, num_qo_heads, num_kv_heads, page_size, *,
                    dtype="bf16", mask_mode=MASK_NONE, block_size=0, sm_scale=0.0,
                    requests=None, heads=None):
    """The oracle: out [sum qo, Hq, D] and lse [sum qo, Hq], both fp64.

    ``requests``/``heads`` restrict the work to a subset (other rows are left NaN), so
    that a sample of a large workload can be checked one request and head at a time.
    """
    if num_qo_heads % num_kv_heads != 0:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    group = num_qo_heads // num_kv_heads
    d = q.shape[-1]
    scale = sm_scale if sm_scale > 0 else 1.0 / math.sqrt(d)
    qo_len, kv_len = request_lengths(qo_indptr, kv_indptr, kv_last_page_len, page_size)
    nq = int(np.asarray(qo_indptr)[-1])
    out = np.full((nq, num_qo_heads, d), np.nan)
    lse = np.full((nq, num_qo_heads), np.nan)
    reqs = range(len(qo_len)) if requests is None else requests
    hs = range(num_qo_heads) if heads is None else heads
    for r in reqs:
        q0, nqr, nkv = int(qo_indptr[r]), int(qo_len[r]), int(kv_len[r])
        if nqr == 0:
            continue
        vis = visible(mask_mode, nqr, nkv, block_size)
        for h in hs:
            hk = h // group
            K = to_f64(gather_pages(k_pages, kv_indptr, kv_page_indices, r, nkv, page_size, hk), dtype)
            V = to_f64(gather_pages(v_pages, kv_indptr, kv_page_indices, r, nkv, page_size, hk), dtype)
            Q = to_f64(q[q0:q0 + nqr, h, :], dtype)
            o, s = attend(Q, K, V, vis, scale)
            out[q0:q0 + nqr, h, :] = o
            lse[q0:q0 + nqr, h] = s
    return out, lse


def ragged_attention(q, k, v, cu_seqlens, num_qo_heads, num_kv_heads, *, dtype="bf16",
                     mask_mode=MASK_BLOCK_CAUSAL, block_size=64, sm_scale=0.0,
                     requests=None, heads=None, cu_seqlens_kv=None):
    """Cacheless attention over spans of packed tensors: no page table.

    q is [Tq, Hq, D] with request r's queries at rows cu_seqlens[r] .. cu_seqlens[r+1].
    k and v are [Tkv, Hkv, D] (or [Tkv, 1, Hkv, D]); request r's keys are the same span
    (self-attention within each span, page "mstar.engine.resources.attn.ragged.base",
    RaggedAttnManager and RaggedBlockCausalAttnManager) or, with cu_seqlens_kv, the span
    cu_seqlens_kv[r] .. cu_seqlens_kv[r+1] of a second packed tensor (cross-attention
    between two spans of each request, RaggedCrossAttnManager on the same page). Query i
    of a span sits at key position kv_len - qo_len + i for the causal masks.
    """
    group = num_qo_heads // num_kv_heads
    d = q.shape[-1]
    scale = sm_scale if sm_scale > 0 else 1.0 / math.sqrt(d)
    cu = np.asarray(cu_seqlens, np.int64)
    cukv = cu if cu_seqlens_kv is None else np.asarray(cu_seqlens_kv, np.int64)
    k = k.reshape(k.shape[0] * (k.shape[1] if k.ndim == 4 else 1), num_kv_heads, d)
    v = v.reshape(v.shape[0] * (v.shape[1] if v.ndim == 4 else 1), num_kv_heads, d)
    t = int(cu[-1])
    out = np.full((t, num_qo_heads, d), np.nan)
    lse = np.full((t, num_qo_heads), np.nan)
    reqs = range(len(cu) - 1) if requests is None else requests
    hs = range(num_qo_heads) if heads is None else heads
    for r in reqs:
        a, b = int(cu[r]), int(cu[r + 1])
        ka, kb = int(cukv[r]), int(cukv[r + 1])
        if b == a:
            continue
        vis = visible(mask_mode, b - a, kb - ka, block_size)
        for h in hs:
            hk = h // group
            o, s = attend(to_f64(q[a:b, h], dtype), to_f64(k[ka:kb, hk], dtype),
                          to_f64(v[ka:kb, hk], dtype), vis, scale)
            out[a:b, h] = o
            lse[a:b, h] = s
    return out, lse


def merge_states(outs, lses):
    """Combine attention over disjoint key sets: the log-sum-exp merge, in fp64.

    outs [c, n, D], lses [c, n] -> (O [n, D], lse [n]). Parts with lse = -inf carry no
    weight; if every part is empty the result is O = 0, lse = -inf.
    """
    outs = np.asarray(outs, np.float64)
    lses = np.asarray(lses, np.float64)
    M = lses.max(axis=0)
    fin = np.isfinite(M)
    Ms = np.where(fin, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms[None, :]), 0.0)
    tot = w.sum(axis=0)
    O = np.zeros(outs.shape[1:])
    O[fin] = (np.einsum("cn,cnd->nd", w, outs)[fin]) / tot[fin, None]
    lse = np.where(fin, Ms + np.log(np.where(fin, tot, 1.0)), -np.inf)
    return O, lse


def write_context(k_src, v_src, k_pages, v_pages, kv_indptr, kv_page_indices, kv_last_page_len,
                  page_size):
    """The context write that precedes the path: each request's keys and values, packed
    in request order as (length, heads, head_dim) rows, go into the slots of its pages
    (page "mstar.engine.resources.attn.cross": the context is written once and then read
    as a paged KV stream; page "mstar.model.components.attention", CrossAttention.compute_kv
    gives a request's keys and values as (length, heads, head_dim)).

    Position t of request r takes slot t % page_size of the page the table lists at
    logical page t // page_size. Returns new pools; every other slot keeps its value.
    """
    kp, vp = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    _, kv_len = request_lengths(np.zeros(len(kv_indptr), np.int64), kv_indptr, kv_last_page_len,
                                page_size)
    start = 0
    for r in range(len(kv_indptr) - 1):
        for t in range(int(kv_len[r])):
            logical = int(kv_indptr[r]) + t // page_size
            page = logical if kv_page_indices is None else int(kv_page_indices[logical])
            kp[page, t % page_size] = k_src[start + t]
            vp[page, t % page_size] = v_src[start + t]
        start += int(kv_len[r])
    return kp, vp


def run_workload(w, requests=None, heads=None):
    """Oracle over a synth.Workload-like object (paged or cacheless)."""
    if w.kv_page_indices is None and w.page_size == 1 and "cu_seqlens" in getattr(w, "meta", {}):
        return ragged_attention(w.q, w.k_pages, w.v_pages, w.meta["cu_seqlens"], w.num_qo_heads,
                                w.num_kv_heads, dtype=w.dtype, mask_mode=w.mask_mode,
                                block_size=w.block_size, sm_scale=w.sm_scale,
                                requests=requests, heads=heads,
                                cu_seqlens_kv=w.meta.get("cu_seqlens_kv"))
    return paged_attention(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr, w.kv_page_indices,
                           w.kv_last_page_len, w.num_qo_heads, w.num_kv_heads, w.page_size,
                           dtype=w.dtype, mask_mode=w.mask_mode, block_size=w.block_size,
                           sm_scale=w.sm_scale, requests=requests, heads=heads)
