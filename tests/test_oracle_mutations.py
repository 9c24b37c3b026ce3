"""Plant plausible mistakes in copies of the oracle; each must trip at least one pin.

The mistakes are planted in the oracle only, on the CPU, by swapping one of its
functions for a broken variant for the duration of one check.
"""
import numpy as np
import pytest

import oracle.ref as ref
from tests import oracle_pins

_orig = {n: getattr(ref, n) for n in ("to_f64", "request_lengths", "gather_pages", "visible",
                                      "attend", "merge_states", "ragged_attention", "paged_attention",
                                      "write_context", "run_workload")}


def _gather_reversed_pages(pool, kv_indptr, kv_page_indices, r, kv_len, page_size, kv_head):
    lo, hi = int(kv_indptr[r]), int(kv_indptr[r + 1])
    pages = np.arange(lo, hi) if kv_page_indices is None else np.asarray(kv_page_indices[lo:hi])
    rows = pool[pages[::-1], :, kv_head, :]
    return rows.reshape(-1, rows.shape[-1])[:kv_len]


def _gather_ignores_table(pool, kv_indptr, kv_page_indices, r, kv_len, page_size, kv_head):
    return _orig["gather_pages"](pool, kv_indptr, None, r, kv_len, page_size, kv_head)


def _gather_wrong_head(pool, kv_indptr, kv_page_indices, r, kv_len, page_size, kv_head):
    return _orig["gather_pages"](pool, kv_indptr, kv_page_indices, r, kv_len, page_size,
                                 (kv_head + 1) % pool.shape[2])


def _visible_top_left(mask_mode, qo_len, kv_len, block_size):
    if mask_mode == ref.MASK_NONE:
        return np.ones((qo_len, kv_len), bool)
    j = np.arange(kv_len)[None, :]
    i = np.arange(qo_len)[:, None]
    return j <= i if mask_mode == ref.MASK_CAUSAL else (j // block_size) <= (i // block_size)


def _visible_block_strict(mask_mode, qo_len, kv_len, block_size):
    if mask_mode != ref.MASK_BLOCK_CAUSAL:
        return _orig["visible"](mask_mode, qo_len, kv_len, block_size)
    j = np.arange(kv_len)[None, :]
    p = (kv_len - qo_len + np.arange(qo_len))[:, None]
    return (j // block_size) < (p // block_size) + (j <= p)  # own block only up to the diagonal


def _visible_causal_off_by_one(mask_mode, qo_len, kv_len, block_size):
    if mask_mode != ref.MASK_CAUSAL:
        return _orig["visible"](mask_mode, qo_len, kv_len, block_size)
    j = np.arange(kv_len)[None, :]
    p = (kv_len - qo_len + np.arange(qo_len))[:, None]
    return j < p


def _attend_no_scale(Q, K, V, vis, scale):
    return _orig["attend"](Q, K, V, vis, 1.0)


def _attend_lse_without_max(Q, K, V, vis, scale):
    O, lse = _orig["attend"](Q, K, V, vis, scale)
    if K.shape[0] == 0:
        return O, lse
    S = np.where(vis, scale * (Q @ K.T), -np.inf)
    m = np.where(vis.any(1), S.max(1), 0.0)
    return O, lse - m


def _attend_ignores_mask(Q, K, V, vis, scale):
    return _orig["attend"](Q, K, V, np.ones_like(vis) & vis.any(1, keepdims=True), scale)


def _attend_unnormalised(Q, K, V, vis, scale):
    O, lse = _orig["attend"](Q, K, V, vis, scale)
    if K.shape[0] == 0:
        return O, lse
    S = np.where(vis, scale * (Q @ K.T), -np.inf)
    m = np.where(vis.any(1), S.max(1), 0.0)
    l = np.where(vis, np.exp(S - m[:, None]), 0).sum(1)
    return O * np.where(l > 0, l, 1)[:, None], lse


def _attend_transposed_v(Q, K, V, vis, scale):
    if V.shape[0] == V.shape[1]:
        V = V.T
    O, lse = _orig["attend"](Q, K, V, vis, scale)
    return O[:, ::-1] if O.shape[1] > 1 else O, lse


def _lengths_full_last_page(qo_indptr, kv_indptr, kv_last_page_len, page_size):
    return _orig["request_lengths"](qo_indptr, kv_indptr, None, page_size)


def _widen_wrong_shift(x, dtype):
    if dtype == "bf16":
        return (np.asarray(x).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return np.asarray(x, np.float64)


def _merge_no_weights(outs, lses):
    outs = np.asarray(outs, np.float64)
    lses = np.asarray(lses, np.float64)
    M = lses.max(0)
    return outs.mean(0), M


def _ragged_keys_from_query_spans(*args, **kw):
    kw.pop("cu_seqlens_kv", None)
    return _orig["ragged_attention"](*args, **kw)


def _write_slot_from_page_index(k_src, v_src, k_pages, v_pages, kv_indptr, kv_page_indices,
                                kv_last_page_len, page_size):
    kp, vp = np.array(k_pages, copy=True), np.array(v_pages, copy=True)
    _, kv_len = ref.request_lengths(np.zeros(len(kv_indptr), np.int64), kv_indptr, kv_last_page_len,
                                    page_size)
    start = 0
    for r in range(len(kv_indptr) - 1):
        for t in range(int(kv_len[r])):
            logical = int(kv_indptr[r]) + t // page_size
            page = logical if kv_page_indices is None else int(kv_page_indices[logical])
            kp[page, (t // page_size) % page_size] = k_src[start + t]
            vp[page, (t // page_size) % page_size] = v_src[start + t]
        start += int(kv_len[r])
    return kp, vp


def _write_ignores_table(k_src, v_src, k_pages, v_pages, kv_indptr, kv_page_indices,
                         kv_last_page_len, page_size):
    return _orig["write_context"](k_src, v_src, k_pages, v_pages, kv_indptr, None, kv_last_page_len,
                                  page_size)


def _write_clears_tails(k_src, v_src, k_pages, v_pages, kv_indptr, kv_page_indices,
                        kv_last_page_len, page_size):
    kp, vp = _orig["write_context"](k_src, v_src, k_pages, v_pages, kv_indptr, kv_page_indices,
                                    kv_last_page_len, page_size)
    kp[:, -1] = 0
    vp[:, -1] = 0
    return kp, vp


def _workload_drops_kv_spans(w, requests=None, heads=None):
    """Routes cross-attention spans as self-attention: keys taken from the query spans."""
    meta = dict(getattr(w, "meta", {}))
    meta.pop("cu_seqlens_kv", None)
    saved = w.meta
    w.meta = meta
    try:
        return _orig["run_workload"](w, requests=requests, heads=heads)
    finally:
        w.meta = saved


def _workload_cacheless_as_paged_rows(w, requests=None, heads=None):
    """Takes the query spans' offsets for the key spans of cacheless workloads."""
    if "cu_seqlens" not in getattr(w, "meta", {}):
        return _orig["run_workload"](w, requests=requests, heads=heads)
    return _orig["ragged_attention"](w.q, w.k_pages, w.v_pages, w.meta["cu_seqlens"], w.num_qo_heads,
                                     w.num_kv_heads, dtype=w.dtype, mask_mode=w.mask_mode,
                                     block_size=w.block_size, sm_scale=w.sm_scale, requests=requests,
                                     heads=heads, cu_seqlens_kv=w.meta["cu_seqlens"])


def _subset_rows_shifted(name):
    """A subset run whose rows land one row off (the full run is untouched)."""
    def f(*args, requests=None, heads=None, **kw):
        out, lse = _orig[name](*args, requests=requests, heads=heads, **kw)
        if requests is not None:
            out, lse = np.roll(out, 1, axis=0), np.roll(lse, 1, axis=0)
        return out, lse
    return f


def _subset_ignores_heads(name):
    """A subset run that computes every head, not only the requested ones."""
    def f(*args, requests=None, heads=None, **kw):
        return _orig[name](*args, requests=requests, heads=None, **kw)
    return f


MUTATIONS = {
    "workload_drops_kv_spans": ("run_workload", _workload_drops_kv_spans),
    "workload_kv_spans_from_query_spans": ("run_workload", _workload_cacheless_as_paged_rows),
    "paged_subset_rows_shifted": ("paged_attention", _subset_rows_shifted("paged_attention")),
    "ragged_subset_rows_shifted": ("ragged_attention", _subset_rows_shifted("ragged_attention")),
    "paged_subset_ignores_heads": ("paged_attention", _subset_ignores_heads("paged_attention")),
    "ragged_subset_ignores_heads": ("ragged_attention", _subset_ignores_heads("ragged_attention")),
    "write_slot_from_page_index": ("write_context", _write_slot_from_page_index),
    "write_ignores_table": ("write_context", _write_ignores_table),
    "write_clears_tails": ("write_context", _write_clears_tails),
    "ragged_keys_from_query_spans": ("ragged_attention", _ragged_keys_from_query_spans),
    "gather_reversed_pages": ("gather_pages", _gather_reversed_pages),
    "gather_ignores_table": ("gather_pages", _gather_ignores_table),
    "gather_wrong_head": ("gather_pages", _gather_wrong_head),
    "visible_top_left": ("visible", _visible_top_left),
    "visible_block_strict": ("visible", _visible_block_strict),
    "visible_causal_off_by_one": ("visible", _visible_causal_off_by_one),
    "attend_no_scale": ("attend", _attend_no_scale),
    "attend_lse_without_max": ("attend", _attend_lse_without_max),
    "attend_ignores_mask": ("attend", _attend_ignores_mask),
    "attend_unnormalised": ("attend", _attend_unnormalised),
    "attend_transposed_v": ("attend", _attend_transposed_v),
    "lengths_full_last_page": ("request_lengths", _lengths_full_last_page),
    "widen_wrong_shift": ("to_f64", _widen_wrong_shift),
    "merge_no_weights": ("merge_states", _merge_no_weights),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ref, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(ref)
        except Exception as e:  # an assertion, or a shape error from a transposed operand
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    for pin in oracle_pins.ALL_PINS:
        pin(ref)
