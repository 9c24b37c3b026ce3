"""Seeded synthetic inputs for paged and ragged attention.

This module is shared by the GPU path, the CPU oracle and the benchmark. It holds
none of the attention arithmetic: it only draws lengths, page tables and N(0,1)
tensors, and rounds fp32 draws to bf16 bit patterns (round to nearest even).

Layouts follow the library's reading of the pages (mstar.engine.resources.attn.cross,
FlashInferCrossManager: "non-causal paged attention over fixed encoder context";
QueryPacking: requests in packed order plus cumulative query lengths):

* ``qo_indptr[B+1]``: cumulative query lengths, in tokens.
* ``kv_indptr[B+1]``: cumulative page counts per request.
* ``kv_page_indices[kv_indptr[B]]``: physical page of each logical page, requests in
  order; ``None`` means the identity table (cacheless spans, page_size 1).
* ``kv_last_page_len[B]``: valid tokens in each request's last page, in [1, page_size].
* ``q``: ``[sum(qo), Hq, D]``; ``k_pages``/``v_pages``: ``[num_pages, page_size, Hkv, D]``.

bf16 tensors are numpy ``uint16`` arrays of bf16 bit patterns; fp32 tensors are
``float32``.

Draw order for a workload built from ``np.random.default_rng(seed)``: lengths, then
the page permutation. Tensors (Q, then the K pool, then the V pool) are drawn from
independent child streams ``default_rng([seed, tensor_id, chunk])`` over fixed
chunks of ``CHUNK_ELEMS`` elements, so that they can be drawn by several threads
and still be the same for every thread count.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BLOCK_CAUSAL = 2

CHUNK_ELEMS = 1 << 24  # elements per independent child stream
TENSOR_Q, TENSOR_K, TENSOR_V = 1, 2, 3
TENSOR_CTX_K, TENSOR_CTX_V = 4, 5  # packed context rows for the context write


@dataclass
class Workload:
    """One batch of synthetic input for the plan/run entry points."""

    name: str
    dtype: str  # "f32" or "bf16"
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_page_indices: np.ndarray | None
    kv_last_page_len: np.ndarray | None
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    mask_mode: int = MASK_NONE
    block_size: int = 0
    sm_scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)
    q: np.ndarray | None = None
    k_pages: np.ndarray | None = None
    v_pages: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def batch_size(self) -> int:
        return len(self.qo_indptr) - 1

    @property
    def num_pages(self) -> int:
        return 0 if self.k_pages is None else int(self.k_pages.shape[0])

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def qo_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr.astype(np.int64))

    def kv_lens(self) -> np.ndarray:
        """Context length of each request, from the page table (0 for no pages)."""
        npages = np.diff(self.kv_indptr.astype(np.int64))
        last = (np.full(len(npages), self.page_size, np.int64) if self.kv_last_page_len is None
                else self.kv_last_page_len.astype(np.int64))
        return np.where(npages > 0, (npages - 1) * self.page_size + last, 0)


# ---------------------------------------------------------------- helpers

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs; NaN kept NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (used only to build test inputs)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_tensor(shape, seed: int, tensor_id: int, dtype: str) -> np.ndarray:
    """N(0,1) tensor drawn in fixed chunks from child streams; bf16 as bit patterns."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    nchunks = (n + CHUNK_ELEMS - 1) // CHUNK_ELEMS

    def work(c: int) -> None:
        lo, hi = c * CHUNK_ELEMS, min(n, (c + 1) * CHUNK_ELEMS)
        g = np.random.default_rng([seed, tensor_id, c])
        x = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = round_to_bf16_bits(x) if dtype == "bf16" else x

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def page_table(kv_lens, page_size: int, perm: np.ndarray | None):
    """CSR page table for requests of the given context lengths.

    Logical pages are numbered in request order; ``perm`` maps logical page i to
    physical page perm[i] (None keeps the identity).
    """
    kv_lens = np.asarray(kv_lens, np.int64)
    npages = (kv_lens + page_size - 1) // page_size
    kv_indptr = np.zeros(len(kv_lens) + 1, np.int64)
    kv_indptr[1:] = np.cumsum(npages)
    last = np.where(npages > 0, kv_lens - (npages - 1) * page_size, page_size)
    total = int(kv_indptr[-1])
    idx = np.arange(total, dtype=np.int64) if perm is None else np.asarray(perm, np.int64)
    return kv_indptr.astype(np.int32), idx.astype(np.int32), last.astype(np.int32), total


def indptr(lens) -> np.ndarray:
    out = np.zeros(len(lens) + 1, np.int64)
    out[1:] = np.cumsum(np.asarray(lens, np.int64))
    return out.astype(np.int32)


# ---------------------------------------------------------------- generic builders

def paged_case(qo_lens, kv_lens, num_qo_heads, num_kv_heads, head_dim, page_size, *,
               dtype="bf16", mask_mode=MASK_NONE, block_size=0, seed=0, shuffle=True,
               tail="normal", extra_pages=0, name="paged", sm_scale=0.0,
               rng: np.random.Generator | None = None) -> Workload:
    """Paged workload: requests with the given query and context lengths.

    ``tail`` sets what the unused slots of each request's last page hold:
    "normal" (the N(0,1) draw) or "nan" (a poison that must never reach a result).
    ``extra_pages`` adds unreferenced pages to the pool.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    kv_indptr, _, last, total = page_table(kv_lens, page_size, None)
    num_pages = total + int(extra_pages)
    perm = rng.permutation(num_pages)[:total] if shuffle else np.arange(total)
    kv_page_indices = perm.astype(np.int32)
    qo_indptr = indptr(qo_lens)
    nq = int(qo_indptr[-1])
    q = normal_tensor((nq, num_qo_heads, head_dim), seed, TENSOR_Q, dtype)
    kp = normal_tensor((num_pages, page_size, num_kv_heads, head_dim), seed, TENSOR_K, dtype)
    vp = normal_tensor((num_pages, page_size, num_kv_heads, head_dim), seed, TENSOR_V, dtype)
    if tail == "nan":
        poison = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
        for r in range(len(kv_lens)):
            npg = int(kv_indptr[r + 1] - kv_indptr[r])
            if npg == 0:
                continue
            p = int(kv_page_indices[kv_indptr[r + 1] - 1])
            kp[p, int(last[r]):] = poison
            vp[p, int(last[r]):] = poison
        used = np.zeros(num_pages, bool)
        used[kv_page_indices] = True
        kp[~used] = poison
        vp[~used] = poison
    return Workload(name=name, dtype=dtype, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                    kv_page_indices=kv_page_indices, kv_last_page_len=last,
                    num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    page_size=page_size, mask_mode=mask_mode, block_size=block_size,
                    sm_scale=sm_scale, q=q, k_pages=kp, v_pages=vp)


def ragged_case(span_lens, num_heads, head_dim, *, num_kv_heads=None, dtype="bf16",
                mask_mode=MASK_BLOCK_CAUSAL, block_size=64, seed=0, name="ragged",
                sm_scale=0.0) -> Workload:
    """Cacheless spans packed by cu_seqlens, expressed as the identity page table.

    q, k and v are ``[T, H, D]``; the pools are k/v viewed as ``[T, 1, Hkv, D]``
    (page_size 1, kv_indptr == qo_indptr == cu_seqlens, no page indices, every page full).
    """
    hkv = num_heads if num_kv_heads is None else num_kv_heads
    cu = indptr(span_lens)
    t = int(cu[-1])
    q = normal_tensor((t, num_heads, head_dim), seed, TENSOR_Q, dtype)
    k = normal_tensor((t, 1, hkv, head_dim), seed, TENSOR_K, dtype)
    v = normal_tensor((t, 1, hkv, head_dim), seed, TENSOR_V, dtype)
    return Workload(name=name, dtype=dtype, qo_indptr=cu, kv_indptr=cu.copy(),
                    kv_page_indices=None, kv_last_page_len=None, num_qo_heads=num_heads,
                    num_kv_heads=hkv, head_dim=head_dim, page_size=1, mask_mode=mask_mode,
                    block_size=block_size, sm_scale=sm_scale, q=q, k_pages=k, v_pages=v,
                    meta={"cu_seqlens": cu})


def ragged_cross_case(q_lens, kv_lens, num_heads, head_dim, *, num_kv_heads=None,
                      dtype="bf16", seed=0, name="ragged_cross", sm_scale=0.0) -> Workload:
    """Cacheless cross-attention between two spans of each request: queries packed by
    cu_q = indptr(q_lens), keys and values by cu_kv = indptr(kv_lens), no mask.

    q is ``[Tq, H, D]``; the pools are k/v ``[Tkv, Hkv, D]`` viewed as ``[Tkv, 1, Hkv, D]``
    (page_size 1, qo_indptr = cu_q, kv_indptr = cu_kv, no page indices).
    """
    hkv = num_heads if num_kv_heads is None else num_kv_heads
    cu_q, cu_kv = indptr(q_lens), indptr(kv_lens)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    q = normal_tensor((tq, num_heads, head_dim), seed, TENSOR_Q, dtype)
    k = normal_tensor((tkv, 1, hkv, head_dim), seed, TENSOR_K, dtype)
    v = normal_tensor((tkv, 1, hkv, head_dim), seed, TENSOR_V, dtype)
    return Workload(name=name, dtype=dtype, qo_indptr=cu_q, kv_indptr=cu_kv,
                    kv_page_indices=None, kv_last_page_len=None, num_qo_heads=num_heads,
                    num_kv_heads=hkv, head_dim=head_dim, page_size=1, mask_mode=MASK_NONE,
                    block_size=0, sm_scale=sm_scale, q=q, k_pages=k, v_pages=v,
                    meta={"cu_seqlens": cu_q, "cu_seqlens_kv": cu_kv})


def context_source(w: Workload, seed: int = 0):
    """Packed context keys and values for w's requests: ``[sum kv_len, Hkv, D]`` each, in
    request order, drawn like the other tensors (N(0,1), rounded to bf16 for bf16)."""
    rows = int(w.kv_lens().sum())
    shape = (rows, w.num_kv_heads, w.head_dim)
    return (normal_tensor(shape, seed, TENSOR_CTX_K, w.dtype),
            normal_tensor(shape, seed, TENSOR_CTX_V, w.dtype))


# ---------------------------------------------------------------- the five workloads

# Length draws, the first draws of each workload's generator (the page permutation and
# the tensors follow from the same generator or from child streams).

def ragged_prefill_query_lengths(rng: np.random.Generator) -> np.ndarray:
    """32 query lengths, uniform integers in [1, 448]."""
    return rng.integers(1, 448, 32, endpoint=True)


def block_causal_span_lengths(rng: np.random.Generator) -> np.ndarray:
    """64 span lengths, uniform integers in [256, 4096]."""
    return rng.integers(256, 4096, 64, endpoint=True)


def gqa_decode_context_lengths(rng: np.random.Generator) -> np.ndarray:
    """256 context lengths, log-uniform in [512, 32768], rounded to the nearest integer."""
    return np.rint(np.exp(rng.uniform(math.log(512), math.log(32768), 256))).astype(np.int64)


def tiny_cross(seed: int = 0) -> Workload:
    """Tiny fp32 non-causal paged cross-attention: query lens [1,3], context [16,40],
    2 heads, head_dim 16, page_size 4, shuffled pages."""
    return paged_case([1, 3], [16, 40], 2, 2, 16, 4, dtype="f32", seed=seed, name="tiny_cross_f32")


def whisper_decode(seed: int = 0) -> Workload:
    """Whisper-large-style decode cross-attention: 64 requests x 1 query, context 1500,
    20 heads (MHA), head_dim 64, bf16, page_size 16, shuffled pages, scale 1/sqrt(64)."""
    return paged_case([1] * 64, [1500] * 64, 20, 20, 64, 16, dtype="bf16", seed=seed,
                      name="whisper_decode_cross", sm_scale=1.0 / 8.0)


def ragged_prefill(seed: int = 0) -> Workload:
    """Ragged prefill cross-attention: 32 requests, query lens U[1,448], context 1500,
    20 heads, head_dim 64, bf16, page_size 16, shuffled pages."""
    rng = np.random.default_rng(seed)
    qo = ragged_prefill_query_lengths(rng)
    return paged_case(qo, [1500] * 32, 20, 20, 64, 16, dtype="bf16", seed=seed, rng=rng,
                      name="ragged_prefill_cross")


def block_causal(seed: int = 0) -> Workload:
    """Cacheless ragged block-causal self-attention: 64 spans U[256,4096], block 64,
    16 heads, head_dim 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = block_causal_span_lengths(rng)
    return ragged_case(lens, 16, 128, dtype="bf16", mask_mode=MASK_BLOCK_CAUSAL, block_size=64,
                       seed=seed, name="block_causal_ragged")


def gqa_decode(seed: int = 0) -> Workload:
    """Causal GQA paged decode: 256 requests x 1 query, 32 q / 8 kv heads, head_dim 128,
    bf16, page_size 16, context lens log-uniform in [512, 32768], shuffled pages."""
    rng = np.random.default_rng(seed)
    kv = gqa_decode_context_lengths(rng)
    return paged_case([1] * 256, kv, 32, 8, 128, 16, dtype="bf16", mask_mode=MASK_CAUSAL,
                      seed=seed, rng=rng, name="gqa_decode_causal")


def gqa_decode_tp8(seed: int = 0) -> Workload:
    """One rank's share of the GQA decode under tensor parallelism over heads, degree 8
    (page "mstar.model.components.distributed.attention", ParallelAttention: each rank
    holds num_heads / tp query heads and num_kv_heads / tp KV heads): 4 q heads and 1 KV
    head per rank, the same 256 contexts and pages."""
    rng = np.random.default_rng(seed)
    kv = gqa_decode_context_lengths(rng)
    return paged_case([1] * 256, kv, 4, 1, 128, 16, dtype="bf16", mask_mode=MASK_CAUSAL,
                      seed=seed, rng=rng, name="gqa_decode_causal_tp8")


def whisper_decode_tp4(seed: int = 0) -> Workload:
    """One rank's share of the Whisper-style decode at tensor parallelism 4: 5 of the 20
    heads (query and KV alike), the same 64 contexts of 1500 positions."""
    return paged_case([1] * 64, [1500] * 64, 5, 5, 64, 16, dtype="bf16", seed=seed,
                      name="whisper_decode_cross_tp4", sm_scale=1.0 / 8.0)


def ragged_cross_spans(seed: int = 0) -> Workload:
    """Cacheless span-to-span cross-attention (page "mstar.engine.resources.attn.ragged.base",
    RaggedCrossAttnManager: each request attends from its query span to its own key span, no
    page table): 32 requests, query spans U[1,448], key spans U[256,4096], 16 heads,
    head_dim 128, bf16, no mask."""
    rng = np.random.default_rng(seed)
    qo = rng.integers(1, 448, 32, endpoint=True)
    kv = rng.integers(256, 4096, 32, endpoint=True)
    return ragged_cross_case(qo, kv, 16, 128, dtype="bf16", seed=seed, name="ragged_cross_spans")


def causal_prefill_paged(seed: int = 0) -> Workload:
    """Multi-token causal prefill over a paged cache (page "mstar.engine.resources.attn.config",
    AttentionStep.causal; page "mstar.model.components.attention", grouped KV heads): 16 requests
    whose whole context is new (qo_len = kv_len, uniform 256-4096), 32 query / 8 KV heads,
    head_dim 128, bf16, page_size 16, shuffled pages."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(256, 4096, 16, endpoint=True)
    return paged_case(lens, lens, 32, 8, 128, 16, dtype="bf16", mask_mode=MASK_CAUSAL, seed=seed,
                      rng=rng, name="causal_prefill_paged")


WORKLOADS = {
    "tiny_cross_f32": tiny_cross,
    "whisper_decode_cross": whisper_decode,
    "ragged_prefill_cross": ragged_prefill,
    "block_causal_ragged": block_causal,
    "gqa_decode_causal": gqa_decode,
}

# the variants of the path beyond the five workloads: cacheless span-to-span cross-attention
# and multi-token causal prefill over a paged cache, measured by `bench.py --all`
NEXT_WORKLOADS = {
    "ragged_cross_spans": ragged_cross_spans,
    "causal_prefill_paged": causal_prefill_paged,
}

# per-rank shapes of tensor parallelism over heads, measured on one GPU
TP_WORKLOADS = {
    "gqa_decode_causal_tp8": gqa_decode_tp8,
    "whisper_decode_cross_tp4": whisper_decode_tp4,
}
