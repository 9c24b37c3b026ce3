"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Tolerances: bf16 inputs max |out error| <= 2e-2, fp32 inputs <= 1e-5; lse <= 1e-3.
The seeded workloads are compared at full size on every output row and head (the
block-causal spans and the GQA decode with the oracle computed request by request on
host threads); small cases cover every kernel family, mask, head grouping, page size,
split and edge case.
"""
import time

import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.gpu_util import compare, log, run_gpu, to_device
from tests.oracle_threads import oracle_by_request

pytestmark = pytest.mark.gpu


def _full(w, gpu, chunk=0):
    log(f"[parity] {w.name} chunk={chunk}")
    out, lse, plan = run_gpu(w, gpu, chunk)
    log(f"  schedule {plan.info()}")
    ro, rl = ref.run_workload(w)
    compare(out, lse, ro, rl, w.dtype, label=w.name)


# ------------------------------------------------------------------ seeded workloads

def test_tiny_cross_f32(gpu):
    _full(synth.tiny_cross(0), gpu)


def test_whisper_decode(gpu):
    _full(synth.whisper_decode(0), gpu)


def test_ragged_prefill(gpu):
    _full(synth.ragged_prefill(0), gpu)


def _full_by_request(w, gpu):
    """The whole workload on the GPU against the oracle over every request and head, the
    oracle computed request by request on a pool of host threads."""
    log(f"[parity] {w.name} (every request and head)")
    out, lse, plan = run_gpu(w, gpu)
    log(f"  schedule {plan.info()}")
    plan.close()
    t0 = time.perf_counter()
    ro, rl = oracle_by_request(w)
    log(f"  oracle over {w.batch_size} requests in {time.perf_counter() - t0:.1f} s")
    compare(out, lse, ro, rl, w.dtype, label=w.name)
    return out, lse


def test_block_causal_full(gpu):
    """Block-causal spans of 256-4096 tokens at full size: every span, every head."""
    _full_by_request(synth.block_causal(0), gpu)


def test_tensor_parallel_rank_shapes(gpu):
    """One rank's heads of the decode workloads under tensor parallelism over heads."""
    _full(synth.whisper_decode_tp4(0), gpu)
    _full_by_request(synth.gqa_decode_tp8(0), gpu)


def test_ragged_cross_spans_full(gpu):
    """Cacheless span-to-span cross-attention at full size: 32 requests, query spans of
    1-448 tokens over key spans of 256-4096, 16 heads, head_dim 128."""
    _full_by_request(synth.ragged_cross_spans(0), gpu)


def test_causal_prefill_paged_full(gpu):
    """Multi-token causal prefill over a paged cache at full size: 16 requests of 256-4096
    new tokens, 32 query / 8 KV heads, head_dim 128, page_size 16."""
    _full_by_request(synth.causal_prefill_paged(0), gpu)


def test_gqa_decode_full(gpu):
    """The GQA decode at full size (9.5 GB of K and V, split contexts merged): every
    request, every head."""
    _full_by_request(synth.gqa_decode(0), gpu)


# ------------------------------------------------------------------ small cases

SMALL = [
    # (name, qo_lens, kv_lens, hq, hkv, d, page_size, mask, block, dtype)
    ("decode_mha_d64", [1] * 9, [1, 2, 15, 16, 17, 100, 513, 1000, 64], 4, 4, 64, 16, 0, 0, "bf16"),
    ("decode_gqa4_causal_d128", [1] * 6, [1, 7, 64, 65, 300, 2049], 8, 2, 128, 16, 1, 0, "bf16"),
    ("gqa8_d128_tiles", [1] * 3, [33, 500, 129], 16, 2, 128, 8, 0, 0, "bf16"),  # 8 rows: tile kernel
    ("decode_rows2_causal", [2, 1, 2], [5, 40, 300], 2, 2, 64, 4, 1, 0, "bf16"),
    ("rows8_mixed", [2, 4, 1], [9, 70, 33], 4, 2, 64, 3, 1, 0, "bf16"),  # 4 and 8 rows: decode and tiles
    ("decode_block", [3, 1], [50, 130], 2, 1, 64, 16, 2, 16, "bf16"),
    ("mma_none_d64", [9, 33, 128, 129, 300], [1500, 77, 300, 129, 1000], 2, 2, 64, 16, 0, 0, "bf16"),
    ("mma_causal_d128", [40, 200, 129], [40, 260, 500], 2, 2, 128, 16, 1, 0, "bf16"),
    ("mma_gqa_causal_d64", [20, 70], [50, 300], 8, 2, 64, 16, 1, 0, "bf16"),
    ("mma_block_d128", [300, 65, 1], [300, 65, 1], 2, 2, 128, 1, 2, 64, "bf16"),
    ("mma_block_odd", [100, 250], [130, 250], 2, 1, 64, 5, 2, 7, "bf16"),
    ("mma_page3", [50, 10], [77, 30], 2, 2, 64, 3, 0, 0, "bf16"),
    # page sizes around the tile kernel's whole-page addressing (a 1 KB load spans 8 rows at
    # head_dim 64 and 4 at 128; tiles are 64 keys)
    ("mma_page8_d64", [70, 3], [200, 90], 2, 2, 64, 8, 0, 0, "bf16"),
    ("mma_page4_d128_causal", [40, 130], [100, 131], 4, 2, 128, 4, 1, 0, "bf16"),
    ("mma_page64_d64", [33, 140], [500, 140], 2, 2, 64, 64, 1, 0, "bf16"),
    ("mma_page128_d128", [20, 9], [300, 129], 2, 2, 128, 128, 0, 0, "bf16"),
    # tile units of 1 to 5 key tiles at head_dim 64, where the tile loads run two tiles ahead
    ("mma_d64_tiles_1to5", [20] * 6, [1, 64, 65, 128, 192, 257], 2, 2, 64, 16, 0, 0, "bf16"),
    ("mma_d64_causal_short", [20, 60, 130], [20, 130, 200], 2, 1, 64, 16, 1, 0, "bf16"),
    ("f32_all_masks_none", [1, 5, 2], [16, 40, 7], 2, 2, 16, 4, 0, 0, "f32"),
    ("f32_causal_gqa", [3, 1, 6], [7, 13, 6], 4, 1, 32, 3, 1, 0, "f32"),
    ("f32_block_d64", [10, 17], [10, 17], 2, 2, 64, 1, 2, 4, "f32"),
    ("f32_long_d128", [2, 1], [3000, 1100], 2, 2, 128, 16, 0, 0, "f32"),
    ("empty_requests", [0, 3, 0, 1], [5, 0, 9, 0], 2, 2, 64, 4, 0, 0, "bf16"),
    ("empty_requests_mma", [0, 20, 0], [5, 0, 9], 2, 2, 64, 4, 0, 0, "bf16"),
]


def _small(case, seed=0, tail="normal"):
    name, qo, kv, hq, hkv, d, ps, mask, blk, dt = case
    return synth.paged_case(qo, kv, hq, hkv, d, ps, dtype=dt, mask_mode=mask, block_size=blk,
                            seed=seed, name=name, tail=tail, extra_pages=3)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("chunk", [0, 64, 17])
def test_small(case, chunk, gpu):
    w = _small(case)
    _full(w, gpu, chunk)


@pytest.mark.parametrize("case", [c for c in SMALL if c[0] in
                                  ("decode_mha_d64", "mma_none_d64", "mma_block_odd", "f32_causal_gqa",
                                   "decode_gqa4_causal_d128")], ids=lambda c: c[0])
def test_nan_poisoned_tails(case, gpu):
    """Unused page slots and unreferenced pages hold NaN: none may reach a result."""
    w = _small(case, seed=3, tail="nan")
    _full(w, gpu, 0)
    _full(w, gpu, 33)


def test_single_key_chunks(gpu):
    """Every key its own chunk: the merge sees up to hundreds of partials per row."""
    w = synth.paged_case([1, 3, 40], [200, 3, 120], 4, 2, 64, 16, mask_mode=1, seed=4, name="chunk1")
    _full(w, gpu, 1)


# ------------------------------------------------------------------ cacheless spans

RAGGED = {
    # cross-attention between a request's query span and its key span (sizes differ; empty
    # spans on either side)
    "ragged_cross_d64": lambda: synth.ragged_cross_case(
        [3, 70, 1, 130, 0, 9], [1500, 64, 7, 300, 20, 0], 4, 64, seed=40, name="ragged_cross_d64"),
    "ragged_cross_gqa_d128": lambda: synth.ragged_cross_case(
        [5, 200, 33], [900, 129, 64], 8, 128, num_kv_heads=2, seed=41, name="ragged_cross_gqa_d128"),
    "ragged_cross_f32": lambda: synth.ragged_cross_case(
        [2, 5], [40, 3], 2, 32, dtype="f32", seed=44, name="ragged_cross_f32"),
    # self-attention within each span without a mask and causally
    "ragged_self_none_d64": lambda: synth.ragged_case(
        [200, 17, 65, 1], 4, 64, mask_mode=0, seed=42, name="ragged_self_none_d64"),
    "ragged_self_causal_d128": lambda: synth.ragged_case(
        [300, 1, 129], 4, 128, num_kv_heads=2, mask_mode=1, seed=43, name="ragged_self_causal_d128"),
}


@pytest.mark.parametrize("case", sorted(RAGGED))
@pytest.mark.parametrize("chunk", [0, 64, 17])
def test_cacheless_spans(case, chunk, gpu):
    """Cacheless spans as the identity page table: cross-attention between two spans of
    each request, and self-attention within spans with no mask or a causal one."""
    _full(RAGGED[case](), gpu, chunk)


def test_empty_batch(gpu):
    import ragged_attention_serving_amd as xa
    import torch
    plan = xa.Plan().plan([0], [0], None, None, 2, 2, 64, 16, 1)
    q = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=gpu)
    k = torch.zeros((1, 16, 2, 64), dtype=torch.bfloat16, device=gpu)
    out, lse = plan.run(q, k, k)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 64)


def test_without_lse(gpu):
    w = _small(SMALL[6])
    out, lse, _ = run_gpu(w, gpu, want_lse=False)
    assert lse is None
    ro, _ = ref.run_workload(w)
    assert np.max(np.abs(out - ro)) <= 2e-2


# ------------------------------------------------------------------ invariants and contracts

def test_page_permutation_is_bitwise_invariant(gpu):
    w = synth.paged_case([1, 1, 30, 200], [900, 40, 300, 700], 4, 2, 128, 16, mask_mode=1, seed=5)
    out1, lse1, _ = run_gpu(w, gpu)
    perm = np.random.default_rng(9).permutation(w.num_pages)
    kp = np.empty_like(w.k_pages)
    vp = np.empty_like(w.v_pages)
    kp[perm] = w.k_pages
    vp[perm] = w.v_pages
    w.k_pages, w.v_pages = kp, vp
    w.kv_page_indices = perm[w.kv_page_indices].astype(np.int32)
    out2, lse2, _ = run_gpu(w, gpu)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_cache_is_never_written(gpu):
    import torch
    w = synth.paged_case([1, 50, 3], [300, 400, 30], 4, 4, 64, 16, seed=6)
    q, k, v = (to_device(w.q, "bf16", gpu), to_device(w.k_pages, "bf16", gpu), to_device(w.v_pages, "bf16", gpu))
    k0, v0 = k.clone(), v.clone()
    for chunk in (0, 64):
        run_gpu(w, gpu, chunk, tensors=(q, k, v))
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16))


def test_uniform_scores_closed_form(gpu):
    """Q = 0: O is the mean of the visible values and lse = ln(visible count)."""
    for mask, blk, qo, kv in ((0, 0, [1, 3, 100], [16, 40, 1500]), (1, 0, [1, 5, 150], [700, 9, 150]),
                              (2, 64, [300, 64], [300, 64])):
        w = synth.paged_case(qo, kv, 2, 2, 64, 16 if mask != 2 else 1, mask_mode=mask, block_size=blk, seed=7)
        w.q = np.zeros_like(w.q)
        out, lse, _ = run_gpu(w, gpu)
        ro, rl = ref.run_workload(w)
        compare(out, lse, ro, rl, "bf16", label=f"Q=0 mask {mask}")
        for r in range(len(qo)):
            for i in range(qo[r]):
                pos = kv[r] - qo[r] + i
                n = kv[r] if mask == 0 else (pos + 1 if mask == 1 else min((pos // blk + 1) * blk, kv[r]))
                assert abs(lse[w.qo_indptr[r] + i, 0] - np.log(n)) < 1e-3


def test_one_plan_many_layers(gpu):
    """One plan serves several runs with different q/k/v (one per layer)."""
    base = synth.paged_case([1, 40, 2], [500, 300, 60], 4, 2, 64, 16, mask_mode=1, seed=8)
    plan = None
    for layer in range(3):
        w = synth.paged_case([1, 40, 2], [500, 300, 60], 4, 2, 64, 16, mask_mode=1, seed=100 + layer)
        w.kv_page_indices = base.kv_page_indices
        out, lse, plan = run_gpu(w, gpu, plan=plan) if plan is None else _run_existing(w, gpu, plan)
        ro, rl = ref.run_workload(w)
        compare(out, lse, ro, rl, "bf16", label=f"layer {layer}")


def _run_existing(w, gpu, plan):
    import torch
    from tests.gpu_util import from_device
    q, k, v = (to_device(w.q, w.dtype, gpu), to_device(w.k_pages, w.dtype, gpu), to_device(w.v_pages, w.dtype, gpu))
    out, lse = plan.run(q, k, v)
    torch.cuda.synchronize()
    return from_device(out), lse.cpu().numpy().astype(np.float64), plan


def test_double_buffered_plans_while_the_gpu_is_busy(gpu):
    """Plan A, run A, plan B, run B while the stream is still busy with earlier work: the
    second plan must not overwrite the staging that run A reads; a third plan waits for
    the slot's fence. The stream is held by ordinary queued matrix products."""
    import torch
    wa = synth.paged_case([1, 30], [700, 300], 4, 2, 64, 16, mask_mode=1, seed=10)
    wb = synth.paged_case([5, 1, 2], [20, 900, 64], 4, 2, 64, 16, mask_mode=1, seed=11)
    ta = [to_device(x, "bf16", gpu) for x in (wa.q, wa.k_pages, wa.v_pages)]
    tb = [to_device(x, "bf16", gpu) for x in (wb.q, wb.k_pages, wb.v_pages)]
    x = torch.randn(4096, 4096, device=gpu)
    torch.cuda.synchronize()
    import ragged_attention_serving_amd as xa
    plan = xa.Plan()
    for _ in range(150):  # hundreds of milliseconds of queued work
        x = torch.tanh(x @ x) * 0.01
    plan.plan(wa.qo_indptr, wa.kv_indptr, wa.kv_page_indices, wa.kv_last_page_len, 4, 2, 64, 16,
              wa.num_pages, 1)
    oa, la = plan.run(*ta)
    plan.plan(wb.qo_indptr, wb.kv_indptr, wb.kv_page_indices, wb.kv_last_page_len, 4, 2, 64, 16,
              wb.num_pages, 1)
    ob, lb = plan.run(*tb)
    busy = not plan.ready()
    # a third plan reuses slot A: it waits on the fence of run A
    plan.plan(wa.qo_indptr, wa.kv_indptr, wa.kv_page_indices, wa.kv_last_page_len, 4, 2, 64, 16,
              wa.num_pages, 1)
    oc, lc = plan.run(*ta)
    torch.cuda.synchronize()
    log(f"  next slot busy while queued: {busy}")
    from tests.gpu_util import from_device
    ra, rla = ref.run_workload(wa)
    rb, rlb = ref.run_workload(wb)
    compare(from_device(oa), la.cpu().numpy().astype(np.float64), ra, rla, "bf16", label="plan A")
    compare(from_device(ob), lb.cpu().numpy().astype(np.float64), rb, rlb, "bf16", label="plan B")
    compare(from_device(oc), lc.cpu().numpy().astype(np.float64), ra, rla, "bf16", label="plan A again")
    assert busy


@pytest.mark.parametrize("rows", [128, 256])
def test_tile_kernel_variants(rows, gpu, monkeypatch):
    """Both MFMA tile heights, on tiles with tails, masks and splits."""
    monkeypatch.setenv("XATTN_TILE_ROWS", str(rows))
    for case in ("mma_none_d64", "mma_causal_d128", "mma_block_odd", "mma_gqa_causal_d64"):
        w = _small([c for c in SMALL if c[0] == case][0])
        _full(w, gpu, 0)
        _full(w, gpu, 130)
    w = synth.ragged_case([700, 65, 300], 2, 128, block_size=64, seed=12, name="block_causal_small")
    _full(w, gpu, 0)


def test_runs_and_plans_on_several_streams(gpu):
    """Two layers of one split plan run at once on two streams, each with its own q, k and
    v: the runs share the slot's workspace of partial results, so they must not mix their
    partials (a run on another stream waits for the latest one). Then plans move to
    another stream: every run still sees its own schedule and leaves the other slot's runs
    intact."""
    import torch
    import ragged_attention_serving_amd as xa
    from tests.gpu_util import forced_chunk, from_device
    qo, kv = [1] * 96 + [30, 7], [2000] * 96 + [700, 300]
    base = synth.paged_case(qo, kv, 4, 2, 64, 16, mask_mode=1, seed=20)
    layers = []
    for i in range(3):
        w = synth.paged_case(qo, kv, 4, 2, 64, 16, mask_mode=1, seed=200 + i)
        w.kv_page_indices = base.kv_page_indices
        layers.append(w)
    tl = [[to_device(x, "bf16", gpu) for x in (w.q, w.k_pages, w.v_pages)] for w in layers]
    wb = synth.paged_case([5, 1, 2], [20, 900, 64], 4, 2, 64, 16, mask_mode=1, seed=21)
    tb = [to_device(x, "bf16", gpu) for x in (wb.q, wb.k_pages, wb.v_pages)]
    main = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    plan = xa.Plan()
    with forced_chunk(64):
        plan.plan(base.qo_indptr, base.kv_indptr, base.kv_page_indices, base.kv_last_page_len, 4, 2, 64, 16,
                  base.num_pages, 1, stream=main)
    info = plan.info()
    log(f"  split schedule {info}")
    assert info["num_merge_rows"] > 0
    outs = []
    for i, st in enumerate((s1, s2, main)):
        with torch.cuda.stream(st):
            outs.append(plan.run(*tl[i], stream=st))
    # the next plans move to stream s1; the first reuses nothing, the second reuses slot A
    with torch.cuda.stream(s1):
        plan.plan(wb.qo_indptr, wb.kv_indptr, wb.kv_page_indices, wb.kv_last_page_len, 4, 2, 64, 16,
                  wb.num_pages, 1, stream=s1)
        ob, lb = plan.run(*tb, stream=s1)
        plan.plan(base.qo_indptr, base.kv_indptr, base.kv_page_indices, base.kv_last_page_len, 4, 2, 64, 16,
                  base.num_pages, 1, stream=s1)
        oc, lc = plan.run(*tl[0], stream=s1)
    torch.cuda.synchronize()
    refs = [ref.run_workload(w) for w in layers]
    rb, rlb = ref.run_workload(wb)
    for i, (o, l) in enumerate(outs):
        compare(from_device(o), l.cpu().numpy().astype(np.float64), *refs[i], "bf16",
                label=f"layer {i} on stream {('s1', 's2', 'main')[i]}")
    compare(from_device(ob), lb.cpu().numpy().astype(np.float64), rb, rlb, "bf16", label="B on s1")
    compare(from_device(oc), lc.cpu().numpy().astype(np.float64), *refs[0], "bf16", label="layer 0 again on s1")
    plan.close()
