"""HIP-graph capture of a run (the reason the plan is double-buffered).

A run launched on its plan's own stream, with timing off, issues only kernel launches,
so it can be captured into a HIP graph and replayed. A replay repeats the captured
schedule: it stays valid while the slot it read keeps that schedule, i.e. through the
next plan (which fills the other slot), and not after the one after that.
"""
import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.gpu_util import compare, forced_chunk, from_device, log, to_device

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def test_captured_run_replays_its_plan(gpu):
    import torch
    import ragged_attention_serving_amd as xa
    # decode rows, MFMA tiles and (with the forced chunk) split rows and the merge
    w = synth.paged_case([1, 40, 1, 130], [2000, 300, 1800, 200], 8, 2, 128, 16, mask_mode=1, seed=70)
    w2 = synth.paged_case([2, 1], [64, 700], 8, 2, 128, 16, mask_mode=1, seed=71)
    s = torch.cuda.Stream()
    rng = np.random.default_rng(5)
    with torch.cuda.stream(s):
        q = to_device(w.q, "bf16", gpu)
        k, v = to_device(w.k_pages, "bf16", gpu), to_device(w.v_pages, "bf16", gpu)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=gpu)
        plan = xa.Plan()
        with forced_chunk(64):
            plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, 8, 2, 128, 16,
                      w.num_pages, 1, stream=s)
        info = plan.info()
        log(f"  schedule {info}")
        assert info["num_merge_rows"] > 0 and info["num_units"][1] > 0 and info["num_units"][2] > 0
        plan.run(q, k, v, out, lse, stream=s)  # eager warm-up
    s.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(q, k, v, out, lse, stream=s)
    s.synchronize()

    def check(label):
        # an eager run of the same inputs into fresh buffers on the same stream
        with torch.cuda.stream(s):
            eo, el = plan.run(q, k, v, stream=s)
        s.synchronize()
        assert np.array_equal(_bits(out), _bits(eo)), f"{label}: out differs from the eager run"
        assert np.array_equal(lse.cpu().numpy(), el.cpu().numpy()), f"{label}: lse differs"

    for rep in range(4):
        # eager work between replays: new query values in place, outputs cleared
        newq = synth.round_to_bf16_bits(rng.standard_normal(w.q.shape).astype(np.float32))
        with torch.cuda.stream(s):
            q.copy_(to_device(newq, "bf16", gpu))
            out.zero_()
            lse.zero_()
        s.synchronize()
        g.replay()
        s.synchronize()
        check(f"replay {rep}")
        w.q = newq
        if rep == 0:
            ro, rl = ref.run_workload(w)
            compare(from_device(out), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", label="replay 0")

    # the next plan fills the other slot: the captured run still replays its own schedule
    with torch.cuda.stream(s):
        plan.plan(w2.qo_indptr, w2.kv_indptr, w2.kv_page_indices, w2.kv_last_page_len, 8, 2, 128, 16,
                  w2.num_pages, 1, stream=s)
        o2, l2 = plan.run(to_device(w2.q, "bf16", gpu), to_device(w2.k_pages, "bf16", gpu),
                          to_device(w2.v_pages, "bf16", gpu), stream=s)
        out.zero_()
    s.synchronize()
    g.replay()
    s.synchronize()
    ro, rl = ref.run_workload(w)
    compare(from_device(out), lse.cpu().numpy().astype(np.float64), ro, rl, "bf16", label="replay after next plan")
    r2, rl2 = ref.run_workload(w2)
    compare(from_device(o2), l2.cpu().numpy().astype(np.float64), r2, rl2, "bf16", label="next plan")
    del g
    plan.close()


def _pool_batch(rng, pool_pages, qo_lens, kv_lens, page_size):
    """A batch's packing over a shared page pool: pages drawn without replacement."""
    npages = [(k + page_size - 1) // page_size for k in kv_lens]
    kv_indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    pages = rng.choice(pool_pages, size=int(kv_indptr[-1]), replace=False).astype(np.int32)
    last = np.array([k - (n - 1) * page_size if n else page_size for k, n in zip(kv_lens, npages)], np.int32)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    return qo_indptr, kv_indptr, pages, last


def test_graph_stable_replays_across_plans(gpu):
    """With XATTN_PLAN_GRAPH_STABLE, one captured graph per slot replays later schedules of
    other shapes: every replay equals an eager run bit for bit and matches the oracle."""
    import torch
    import ragged_attention_serving_amd as xa
    hq, hkv, d, ps = 8, 2, 128, 16
    rng = np.random.default_rng(90)
    pool_pages = 3000
    k_np = synth.normal_tensor((pool_pages, ps, hkv, d), 90, synth.TENSOR_K, "bf16")
    v_np = synth.normal_tensor((pool_pages, ps, hkv, d), 90, synth.TENSOR_V, "bf16")
    # the first two plans (one per slot) set the capacities: decode units (1 token, 4 rows; 2
    # tokens are 8 rows and go to tiles), split long contexts (merges) and multi-token tiles;
    # every later plan in the same slot needs no more units of any family, merge rows,
    # workspace rows, requests or pages
    batches = [([1, 2, 1, 40, 130], [20000, 3000, 700, 300, 200]),
               ([1, 1, 1, 60, 100], [20000, 9000, 900, 500, 260]),
               ([1, 1, 37], [12000, 100, 90]),
               ([1, 2, 1, 1], [18000, 40, 5000, 16]),
               ([90, 1], [150, 16000]),
               ([1, 1, 1, 3], [1, 17, 10000, 64])]
    max_q = max(sum(q) for q, _ in batches)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        k = to_device(k_np, "bf16", gpu)
        v = to_device(v_np, "bf16", gpu)
        qbuf = torch.zeros((max_q, hq, d), dtype=torch.bfloat16, device=gpu)
        obuf = torch.zeros_like(qbuf)
        lbuf = torch.zeros((max_q, hq), dtype=torch.float32, device=gpu)
    plan = xa.Plan(graph_stable=True)
    graphs, gens = {}, {}
    for step, (qo_lens, kv_lens) in enumerate(batches):
        qo_indptr, kv_indptr, pages, last = _pool_batch(rng, pool_pages, qo_lens, kv_lens, ps)
        nq = int(qo_indptr[-1])
        q_np = synth.round_to_bf16_bits(rng.standard_normal((nq, hq, d)).astype(np.float32))
        with torch.cuda.stream(s):
            plan.plan(qo_indptr, kv_indptr, pages, last, hq, hkv, d, ps, pool_pages, 1, stream=s)
            qbuf[:nq].copy_(to_device(q_np, "bf16", gpu))
            obuf.zero_()
            lbuf.zero_()
        s.synchronize()
        info = plan.info()
        slot, gen = info["slot"], info["layout_generation"]
        log(f"  step {step}: slot {slot} generation {gen} units {info['num_units']} merges {info['num_merge_rows']}")
        qv, ov, lv = qbuf[:nq], obuf[:nq], lbuf[:nq]
        if slot not in graphs:
            with torch.cuda.stream(s):
                plan.run(qv, k, v, ov, lv, stream=s)  # eager warm-up before the capture
            s.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                plan.run(qv, k, v, ov, lv, stream=s)
            s.synchronize()
            graphs[slot], gens[slot] = g, gen
            with torch.cuda.stream(s):
                obuf.zero_()
                lbuf.zero_()
            s.synchronize()
        else:
            assert gen == gens[slot], "a smaller schedule must keep the slot's layout"
        graphs[slot].replay()
        s.synchronize()
        with torch.cuda.stream(s):
            eo, el = plan.run(qv, k, v, stream=s)
        s.synchronize()
        assert np.array_equal(_bits(ov), _bits(eo)), f"step {step}: replay differs from the eager run"
        assert np.array_equal(lv.cpu().numpy(), el.cpu().numpy()), f"step {step}: lse differs"
        ro, rl = ref.paged_attention(q_np, k_np, v_np, qo_indptr, kv_indptr, pages, last, hq, hkv, ps,
                                     dtype="bf16", mask_mode=1)
        compare(from_device(ov), lv.cpu().numpy().astype(np.float64), ro, rl, "bf16", label=f"step {step} replay")
    del graphs
    plan.close()
