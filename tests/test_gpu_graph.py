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
