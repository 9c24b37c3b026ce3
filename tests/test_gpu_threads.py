"""Distinct handles on distinct host threads are independent: each thread re-plans and
runs its own workload on its own stream, with no lock around the library, and every run
matches the oracle."""
import threading

import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.gpu_util import compare, from_device, log, to_device

pytestmark = pytest.mark.gpu

ROUNDS = 12


def test_handles_on_several_threads(gpu):
    import torch
    import ragged_attention_serving_amd as xa
    works = [
        synth.paged_case([1] * 5, [900, 20, 1500, 64, 333], 4, 2, 64, 16, mask_mode=1, seed=40, name="gqa_decode"),
        synth.paged_case([40, 3, 129], [300, 64, 1500], 2, 2, 128, 16, seed=41, name="prefill"),
        synth.ragged_case([130, 64, 257], 2, 64, block_size=64, seed=42, name="block_causal"),
        synth.paged_case([2, 1], [5000, 17], 8, 1, 128, 32, mask_mode=1, seed=43, name="split_decode"),
    ]
    refs = [ref.run_workload(w) for w in works]
    tensors = [[to_device(x, w.dtype, gpu) for x in (w.q, w.k_pages, w.v_pages)] for w in works]
    torch.cuda.synchronize()
    results = [None] * len(works)
    errors = []

    def worker(i):
        try:
            w = works[i]
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.default_stream())
            plan = xa.Plan()
            outs = []
            with torch.cuda.stream(st):
                for _ in range(ROUNDS):
                    # a new plan each round: the two slots alternate while earlier runs are in flight
                    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
                              w.num_kv_heads, w.head_dim, w.page_size, max(w.num_pages, 1), w.mask_mode,
                              w.block_size, w.sm_scale, w.dtype, stream=st)
                    outs.append(plan.run(*tensors[i], stream=st))
            st.synchronize()
            results[i] = [(from_device(o), l.cpu().numpy().astype(np.float64)) for o, l in outs]
            plan.close()
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i} ({works[i].name}): {e!r}")

    log(f"[threads] {len(works)} threads x {ROUNDS} plan+run rounds")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(works))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, res in enumerate(results):
        for k, (o, l) in enumerate(res):
            compare(o, l, *refs[i], works[i].dtype, label=f"{works[i].name} round {k}")
