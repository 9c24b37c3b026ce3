"""The request-by-request oracle used for full-size GPU comparisons equals the oracle's own
entry point exactly, on every route (paged, identity table, cacheless self and cross
spans, empty requests) and on request subsets."""
import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.oracle_threads import oracle_by_request

CASES = {
    "paged_causal_gqa": lambda: synth.paged_case([3, 0, 1, 7], [9, 5, 40, 7], 4, 2, 8, 3, dtype="bf16",
                                                 mask_mode=1, seed=70, extra_pages=2),
    "paged_identity_block": lambda: synth.paged_case([5, 2], [11, 6], 2, 2, 8, 2, dtype="f32",
                                                     mask_mode=2, block_size=3, seed=71, shuffle=False),
    "paged_no_last_len": lambda: _full_last_pages(),
    "cacheless_block": lambda: synth.ragged_case([9, 0, 17, 4], 4, 8, num_kv_heads=2, block_size=4, seed=72),
    "cacheless_cross": lambda: synth.ragged_cross_case([3, 0, 6, 2], [8, 5, 0, 4], 2, 8, seed=73),
}


def _full_last_pages():
    w = synth.paged_case([2, 3], [8, 12], 2, 1, 8, 4, dtype="f32", seed=74)
    w.kv_last_page_len = None  # every last page is full
    return w


@pytest.mark.parametrize("name", sorted(CASES))
def test_matches_entry_point(name):
    w = CASES[name]()
    ro, rl = ref.run_workload(w)
    for threads in (1, 3):
        o, l = oracle_by_request(w, threads=threads)
        assert np.array_equal(o, ro, equal_nan=True) and np.array_equal(l, rl, equal_nan=True)
    reqs = [w.batch_size - 1, 0]
    so, sl = ref.run_workload(w, requests=reqs)
    o, l = oracle_by_request(w, threads=2, requests=reqs)
    assert np.array_equal(o, so, equal_nan=True) and np.array_equal(l, sl, equal_nan=True)
