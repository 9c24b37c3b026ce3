"""Stored oracle values for the tiny workload still match (guards the generator and oracle)."""
import os

import numpy as np

from oracle import ref
from ragged_attention_serving_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden():
    rows = np.loadtxt(os.path.join(HERE, "golden", "tiny_cross_f32.txt"))
    return rows


def test_tiny_cross_golden():
    g = load_golden()
    w = synth.tiny_cross(0)
    out, lse = ref.run_workload(w)
    for row in g:
        i, h = int(row[0]), int(row[1])
        assert abs(lse[i, h] - row[2]) < 1e-13
        assert np.allclose(out[i, h], row[3:], atol=1e-13, rtol=0)


def test_generator_self_check():
    """Lengths of the seeded workloads: numpy 2.2 draws from default_rng(0) in the fixed order."""
    rng = np.random.default_rng(0)
    lens = synth.block_causal_span_lengths(rng)
    assert int(lens.sum()) == 141675 and list(lens[:4]) == [3523, 2702, 2219, 1292]
    rng = np.random.default_rng(0)
    kv = synth.gqa_decode_context_lengths(rng)
    assert int(kv.sum()) == 2321997 and list(kv[:4]) == [7240, 1572, 607, 548]
    assert kv.min() >= 512 and kv.max() <= 32768
    qo = synth.ragged_prefill_query_lengths(np.random.default_rng(0))
    assert int(qo.sum()) == 7569 and list(qo[:4]) == [382, 286, 229, 121]
    w6 = synth.ragged_cross_spans(0)
    assert int(w6.qo_indptr[-1]) == 7569 and int(w6.kv_indptr[-1]) == 68724
    assert list(w6.qo_lens()[:4]) == [382, 286, 229, 121] and w6.k_pages.shape == (68724, 1, 16, 128)
    w7_lens = np.random.default_rng(0).integers(256, 4096, 16, endpoint=True)
    assert int(w7_lens.sum()) == 35086
    w2 = synth.whisper_decode(0)
    assert list(set(w2.kv_lens())) == [1500] and int(w2.kv_indptr[-1]) == 6016
    assert set(w2.kv_last_page_len) == {12} and w2.num_pages == 6016
    w3 = synth.ragged_prefill(0)
    assert int(w3.qo_indptr[-1]) == 7569 and list(w3.qo_lens()[:4]) == [382, 286, 229, 121]
    assert w3.k_pages.shape == (3008, 16, 20, 64)
    w1 = synth.tiny_cross(0)
    assert list(w1.kv_lens()) == [16, 40] and w1.k_pages.shape == (14, 4, 2, 16)
