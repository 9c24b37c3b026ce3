"""GPU parity of the context write (xattn_write_kv) against the oracle's write.

The write is a byte copy, so the bar is bit-exact: both pools after the write must
equal the oracle's pools everywhere, including the slots the write must not touch
(tails of last pages and pages of no request, filled beforehand with other values).
Attention over the written pools is then checked against the oracle as usual.
"""
import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.gpu_util import compare, log, plan_for, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "paged_bf16_d64_ps16": lambda: synth.paged_case([1] * 5, [1500, 17, 16, 1, 300], 4, 4, 64, 16,
                                                     seed=60, extra_pages=5, name="paged_bf16_d64_ps16"),
    "paged_gqa_bf16_d128_ps3": lambda: synth.paged_case([2, 1, 40], [7, 100, 64], 8, 2, 128, 3,
                                                         seed=61, extra_pages=4, mask_mode=1,
                                                         name="paged_gqa_bf16_d128_ps3"),
    "paged_f32_d32_ps4_empty": lambda: synth.paged_case([1, 1, 1], [9, 0, 6], 2, 2, 32, 4, dtype="f32",
                                                         seed=62, extra_pages=3, name="paged_f32_d32_ps4_empty"),
    "identity_bf16_d64": lambda: synth.ragged_cross_case([3, 5, 1], [200, 1, 64], 2, 64, seed=63,
                                                          name="identity_bf16_d64"),
    "whisper_decode_cross": lambda: synth.whisper_decode(0),
}


def _bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def _as_bits(a, dtype):
    a = np.ascontiguousarray(a)
    return a.view(np.int16) if dtype == "bf16" else a.astype(np.float32).view(np.int32)


@pytest.mark.parametrize("case", sorted(CASES))
def test_context_write_bit_exact(case, gpu):
    import torch
    w = CASES[case]()
    log(f"[write_kv] {w.name}")
    ks, vs = synth.context_source(w, seed=9)
    # the pools hold other values beforehand: the workload's own tensors
    kp_ref, vp_ref = ref.write_context(ks, vs, w.k_pages, w.v_pages, w.kv_indptr, w.kv_page_indices,
                                       w.kv_last_page_len, w.page_size)
    kpool, vpool = to_device(w.k_pages, w.dtype, gpu), to_device(w.v_pages, w.dtype, gpu)
    ksrc, vsrc = to_device(ks, w.dtype, gpu), to_device(vs, w.dtype, gpu)
    plan = plan_for(w)
    plan.write_kv(ksrc, vsrc, kpool, vpool)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kpool), _as_bits(kp_ref, w.dtype)), "k_pages differ"
    assert np.array_equal(_bits(vpool), _as_bits(vp_ref, w.dtype)), "v_pages differ"
    # then read it back through attention
    q = to_device(w.q, w.dtype, gpu)
    out, lse = plan.run(q, kpool, vpool)
    torch.cuda.synchronize()
    w.k_pages, w.v_pages = kp_ref, vp_ref
    if w.name == "whisper_decode_cross":
        ro, rl = ref.run_workload(w, requests=range(0, w.batch_size, 9))
        rows = np.concatenate([np.arange(w.qo_indptr[r], w.qo_indptr[r + 1]) for r in range(0, w.batch_size, 9)])
    else:
        ro, rl = ref.run_workload(w)
        rows = None
    from tests.gpu_util import from_device
    compare(from_device(out), lse.cpu().numpy().astype(np.float64), ro, rl, w.dtype, rows=rows,
            label=f"{w.name} after write")
    plan.close()


def test_context_write_on_another_stream(gpu):
    """A write on a stream other than the plan's waits for the schedule's copy."""
    import torch
    w = CASES["paged_bf16_d64_ps16"]()
    ks, vs = synth.context_source(w, seed=10)
    kp_ref, vp_ref = ref.write_context(ks, vs, w.k_pages, w.v_pages, w.kv_indptr, w.kv_page_indices,
                                       w.kv_last_page_len, w.page_size)
    kpool, vpool = to_device(w.k_pages, w.dtype, gpu), to_device(w.v_pages, w.dtype, gpu)
    ksrc, vsrc = to_device(ks, w.dtype, gpu), to_device(vs, w.dtype, gpu)
    side = torch.cuda.Stream()
    plan = plan_for(w)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.write_kv(ksrc, vsrc, kpool, vpool, stream=side)
    side.synchronize()
    assert np.array_equal(_bits(kpool), _as_bits(kp_ref, w.dtype))
    assert np.array_equal(_bits(vpool), _as_bits(vp_ref, w.dtype))
    plan.close()
