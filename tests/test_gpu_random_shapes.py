"""GPU parity over seeded random shapes: head counts and groups, head dims, page sizes,
masks, query and context lengths, forced chunk lengths, and both tile heights. Each case
is small enough for the oracle; together they cross the kernels' addressing paths (whole
pages or per-row tables, buffer or global loads, the identity table of cacheless spans)
with ragged tails, in bf16 and in fp32."""
import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.gpu_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 64
N_SPANS = 16
N_F32 = 16


def _case(i):
    rng = np.random.default_rng(1000 + i)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    ps = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64, 128]))
    mask = int(rng.integers(0, 3))
    b = int(rng.integers(1, 6))
    kv = rng.integers(1, 700, b)
    decode_like = rng.random() < 0.4  # one or two query tokens: the decode kernel's rows
    hi = 3 if decode_like else 160
    if mask == 0:
        qo = rng.integers(0 if not decode_like else 1, hi, b)
    else:
        qo = np.minimum(rng.integers(1, hi, b), kv)
    block = int(rng.choice([1, 7, 16, 64])) if mask == 2 else 0
    chunk = int(rng.choice([0, 0, 64, 100, 257]))
    rows = int(rng.choice([128, 256]))
    w = synth.paged_case(qo, kv, hkv * g, hkv, d, ps, mask_mode=mask, block_size=block, seed=2000 + i,
                         name=f"random_{i}", extra_pages=int(rng.integers(0, 5)))
    return w, chunk, rows


def _span_case(i):
    """Cacheless spans (the identity table): self-attention under any mask, or
    cross-attention between a request's query span and a key span of its own."""
    rng = np.random.default_rng(3000 + i)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4]))
    b = int(rng.integers(1, 6))
    chunk = int(rng.choice([0, 0, 64, 100]))
    rows = int(rng.choice([128, 256]))
    if rng.random() < 0.5:
        mask = int(rng.integers(0, 3))
        block = int(rng.choice([1, 7, 16, 64])) if mask == 2 else 0
        w = synth.ragged_case(rng.integers(1, 600, b), hkv * g, d, num_kv_heads=hkv, mask_mode=mask,
                              block_size=block, seed=4000 + i, name=f"random_spans_{i}")
    else:
        w = synth.ragged_cross_case(rng.integers(0, 200, b), rng.integers(0, 700, b), hkv * g, d,
                                    num_kv_heads=hkv, seed=4000 + i, name=f"random_cross_spans_{i}")
    return w, chunk, rows


def _f32_case(i):
    rng = np.random.default_rng(5000 + i)
    d = int(rng.choice([16, 32, 64, 128]))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4]))
    ps = int(rng.choice([1, 3, 4, 16, 64]))
    mask = int(rng.integers(0, 3))
    b = int(rng.integers(1, 5))
    kv = rng.integers(1, 1500, b)
    qo = rng.integers(1, 12, b)
    if mask != 0:
        qo = np.minimum(qo, kv)
    block = int(rng.choice([1, 7, 16])) if mask == 2 else 0
    chunk = int(rng.choice([0, 0, 64, 257]))
    w = synth.paged_case(qo, kv, hkv * g, hkv, d, ps, dtype="f32", mask_mode=mask, block_size=block,
                         seed=6000 + i, name=f"random_f32_{i}")
    return w, chunk, 128


def _run_case(w, chunk, rows, gpu, monkeypatch, i):
    monkeypatch.setenv("XATTN_TILE_ROWS", str(rows))
    log(f"[random] {w.name}: hq {w.num_qo_heads} hkv {w.num_kv_heads} d {w.head_dim} page {w.page_size} "
        f"mask {w.mask_mode} block {w.block_size} qo {list(np.diff(w.qo_indptr))} "
        f"kv {list(w.kv_lens())} chunk {chunk} rows {rows}")
    out, lse, plan = run_gpu(w, gpu, chunk)
    log(f"  schedule {plan.info()}")
    ro, rl = ref.run_workload(w)
    compare(out, lse, ro, rl, w.dtype, label=w.name)
    plan.close()


@pytest.mark.parametrize("i", range(N_SPANS))
def test_random_spans(i, gpu, monkeypatch):
    _run_case(*_span_case(i), gpu, monkeypatch, i)


@pytest.mark.parametrize("i", range(N_F32))
def test_random_f32(i, gpu, monkeypatch):
    _run_case(*_f32_case(i), gpu, monkeypatch, i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i, gpu, monkeypatch):
    w, chunk, rows = _case(i)
    monkeypatch.setenv("XATTN_TILE_ROWS", str(rows))
    log(f"[random] case {i}: hq {w.num_qo_heads} hkv {w.num_kv_heads} d {w.head_dim} page {w.page_size} "
        f"mask {w.mask_mode} block {w.block_size} qo {list(np.diff(w.qo_indptr))} "
        f"kv {list(w.kv_lens())} chunk {chunk} rows {rows}")
    out, lse, plan = run_gpu(w, gpu, chunk)
    log(f"  schedule {plan.info()}")
    ro, rl = ref.run_workload(w)
    compare(out, lse, ro, rl, w.dtype, label=w.name)
    plan.close()
