"""GPU parity where the running max moves: scores that drift along each context, and
softmax scales far from 1/sqrt(head_dim).

With N(0,1) inputs and the default scale the scores stay within a few units, so a kernel's
running max rarely moves after its first key tile. Here a shared direction is given to every
query and, growing (or shrinking) with the key's position, to every key, so the scaled scores
drift by a fixed step per key: rising scores move the max again and again (and rescale the
partial sums each time), falling ones leave the first tile's max in place while the later
weights shrink toward underflow. Every kernel family runs each case, unsplit and with forced
64-key chunks (whose partial results the merge combines across a wide spread of lse).

Tolerances: bf16 as everywhere (2e-2 on out, 1e-3 on lse). The fp32 gate of 1e-5 on out
holds for scores of order one (|s| up to about 4 in the seeded fp32 workload); an fp32
score carries a rounding error relative to its own size, and a weight exp(s - m) carries
that error as a relative one, so here the fp32 out gate is 1e-5 * max(1, s_max / 4), with
s_max the largest |scaled score| over the case's visible pairs, taken in fp64.
"""
import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.gpu_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu

# (name, qo_lens, kv_lens, hq, hkv, d, page_size, mask, block, dtype): one per kernel family
FAMILIES = [
    ("decode_d64", [1, 1, 1], [100, 700, 1000], 4, 4, 64, 16, 0, 0, "bf16"),
    ("decode_gqa4_d128_causal", [1, 1], [300, 1000], 8, 2, 128, 16, 1, 0, "bf16"),
    ("tiles_d64", [70, 20], [900, 400], 2, 2, 64, 16, 0, 0, "bf16"),
    ("tiles_d128_causal", [130, 33], [800, 500], 4, 2, 128, 16, 1, 0, "bf16"),
    ("tiles_d128_block", [300, 700], [300, 700], 2, 2, 128, 1, 2, 64, "bf16"),
    ("f32_d32", [3, 1], [600, 250], 2, 2, 32, 8, 0, 0, "f32"),
]


def _case(fam, sm_scale=0.0, seed=0):
    name, qo, kv, hq, hkv, d, ps, mask, blk, dt = fam
    if ps == 1:  # cacheless spans: the identity table
        return synth.ragged_case(qo, hq, d, num_kv_heads=hkv, dtype=dt, mask_mode=mask,
                                 block_size=blk, seed=seed, name=name, sm_scale=sm_scale)
    return synth.paged_case(qo, kv, hq, hkv, d, ps, dtype=dt, mask_mode=mask, block_size=blk,
                            seed=seed, name=name, sm_scale=sm_scale)


def _f32(a, dtype):
    return synth.bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)


def _store(a, dtype):
    return synth.round_to_bf16_bits(a) if dtype == "bf16" else a.astype(np.float32)


def with_drift(w, nats_per_key):
    """w with dimension 0 of every query set to c and of the key at context position t set to
    beta * t (beta of the sign of the drift), so that the scaled score of that key moves by
    nats_per_key per position on top of the N(0,1) part of the other dimensions."""
    c = 4.0
    beta = nats_per_key / (w.scale * c)
    q = _f32(w.q, w.dtype)
    q[:, :, 0] = c
    k = _f32(w.k_pages, w.dtype)
    kv_lens = w.kv_lens()
    for r in range(w.batch_size):
        t = np.arange(int(kv_lens[r]))
        if w.kv_page_indices is None:  # identity table: request r's keys are rows kv_indptr[r]...
            k[int(w.kv_indptr[r]) + t, 0, :, 0] = (beta * t)[:, None]
        else:
            pages = w.kv_page_indices[w.kv_indptr[r] + t // w.page_size]
            k[pages, t % w.page_size, :, 0] = (beta * t)[:, None]
    w.q, w.k_pages = _store(q, w.dtype), _store(k, w.dtype)
    w.name += f"_drift{nats_per_key:+g}"
    return w


def max_abs_score(w):
    """Largest |scale * q.k| over the visible (query, key) pairs of w, in fp64."""
    q, pool = ref.to_f64(w.q, w.dtype), ref.to_f64(w.k_pages, w.dtype)
    group = w.num_qo_heads // w.num_kv_heads
    qo_lens, kv_lens = w.qo_lens(), w.kv_lens()
    best = 0.0
    for r in range(w.batch_size):
        nq, nk = int(qo_lens[r]), int(kv_lens[r])
        if nq == 0 or nk == 0:
            continue
        vis = ref.visible(w.mask_mode, nq, nk, w.block_size)
        for h in range(w.num_qo_heads):
            if w.kv_page_indices is None:
                k = pool[int(w.kv_indptr[r]):int(w.kv_indptr[r]) + nk, 0, h // group]
            else:
                k = ref.gather_pages(pool, w.kv_indptr, w.kv_page_indices, r, nk, w.page_size, h // group)
            s = np.abs(w.scale * q[int(w.qo_indptr[r]):int(w.qo_indptr[r + 1]), h] @ k.T)
            best = max(best, float(s[vis].max()))
    return best


def _check(w, gpu, chunk):
    log(f"[rescale] {w.name} scale={w.scale:.4g} chunk={chunk}")
    out, lse, plan = run_gpu(w, gpu, chunk)
    ro, rl = ref.run_workload(w)
    tol = None
    if w.dtype == "f32":
        tol = (1e-5 * max(1.0, max_abs_score(w) / 4.0), 1e-3)
    compare(out, lse, ro, rl, w.dtype, label=f"{w.name} chunk={chunk}", tol=tol)
    return rl


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("chunk", [0, 64])
def test_rising_scores(fam, chunk, gpu):
    # 0.1 nats per key: about 9 log2 units per 64-key tile, past the 2^8 rescale slack
    rl = _check(with_drift(_case(fam), 0.1), gpu, chunk)
    assert np.nanmax(rl) > 20.0  # the drift dominates the lse


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_falling_scores(fam, gpu):
    _check(with_drift(_case(fam), -0.1), gpu, 0)


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("factor", [8.0, 1e-3])
def test_softmax_scale_far_from_default(fam, factor, gpu):
    d = fam[5]
    _check(_case(fam, sm_scale=factor / np.sqrt(d)), gpu, 0)
