"""Pins for the fp64 oracle: facts fixed by the pages and by the mathematics.

Each ``pin_*`` function takes the oracle module and raises AssertionError when the
oracle disagrees with something it does not itself define: a closed form, an
invariant, a library routine or brute force over scalar loops. The same functions
are run against deliberately broken copies of the oracle (test_oracle_mutations.py),
and every planted mistake must trip at least one of them.
"""
from __future__ import annotations

import math

import numpy as np

from ragged_attention_serving_amd import synth

NONE, CAUSAL, BLOCK = 0, 1, 2


# ----------------------------------------------------------------- independent helpers

def _widen(x, dtype):
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, np.float64)


def _token_rows(w, r, hk, pool):
    """Keys or values of request r, head hk, walking the page table one token at a time."""
    npages = int(w.kv_indptr[r + 1] - w.kv_indptr[r])
    if npages == 0:
        return np.zeros((0, w.head_dim))
    last = w.page_size if w.kv_last_page_len is None else int(w.kv_last_page_len[r])
    n = (npages - 1) * w.page_size + last
    rows = []
    for t in range(n):
        logical = int(w.kv_indptr[r]) + t // w.page_size
        phys = logical if w.kv_page_indices is None else int(w.kv_page_indices[logical])
        rows.append(_widen(pool[phys, t % w.page_size, hk], w.dtype))
    return np.array(rows).reshape(n, w.head_dim)


def _n_visible(mask, qo_len, kv_len, i, block):
    """Closed-form count of keys row i sees (queries are the last qo_len positions)."""
    if mask == NONE:
        return kv_len
    pos = kv_len - qo_len + i
    if mask == CAUSAL:
        return pos + 1
    return min((pos // block + 1) * block, kv_len)


def _run(ref, w, **kw):
    return ref.paged_attention(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr,
                               w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
                               w.num_kv_heads, w.page_size, dtype=w.dtype, mask_mode=w.mask_mode,
                               block_size=w.block_size, sm_scale=w.sm_scale, **kw)


def _tiny_cases():
    """Small paged cases over every mask, GQA, partial last pages and an empty context."""
    cases = []
    cases.append(synth.paged_case([2, 5, 1], [9, 23, 4], 4, 2, 8, 4, dtype="f32", seed=11,
                                  mask_mode=NONE))
    cases.append(synth.paged_case([3, 1, 6], [7, 13, 6], 4, 1, 8, 3, dtype="f32", seed=12,
                                  mask_mode=CAUSAL))
    cases.append(synth.paged_case([10, 17], [10, 17], 2, 2, 8, 1, dtype="bf16", seed=13,
                                  mask_mode=BLOCK, block_size=4))
    cases.append(synth.paged_case([4, 2], [0, 5], 2, 2, 4, 2, dtype="f32", seed=14, mask_mode=NONE))
    cases.append(synth.paged_case([2, 3], [5, 11], 6, 3, 16, 4, dtype="bf16", seed=15,
                                  mask_mode=BLOCK, block_size=3))
    return cases


# ----------------------------------------------------------------- pins

def pin_bf16_widening(ref):
    """bf16 bit patterns widen to the values IEEE-754 binary16-brain fixes."""
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x7F7F, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.5, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 3.140625]
    got = ref.to_f64(bits, "bf16")
    assert np.array_equal(got, np.array(want)), got


def pin_lengths(ref):
    """Hand-worked page-table lengths: pages [2,0,3], last [3,4,1], page_size 4 -> [7,0,9]."""
    qo, kv = ref.request_lengths([0, 1, 1, 4], [0, 2, 2, 5], [3, 4, 1], 4)
    assert list(qo) == [1, 0, 3] and list(kv) == [7, 0, 9], (qo, kv)


def pin_uniform_scores(ref):
    """Q = 0 makes every visible score equal: O = mean of visible V, lse = ln(count)."""
    for w in _tiny_cases() + [synth.tiny_cross(0)]:
        w.q = np.zeros_like(w.q)
        out, lse = _run(ref, w)
        g = w.num_qo_heads // w.num_kv_heads
        qo_lens = w.qo_lens()
        for r in range(w.batch_size):
            kv_len = int(w.kv_lens()[r])
            for h in range(w.num_qo_heads):
                V = _token_rows(w, r, h // g, w.v_pages)
                for i in range(int(qo_lens[r])):
                    row = int(w.qo_indptr[r]) + i
                    n = _n_visible(w.mask_mode, int(qo_lens[r]), kv_len, i, w.block_size)
                    if n <= 0:
                        assert lse[row, h] == -np.inf and np.all(out[row, h] == 0)
                        continue
                    assert abs(lse[row, h] - math.log(n)) < 1e-12, (w.name, r, i, lse[row, h], n)
                    assert np.allclose(out[row, h], V[:n].mean(axis=0), atol=1e-12, rtol=0)
    # the tiny cross-attention workload: contexts of 16 and 40 keys
    w = synth.tiny_cross(0)
    w.q = np.zeros_like(w.q)
    _, lse = _run(ref, w)
    assert np.allclose(lse[0], 2.772588722239781) and np.allclose(lse[1:], 3.6888794541139363)


def pin_single_key(ref):
    """One key: O = V_0 and lse = scale * q . k_0."""
    w = synth.paged_case([3, 1], [1, 1], 4, 2, 8, 2, dtype="f32", seed=21)
    out, lse = _run(ref, w)
    g = 2
    for r in range(2):
        for h in range(4):
            k0 = _token_rows(w, r, h // g, w.k_pages)[0]
            v0 = _token_rows(w, r, h // g, w.v_pages)[0]
            for i in range(int(w.qo_lens()[r])):
                row = int(w.qo_indptr[r]) + i
                s = math.fsum(float(a) * float(b) for a, b in zip(w.q[row, h], k0)) / math.sqrt(8)
                assert abs(lse[row, h] - s) < 1e-12
                assert np.allclose(out[row, h], v0, atol=1e-14, rtol=0)


def pin_two_keys(ref):
    """Two keys: O = sigma(s0 - s1) V0 + sigma(s1 - s0) V1, lse = log(e^s0 + e^s1)."""
    w = synth.paged_case([2], [2], 2, 2, 4, 1, dtype="f32", seed=22, sm_scale=0.7)
    out, lse = _run(ref, w)
    for h in range(2):
        K = _token_rows(w, 0, h, w.k_pages)
        V = _token_rows(w, 0, h, w.v_pages)
        for i in range(2):
            q = w.q[i, h].astype(np.float64)
            s0, s1 = 0.7 * float(q @ K[0]), 0.7 * float(q @ K[1])
            sig = 1.0 / (1.0 + math.exp(s1 - s0))
            assert np.allclose(out[i, h], sig * V[0] + (1 - sig) * V[1], atol=1e-13, rtol=0)
            assert abs(lse[i, h] - np.logaddexp(s0, s1)) < 1e-12


def pin_page_permutation(ref):
    """Moving pages in the pool and remapping the table leaves the result unchanged."""
    for w in _tiny_cases():
        out, lse = _run(ref, w)
        rng = np.random.default_rng(5)
        n = w.k_pages.shape[0]
        perm = rng.permutation(n)  # new position of old page p is perm[p]
        kp = np.empty_like(w.k_pages)
        vp = np.empty_like(w.v_pages)
        kp[perm] = w.k_pages
        vp[perm] = w.v_pages
        w.k_pages, w.v_pages = kp, vp
        w.kv_page_indices = perm[w.kv_page_indices].astype(np.int32)
        out2, lse2 = _run(ref, w)
        assert np.array_equal(out, out2, equal_nan=True) and np.array_equal(lse, lse2, equal_nan=True)


def pin_gqa_repeat(ref):
    """GQA equals multi-head attention over KV heads repeated Hq/Hkv times, consecutively."""
    for mask, blk in ((NONE, 0), (CAUSAL, 0), (BLOCK, 3)):
        w = synth.paged_case([2, 4], [6, 9], 6, 2, 8, 2, dtype="f32", seed=23, mask_mode=mask,
                             block_size=blk)
        out, lse = _run(ref, w)
        w.k_pages = np.repeat(w.k_pages, 3, axis=2)
        w.v_pages = np.repeat(w.v_pages, 3, axis=2)
        w.num_kv_heads = 6
        out2, lse2 = _run(ref, w)
        assert np.allclose(out, out2, atol=1e-14, rtol=0) and np.allclose(lse, lse2, atol=1e-14, rtol=0)


def pin_key_shift(ref):
    """Adding u to every key leaves O unchanged and adds scale * q . u to lse."""
    w = synth.paged_case([3, 2], [7, 5], 2, 2, 8, 3, dtype="f32", seed=24, mask_mode=CAUSAL)
    out, lse = _run(ref, w)
    u = np.random.default_rng(1).standard_normal(8)
    w.k_pages = w.k_pages.astype(np.float64) + u
    out2, lse2 = _run(ref, w)
    shift = np.einsum("nhd,d->nh", w.q.astype(np.float64), u) / math.sqrt(8)
    assert np.allclose(out, out2, atol=1e-12, rtol=0)
    assert np.allclose(lse + shift, lse2, atol=1e-12, rtol=0)


def pin_value_affine(ref):
    """V -> a V + b maps O -> a O + b (softmax weights sum to one)."""
    w = synth.paged_case([2, 3], [5, 8], 2, 2, 4, 2, dtype="f32", seed=25, mask_mode=BLOCK, block_size=2)
    out, _ = _run(ref, w)
    b = np.array([0.5, -1.0, 2.0, 3.0])
    w.v_pages = -1.5 * w.v_pages.astype(np.float64) + b
    out2, _ = _run(ref, w)
    assert np.allclose(-1.5 * out + b, out2, atol=1e-12, rtol=0)


def pin_request_permutation(ref):
    """Packing the requests in another order moves each request's rows with it."""
    w = synth.paged_case([2, 1, 3], [5, 9, 4], 2, 2, 4, 2, dtype="f32", seed=26, mask_mode=CAUSAL)
    out, lse = _run(ref, w)
    order = [2, 0, 1]
    qo = w.qo_lens()
    npg = np.diff(w.kv_indptr)
    rows = np.concatenate([np.arange(w.qo_indptr[r], w.qo_indptr[r + 1]) for r in order])
    pages = np.concatenate([w.kv_page_indices[w.kv_indptr[r]:w.kv_indptr[r + 1]] for r in order])
    w2 = synth.Workload(name="perm", dtype="f32", qo_indptr=synth.indptr(qo[order]),
                        kv_indptr=synth.indptr(npg[order]), kv_page_indices=pages.astype(np.int32),
                        kv_last_page_len=w.kv_last_page_len[order], num_qo_heads=2, num_kv_heads=2,
                        head_dim=4, page_size=2, mask_mode=CAUSAL, q=w.q[rows], k_pages=w.k_pages,
                        v_pages=w.v_pages)
    out2, lse2 = _run(ref, w2)
    assert np.array_equal(out[rows], out2) and np.array_equal(lse[rows], lse2)


def pin_split_merge(ref):
    """Attention over disjoint key ranges, merged on the log-sum-exp, equals the whole."""
    rng = np.random.default_rng(27)
    Q, K, V = rng.standard_normal((5, 8)), rng.standard_normal((23, 8)), rng.standard_normal((23, 8))
    vis = np.ones((5, 23), bool)
    vis[0, 3:] = False  # a row that sees only the first chunk
    vis[1, :] = False  # a row that sees nothing
    O, lse = ref.attend(Q, K, V, vis, 0.3)
    for cuts in ([0, 10, 23], [0, 1, 2, 16, 23], [0, 3, 3, 23]):
        parts = [ref.attend(Q, K[a:b], V[a:b], vis[:, a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
        Om, lm = ref.merge_states([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(O, Om, atol=1e-13, rtol=0)
        assert np.array_equal(np.isinf(lse), np.isinf(lm))
        assert np.allclose(lse[np.isfinite(lse)], lm[np.isfinite(lm)], atol=1e-13, rtol=0)
    assert lse[1] == -np.inf and np.all(O[1] == 0)


def pin_library_sdpa(ref):
    """torch's scaled_dot_product_attention (fp64, CPU, explicit boolean mask) and
    scipy's logsumexp agree with the oracle on every row that sees a key."""
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    for w in _tiny_cases():
        out, lse = _run(ref, w)
        g = w.num_qo_heads // w.num_kv_heads
        qo_lens = w.qo_lens()
        for r in range(w.batch_size):
            kv_len = int(w.kv_lens()[r])
            nq = int(qo_lens[r])
            if kv_len == 0 or nq == 0:
                continue
            j = np.arange(kv_len)[None, :]
            n_vis = np.array([_n_visible(w.mask_mode, nq, kv_len, ii, w.block_size) for ii in range(nq)])
            mask = j < n_vis[:, None]
            for h in range(w.num_qo_heads):
                K = _token_rows(w, r, h // g, w.k_pages)
                V = _token_rows(w, r, h // g, w.v_pages)
                Q = _widen(w.q[w.qo_indptr[r]:w.qo_indptr[r + 1], h], w.dtype)
                sc = 1.0 / math.sqrt(w.head_dim)
                o = F.scaled_dot_product_attention(torch.from_numpy(Q)[None], torch.from_numpy(K)[None],
                                                   torch.from_numpy(V)[None],
                                                   attn_mask=torch.from_numpy(mask)[None], scale=sc)[0].numpy()
                S = np.where(mask, sc * (Q @ K.T), -np.inf)
                ls = logsumexp(S, axis=1)
                rows = slice(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1]))
                assert np.allclose(out[rows, h], o, atol=1e-12, rtol=0), (w.name, r, h)
                assert np.allclose(lse[rows, h], ls, atol=1e-12, rtol=0)


def _brute(w):
    """Scalar loops with math.fsum: out and lse for every row of a paged workload."""
    g = w.num_qo_heads // w.num_kv_heads
    nq = int(w.qo_indptr[-1])
    out = np.zeros((nq, w.num_qo_heads, w.head_dim))
    lse = np.full((nq, w.num_qo_heads), -np.inf)
    sc = w.scale
    for r in range(w.batch_size):
        kv_len = int(w.kv_lens()[r])
        nqr = int(w.qo_lens()[r])
        for h in range(w.num_qo_heads):
            K = _token_rows(w, r, h // g, w.k_pages).tolist()
            V = _token_rows(w, r, h // g, w.v_pages).tolist()
            for i in range(nqr):
                row = int(w.qo_indptr[r]) + i
                q = _widen(w.q[row, h], w.dtype).tolist()
                n = _n_visible(w.mask_mode, nqr, kv_len, i, w.block_size)
                if n <= 0:
                    continue
                s = [sc * math.fsum(a * b for a, b in zip(q, K[j])) for j in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for d in range(w.head_dim):
                    out[row, h, d] = math.fsum(e[j] * V[j][d] for j in range(n)) / tot
                lse[row, h] = m + math.log(tot)
    return out, lse


def pin_brute_force(ref):
    """Scalar-loop brute force on the tiny cross-attention workload and the small cases."""
    for w in [synth.tiny_cross(0)] + _tiny_cases():
        out, lse = _run(ref, w)
        bo, bl = _brute(w)
        assert np.allclose(out, bo, atol=1e-12, rtol=0), w.name
        assert np.array_equal(np.isinf(lse), np.isinf(bl))
        fin = np.isfinite(bl)
        assert np.allclose(lse[fin], bl[fin], atol=1e-12, rtol=0)


def pin_cacheless_slices(ref):
    """Cacheless spans: slicing the packed tensors equals brute force over the spans, for
    self-attention within each span under every mask and for cross-attention between a
    request's query span and its (differently sized) key span."""
    cases = [synth.ragged_case([5, 9, 1], 4, 8, num_kv_heads=2, dtype="bf16", block_size=4, seed=28),
             synth.ragged_case([7, 2, 12], 2, 8, dtype="f32", mask_mode=NONE, seed=29),
             synth.ragged_case([6, 1, 11], 4, 8, num_kv_heads=1, dtype="bf16", mask_mode=CAUSAL, seed=30),
             synth.ragged_cross_case([3, 7, 0, 2], [9, 4, 5, 0], 4, 8, num_kv_heads=2, dtype="bf16", seed=31),
             synth.ragged_cross_case([1, 5], [17, 6], 2, 16, dtype="f32", seed=32)]
    for w in cases:
        out, lse = ref.ragged_attention(w.q, w.k_pages, w.v_pages, w.meta["cu_seqlens"], w.num_qo_heads,
                                        w.num_kv_heads, dtype=w.dtype, mask_mode=w.mask_mode,
                                        block_size=w.block_size,
                                        cu_seqlens_kv=w.meta.get("cu_seqlens_kv"))
        bo, bl = _brute(w)
        assert np.allclose(out, bo, atol=1e-12, rtol=0), w.name
        assert np.array_equal(np.isinf(lse), np.isinf(bl)), w.name
        fin = np.isfinite(bl)
        assert np.allclose(lse[fin], bl[fin], atol=1e-12, rtol=0), w.name


def _dispatch_cases():
    """Workloads of each route of the oracle's workload entry point: cacheless spans under
    every mask (an empty span among them), cacheless cross-attention between differently
    sized query and key spans with empty spans on either side, and a shuffled paged table."""
    return [synth.ragged_case([5, 9, 0, 1], 4, 8, num_kv_heads=2, dtype="bf16", mask_mode=NONE, seed=60),
            synth.ragged_case([6, 1, 11, 0], 4, 8, num_kv_heads=1, dtype="bf16", mask_mode=CAUSAL, seed=61),
            synth.ragged_case([7, 0, 12], 2, 8, dtype="f32", mask_mode=BLOCK, block_size=4, seed=62),
            synth.ragged_cross_case([3, 0, 7, 2, 4], [9, 4, 0, 5, 1], 4, 8, num_kv_heads=2, dtype="bf16",
                                    seed=63),
            synth.paged_case([2, 0, 3, 1], [7, 5, 11, 0], 4, 2, 8, 3, dtype="f32", mask_mode=CAUSAL, seed=64)]


def pin_run_workload(ref):
    """The oracle's entry point over a workload (the one every GPU comparison calls)
    equals scalar brute force that walks the workload's own page table token by token:
    cacheless spans (identity table, page_size 1) under every mask, cross-attention whose
    keys come from the second span set, and a paged table."""
    for w in _dispatch_cases():
        out, lse = ref.run_workload(w)
        bo, bl = _brute(w)
        assert out.shape == bo.shape, (w.name, out.shape, bo.shape)
        assert np.allclose(out, bo, atol=1e-12, rtol=0), w.name
        assert np.array_equal(np.isinf(lse), np.isinf(bl)), w.name
        fin = np.isfinite(bl)
        assert np.allclose(lse[fin], bl[fin], atol=1e-12, rtol=0), w.name


def pin_workload_subsets(ref):
    """A run restricted to some requests and heads reproduces exactly those rows and heads
    of the full run and leaves every other entry NaN (the sampled comparisons rely on it)."""
    for w in _dispatch_cases():
        full_o, full_l = ref.run_workload(w)
        nq, hq = full_l.shape
        for reqs, heads in (([2, 0], sorted({hq - 1, hq // 2}, reverse=True)), ([w.batch_size - 1], None),
                            (None, [0])):
            so, sl = ref.run_workload(w, requests=reqs, heads=heads)
            sel = np.zeros((nq, hq), bool)
            rs = range(w.batch_size) if reqs is None else reqs
            hs = list(range(hq)) if heads is None else heads
            for r in rs:
                for h in hs:
                    sel[int(w.qo_indptr[r]):int(w.qo_indptr[r + 1]), h] = True
            assert np.array_equal(so[sel], full_o[sel]), (w.name, reqs, heads)
            assert np.array_equal(sl[sel], full_l[sel]), (w.name, reqs, heads)
            assert np.isnan(so[~sel]).all() and np.isnan(sl[~sel]).all(), (w.name, reqs, heads)


def _write_cases():
    """Shuffled pages with spare pages and partial last pages, an empty context, page
    sizes 1, 3 and 4, bf16 and fp32, and the identity table."""
    return [synth.paged_case([1, 1, 1], [9, 0, 6], 2, 2, 4, 4, dtype="f32", seed=50, extra_pages=3),
            synth.paged_case([1, 2], [7, 5], 4, 2, 8, 3, dtype="bf16", seed=51, extra_pages=2),
            synth.ragged_case([3, 5], 2, 4, dtype="f32", mask_mode=NONE, seed=52)]


def pin_context_write(ref):
    """The context write puts position t of request r at slot t % page_size of the page
    the table lists for t // page_size (walked one position at a time here), bit for bit,
    and leaves every other slot of both pools as it was."""
    for w in _write_cases():
        ks, vs = synth.context_source(w, seed=7)
        kp, vp = ref.write_context(ks, vs, w.k_pages, w.v_pages, w.kv_indptr, w.kv_page_indices,
                                   w.kv_last_page_len, w.page_size)
        written = np.zeros(w.k_pages.shape[:2], bool)
        row = 0
        for r in range(w.batch_size):
            npages = int(w.kv_indptr[r + 1] - w.kv_indptr[r])
            last = w.page_size if w.kv_last_page_len is None else int(w.kv_last_page_len[r])
            n = 0 if npages == 0 else (npages - 1) * w.page_size + last
            for t in range(n):
                logical = int(w.kv_indptr[r]) + t // w.page_size
                phys = logical if w.kv_page_indices is None else int(w.kv_page_indices[logical])
                assert np.array_equal(kp[phys, t % w.page_size], ks[row]), (w.name, r, t)
                assert np.array_equal(vp[phys, t % w.page_size], vs[row]), (w.name, r, t)
                written[phys, t % w.page_size] = True
                row += 1
        assert row == ks.shape[0]
        assert np.array_equal(kp[~written], w.k_pages[~written]), w.name
        assert np.array_equal(vp[~written], w.v_pages[~written]), w.name


ALL_PINS = [pin_bf16_widening, pin_lengths, pin_uniform_scores, pin_single_key, pin_two_keys,
            pin_page_permutation, pin_gqa_repeat, pin_key_shift, pin_value_affine,
            pin_request_permutation, pin_split_merge, pin_library_sdpa, pin_brute_force,
            pin_cacheless_slices, pin_run_workload, pin_workload_subsets, pin_context_write]
