"""Host partitioner: every visible (row, key) pair is covered exactly once, split rows
have a consistent merge map, and units are ordered longest first (CPU only).

The checks re-derive coverage from the unit and merge records independently of the
C++ partitioner."""
import numpy as np
import pytest

import ragged_attention_serving_amd as xa
from ragged_attention_serving_amd import synth


def last_visible(mask, block, qo, kv, qi):
    if kv <= 0:
        return -1
    pos = kv - qo + qi
    if mask == 0:
        return kv - 1
    if mask == 1:
        return min(pos, kv - 1)
    return min((pos // block + 1) * block, kv) - 1


def check_schedule(qo_lens, kv_lens, hq, hkv, page_size, mask, block, dtype, force_chunk=0, d=64):
    kv_indptr, idx, last, total = synth.page_table(kv_lens, page_size, None)
    qo_indptr = synth.indptr(qo_lens)
    info, units, merges = xa.xattn_schedule(qo_indptr, kv_indptr, idx, last, hq, hkv, d if dtype == "bf16" else 16,
                                            page_size, max(total, 1), mask, block, dtype, force_chunk)
    g = hq // hkv
    B = len(qo_lens)
    caps = {0: 4, 1: 8, 2: 128}
    # family of each unit from the counts
    fam = np.repeat([0, 1, 2], info["num_units"])
    assert len(units) == sum(info["num_units"])
    cover = {}  # (r, hk, row) -> list of (kv0, kv1, ws_row_for_row)
    ws_seen = set()
    for f, u in zip(fam, units):
        r, hk, row0, nrows, kv0, kv1, ws_row, cost = map(int, u)
        rows = qo_lens[r] * g
        assert 0 <= r < B and 0 <= hk < hkv and qo_lens[r] > 0
        assert 1 <= nrows <= caps[f] and 0 <= row0 and row0 + nrows <= rows
        assert 0 <= kv0 <= kv1 <= kv_lens[r]
        if dtype == "f32":
            assert f == 0
        elif rows > 8:
            assert f == 2
        else:
            assert f in (1, 2)
        if force_chunk:
            assert kv1 - kv0 <= force_chunk
        for rr in range(nrows):
            w = -1 if ws_row < 0 else ws_row + rr
            if w >= 0:
                assert w not in ws_seen
                ws_seen.add(w)
                assert w < info["workspace_rows"]
            cover.setdefault((r, hk, row0 + rr), []).append((kv0, kv1, w))
    # every row of every request with queries is covered; keys exactly once
    out_written = {}
    merge_by_out = {int(m[0]): m for m in merges}
    for r in range(B):
        for hk in range(hkv):
            for row in range(qo_lens[r] * g):
                qi, h = row // g, hk * g + row % g
                lst = sorted(cover[(r, hk, row)])
                lim = last_visible(mask, block, qo_lens[r], kv_lens[r], qi)
                covered = np.zeros(kv_lens[r], int)
                for kv0, kv1, _ in lst:
                    covered[kv0:kv1] += 1
                assert covered.max(initial=0) <= 1
                assert covered[:lim + 1].min(initial=1) == 1, (r, hk, row)
                out_row = (synth.indptr(qo_lens)[r] + qi) * hq + h
                if len(lst) == 1 and lst[0][2] < 0:
                    assert out_row not in merge_by_out
                else:
                    m = merge_by_out[out_row]
                    nch, stride, ws0 = int(m[2]), int(m[3]), int(m[1])
                    assert nch == len(lst)
                    got = sorted(ws0 + c * stride for c in range(nch))
                    assert got == sorted(w for _, _, w in lst)
                out_written[out_row] = out_written.get(out_row, 0) + 1
    assert all(v == 1 for v in out_written.values())
    assert len(merges) == info["num_merge_rows"]
    # decode units: longest first
    c = units[fam == 1][:, 7]
    assert np.all(np.diff(c) <= 0)
    # tile units: each (request, kv head) group on one XCD (launch position mod 8), its units
    # consecutive in that XCD's sequence (a group is split only when no XCD has room left)
    for f in (0, 2):
        fu = units[fam == f]
        if len(fu) <= 8:
            continue
        split = 0
        groups = {}
        for pos, u in enumerate(fu):
            groups.setdefault((int(u[0]), int(u[1])), []).append(pos)
        for key, pos in groups.items():
            res = {p % 8 for p in pos}
            if len(res) > 1:
                split += 1
                continue
            seq = [p // 8 for p in pos]
            assert seq == list(range(seq[0], seq[0] + len(seq))), key
        assert split <= max(8, len(groups) // 4), (split, len(groups))
    return info, units, merges


CASES = [
    ([1] * 5, [100, 1, 37, 1500, 64], 4, 4, 16, 0, 0, "bf16"),
    ([1] * 7, [5000, 512, 700, 9, 33, 1, 2], 8, 2, 16, 1, 0, "bf16"),
    ([3, 1, 2], [20, 9, 40], 6, 3, 4, 1, 0, "bf16"),
    ([200, 7, 129, 1], [300, 9, 900, 1], 4, 4, 16, 0, 0, "bf16"),
    ([130, 64, 300], [130, 64, 300], 2, 2, 1, 2, 64, "bf16"),
    ([50, 3], [77, 3], 2, 1, 5, 2, 7, "bf16"),
    ([1, 3], [16, 40], 2, 2, 4, 0, 0, "f32"),
    ([9, 2, 5], [30, 2000, 5], 4, 2, 3, 1, 0, "f32"),
    ([0, 4, 0], [10, 0, 7], 2, 2, 4, 0, 0, "bf16"),
]


@pytest.mark.parametrize("case", CASES)
def test_coverage_default(case):
    check_schedule(*case)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("chunk", [1, 17, 64, 256])
def test_coverage_forced_chunks(case, chunk):
    check_schedule(*case, force_chunk=chunk)


def test_random_cases():
    rng = np.random.default_rng(3)
    for _ in range(40):
        b = int(rng.integers(1, 6))
        mask = int(rng.integers(0, 3))
        hkv = int(rng.integers(1, 4))
        hq = hkv * int(rng.choice([1, 2, 4]))
        kv = rng.integers(0 if mask == 0 else 1, 700, b)
        qo = np.array([int(rng.integers(0, (k if mask else 300) + 1)) for k in kv])
        if mask:
            qo = np.minimum(qo, kv)
        check_schedule(list(map(int, qo)), list(map(int, kv)), hq, hkv, int(rng.integers(1, 20)), mask,
                       int(rng.integers(1, 100)), "bf16" if rng.random() < 0.8 else "f32",
                       force_chunk=int(rng.choice([0, 0, 33, 128])))


def test_decode_split_sizes():
    """Whisper-style decode: 64 x 1500-key contexts split evenly into 64-key multiples."""
    info, units, merges = check_schedule([1] * 64, [1500] * 64, 20, 20, 16, 0, 0, "bf16")
    assert info["num_units"][1] == len(units)
    lens = units[:, 5] - units[:, 4]
    assert lens.max() - lens.min() <= 64
    assert info["decode_rows"] == 1


def test_gqa_decode_rows():
    info, units, _ = check_schedule([1] * 4, [700, 9000, 20, 513], 32, 8, 16, 1, 0, "bf16", d=128)
    assert info["decode_rows"] == 4


def test_visible_pairs_counts_the_mask():
    info, _, _ = check_schedule([64], [64], 1, 1, 1, 2, 16, "bf16")
    # block-causal, 4 blocks of 16: row i sees (i // 16 + 1) * 16 keys
    assert info["visible_pairs"] == sum((i // 16 + 1) * 16 for i in range(64))


@pytest.mark.parametrize("ps,chunk", [(1, 0), (1, 5000), (16, 0), (3, 0), (16, 100000)])
def test_mma_units_stay_within_the_page_cap(ps, chunk):
    """A paged MFMA unit stages its page indices in LDS: it may span at most 1024 pages."""
    kv = [40000, 17000, 2048] if ps > 1 else [9000, 2500, 300]
    qo = [300, 9, 129]
    kv_indptr, idx, last, total = synth.page_table(kv, ps, None)
    info, units, _ = xa.xattn_schedule(synth.indptr(qo), kv_indptr, idx, last, 4, 4, 64, ps, total, 0, 0,
                                       "bf16", chunk)
    mma = units[sum(info["num_units"][:2]):]
    assert len(mma)
    for u in mma:
        kv0, kv1 = int(u[4]), int(u[5])
        if kv1 > kv0:
            assert (kv1 - 1) // ps - kv0 // ps + 1 <= 1024, (kv0, kv1)
    check_schedule(qo, kv, 4, 4, ps, 0, 0, "bf16", force_chunk=chunk)


def test_short_requests_ride_with_prefill():
    """A batch whose KV traffic is mostly prefill runs its short requests in the tile launch."""
    info, units, _ = check_schedule([300, 1, 2, 200], [1500] * 4, 4, 4, 16, 0, 0, "bf16")
    assert info["num_units"][1] == 0 and info["num_units"][2] > 0
    info, units, _ = check_schedule([1] * 30 + [20], [1500] * 31, 4, 4, 16, 0, 0, "bf16")
    assert info["num_units"][1] > 0 and info["num_units"][2] > 0


@pytest.mark.parametrize("ps,chunk", [(1, 0), (1, 9000), (16, 0), (16, 100000)])
def test_decode_units_stay_within_the_page_cap(ps, chunk):
    """A paged decode unit stages its page indices in LDS: it may span at most 2048 pages."""
    kv = [40000, 3000, 70000] if ps > 1 else [9000, 2500, 5000]
    kv_indptr, idx, last, total = synth.page_table(kv, ps, None)
    info, units, _ = xa.xattn_schedule(synth.indptr([1, 1, 1]), kv_indptr, idx, last, 4, 4, 64, ps, total, 0, 0,
                                       "bf16", chunk)
    assert info["num_units"][1] == len(units) > 0
    for u in units:
        kv0, kv1 = int(u[4]), int(u[5])
        if kv1 > kv0:
            assert (kv1 - 1) // ps - kv0 // ps + 1 <= 2048, (kv0, kv1)
    check_schedule([1, 1, 1], kv, 4, 4, ps, 0, 0, "bf16", force_chunk=chunk)
