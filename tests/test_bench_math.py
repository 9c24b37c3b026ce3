"""The benchmark's arithmetic on the CPU: algorithmic work per workload, the value and the
roofline fraction from given timings (no GPU involved)."""
import numpy as np

import bench
from ragged_attention_serving_amd import synth


def test_algorithmic_work_matches_the_closed_forms():
    w = synth.whisper_decode(0)
    kv_bytes, flops, decode = bench.workload_numbers(w, {"visible_pairs": 64 * 20 * 1500})
    assert decode and kv_bytes == 64 * 1500 * 20 * 64 * 2 * 2 == 491_520_000
    assert flops == 4 * 64 * 64 * 20 * 1500
    w = synth.ragged_prefill(0)
    work = bench._request_work(w)
    # non-causal cross-attention: every query sees all 1500 keys of its request
    assert int(work.sum()) == 4 * 64 * 20 * 1500 * int(w.qo_indptr[-1]) == 58_129_920_000
    lens = synth.block_causal_span_lengths(np.random.default_rng(0))
    w = synth.Workload(name="b", dtype="bf16", qo_indptr=synth.indptr(lens), kv_indptr=synth.indptr(lens),
                       kv_page_indices=None, kv_last_page_len=None, num_qo_heads=16, num_kv_heads=16,
                       head_dim=128, page_size=1, mask_mode=synth.MASK_BLOCK_CAUSAL, block_size=64)
    pairs = sum(min((i // 64 + 1) * 64, int(L)) for L in lens for i in range(int(L)))
    assert int(bench._request_work(w).sum()) == 4 * 128 * 16 * pairs == 1_669_034_270_720


def test_summary_value_and_roofline():
    w = synth.whisper_decode(0)
    info = {"visible_pairs": 64 * 20 * 1500, "num_units": [0, 1280, 0]}
    m = {"info": info, "cold": [0.090, 0.080, 0.085], "warm": [0.079, 0.081],
         "cold_kernel": {"decode": 0.0768}, "warm_kernel": {"decode": 0.075}, "warm_wall_ms": 0.08,
         "plan_ms": 0.5, "warmup": 5}
    r = bench.summarize(w, m, 3)
    assert r["ms_per_step"] == 0.085 and r["unit"] == "GB/s"
    assert abs(r["value"] - 491.52e6 / 0.085e-3 / 1e9) < 1e-2
    assert abs(r["value_best"] - 491.52e6 / 0.080e-3 / 1e9) < 1e-2
    roof = r["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["kernel"] == "attn_decode_kernel"
    assert abs(roof["achieved"] - 491.52e6 / 0.0768e-3 / 1e9) < 0.01
    assert abs(roof["frac"] - roof["achieved"] / 8000.0) < 1e-4


def test_timed_output_parity_uses_the_baseline_results():
    """The CPU-baseline leg keeps the oracle's results of the requests it covered; the
    bench compares them with the rows of the timed run: the oracle's own rows pass, a
    perturbed row fails."""
    w = synth.tiny_cross(0)
    line, kept = bench.cpu_baseline(w, cpu_seconds=1.0)
    assert line["kind"] == "oracle" and sorted(kept) == list(range(w.batch_size))
    from oracle import ref
    ro, rl = ref.run_workload(w)
    rows = np.concatenate([np.arange(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])) for r in sorted(kept)])
    good = bench.timed_output_parity(w, kept, (ro[rows], rl[rows]))
    assert good["pass"] and good["rows"] == len(rows) and good["max_abs_out_err"] < 1e-6
    bad_o = ro[rows].copy()
    bad_o[0, 0, 0] += 1e-4  # past the fp32 gate of 1e-5
    assert not bench.timed_output_parity(w, kept, (bad_o, rl[rows]))["pass"]
    bad_l = rl[rows].copy()
    bad_l[-1, -1] += 2e-3
    assert not bench.timed_output_parity(w, kept, (ro[rows], bad_l))["pass"]
