"""The C ABI from plain C: include/xattn.h compiles as C11 and C++17, and a C11 program
linked against libxattn.so (tests/c_client/xattn_client.c) plans and runs workloads
that the oracle checks."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import ref
from ragged_attention_serving_amd import synth
from tests.c_client import build_client
from tests.gpu_util import TOL, log

HEADER = os.path.join(build_client.ROOT, "include", "xattn.h")


@pytest.mark.parametrize("lang,std", [("c", "c11"), ("c", "c99"), ("c++", "c++17")])
def test_header_compiles(lang, std, tmp_path):
    """xattn.h is self-contained and warning-free in C and C++ (no HIP or C++ types)."""
    cc = shutil.which("gcc" if lang == "c" else "g++")
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "xattn.h"\nint main(void) { xattn_plan_t h = 0; (void)h; return 0; }\n')
    r = subprocess.run([cc, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        "-I", os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_client_host_only():
    """Schedule, validation errors with messages, and destroy(NULL), called from C."""
    exe = build_client.build()
    r = subprocess.run([exe, "--host-only"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "host-only ok" in r.stdout


def _write_workload(w, d):
    has_pages = w.kv_page_indices is not None
    has_last = w.kv_last_page_len is not None
    q_rows = int(w.qo_indptr[-1])
    dtype = 1 if w.dtype == "bf16" else 0
    (d / "meta.txt").write_text(
        f"{w.batch_size} {w.num_qo_heads} {w.num_kv_heads} {w.head_dim} {w.page_size} {w.num_pages} "
        f"{w.mask_mode} {w.block_size} {dtype} {q_rows} {int(has_pages)} {int(has_last)} {w.sm_scale!r}\n")
    np.ascontiguousarray(w.qo_indptr, dtype=np.int32).tofile(d / "qo_indptr.bin")
    np.ascontiguousarray(w.kv_indptr, dtype=np.int32).tofile(d / "kv_indptr.bin")
    if has_pages:
        np.ascontiguousarray(w.kv_page_indices, dtype=np.int32).tofile(d / "kv_page_indices.bin")
    if has_last:
        np.ascontiguousarray(w.kv_last_page_len, dtype=np.int32).tofile(d / "kv_last_page_len.bin")
    for name, a in (("q", w.q), ("k", w.k_pages), ("v", w.v_pages)):
        np.ascontiguousarray(a).tofile(d / f"{name}.bin")
    return q_rows


CASES = {
    "tiny_cross_f32": lambda: synth.tiny_cross(0),
    "paged_gqa_causal_prefill": lambda: synth.paged_case([5, 130, 1], [300, 700, 64], 8, 2, 128, 16,
                                                         mask_mode=synth.MASK_CAUSAL, seed=11,
                                                         name="paged_gqa_causal_prefill"),
    "decode_cross": lambda: synth.paged_case([1] * 6, [1500, 37, 900, 16, 1, 2000], 4, 4, 64, 16, seed=12,
                                             name="decode_cross"),
    "cacheless_block_causal": lambda: synth.ragged_case([200, 67, 330], 2, 64, block_size=64, seed=13,
                                                        name="cacheless_block_causal"),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(CASES))
def test_client_runs_workloads(case, tmp_path):
    """The C program's outputs match the oracle within the parity tolerances."""
    w = CASES[case]()
    exe = build_client.build()
    q_rows = _write_workload(w, tmp_path)
    log(f"[c_client] {case}: {w.batch_size} requests, dtype {w.dtype}")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    shape = (q_rows, w.num_qo_heads, w.head_dim)
    if w.dtype == "bf16":
        out = synth.bf16_bits_to_f32(np.fromfile(tmp_path / "out.bin", dtype=np.uint16)).reshape(shape)
    else:
        out = np.fromfile(tmp_path / "out.bin", dtype=np.float32).reshape(shape)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(q_rows, w.num_qo_heads)
    ro, rl = ref.run_workload(w)
    tol_o, tol_l = TOL[w.dtype]
    err_o = float(np.max(np.abs(out.astype(np.float64) - ro)))
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    err_l = float(np.max(np.abs(lse[fin].astype(np.float64) - rl[fin]))) if fin.any() else 0.0
    log(f"[c_client] {case}: max|dout|={err_o:.2e} max|dlse|={err_l:.2e}")
    assert err_o <= tol_o and err_l <= tol_l
