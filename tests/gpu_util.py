"""Helpers for GPU tests: upload a synthetic workload, run it through the C ABI, compare."""
from __future__ import annotations

import contextlib
import os
import sys

import numpy as np

import ragged_attention_serving_amd as xa

TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-3)}  # (max |out| error, max |lse| error)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arr, dtype, device):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def from_device(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


@contextlib.contextmanager
def forced_chunk(n):
    old = os.environ.get("XATTN_FORCE_CHUNK")
    if n:
        os.environ["XATTN_FORCE_CHUNK"] = str(n)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("XATTN_FORCE_CHUNK", None)
        else:
            os.environ["XATTN_FORCE_CHUNK"] = old


def plan_for(w, plan=None, chunk=0):
    plan = plan or xa.Plan()
    with forced_chunk(chunk):
        plan.plan(w.qo_indptr, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, w.num_qo_heads,
                  w.num_kv_heads, w.head_dim, w.page_size, max(w.num_pages, 1), w.mask_mode,
                  w.block_size, w.sm_scale, w.dtype)
    return plan


def run_gpu(w, device, chunk=0, tensors=None, plan=None, want_lse=True):
    """Plans and runs w on the GPU; returns (out fp64, lse fp64 or None, plan)."""
    import torch
    q, k, v = tensors if tensors is not None else (to_device(w.q, w.dtype, device),
                                                   to_device(w.k_pages, w.dtype, device),
                                                   to_device(w.v_pages, w.dtype, device))
    plan = plan_for(w, plan, chunk)
    out, lse = plan.run(q, k, v, want_lse=want_lse)
    torch.cuda.synchronize()
    return from_device(out), (lse.cpu().numpy().astype(np.float64) if lse is not None else None), plan


def compare(out, lse, ref_out, ref_lse, dtype, rows=None, label="", tol=None):
    """Asserts parity within the dtype's tolerance (or ``tol`` = (out, lse) where a test
    derives its own) on the given rows (all if None)."""
    tol_o, tol_l = TOL[dtype] if tol is None else tol
    if rows is not None:
        out, lse, ref_out, ref_lse = out[rows], lse[rows], ref_out[rows], ref_lse[rows]
    assert not np.isnan(out).any(), f"{label}: NaN in out"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{label}: -inf rows differ"
    assert np.all(out[~fin] == 0), f"{label}: rows with no key must be 0"
    err_o = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    scale = float(np.max(np.abs(ref_out))) if out.size else 0.0
    rms = float(np.sqrt(np.mean((out - ref_out) ** 2))) if out.size else 0.0
    log(f"  {label}: max|dout|={err_o:.3e} (rel {err_o / max(scale, 1e-30):.2e}, rms {rms:.2e}) "
        f"max|dlse|={err_l:.3e}")
    assert err_o <= tol_o, f"{label}: out error {err_o} > {tol_o}"
    assert err_l <= tol_l, f"{label}: lse error {err_l} > {tol_l}"
    return err_o, err_l
