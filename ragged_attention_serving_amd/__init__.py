"""libxattn: plan/run paged attention on AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI in include/xattn.h: the functions below carry
the C entry points' names and only marshal arguments. Every step of the attention
runs in the library's HIP kernels; there is no fallback. PyTorch is used for device
memory and streams only.

    from ragged_attention_serving_amd import Plan
    plan = Plan()
    plan.plan(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len,
              num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, mask_mode=MASK_NONE)
    out, lse = plan.run(q, k_pages, v_pages)   # once per layer
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BLOCK_CAUSAL = 2
F32 = 0
BF16 = 1

XATTN_OK = 0
XATTN_ERR_INVALID_ARG = -1
XATTN_ERR_UNSUPPORTED = -2
XATTN_ERR_HIP = -3
XATTN_ERR_OOM = -4
XATTN_ERR_BUSY = -5

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxattn.so")
EXPORTED = ("xattn_plan_create", "xattn_plan", "xattn_run", "xattn_run_noalloc", "xattn_write_kv", "xattn_plan_ready", "xattn_plan_destroy",
            "xattn_last_error", "xattn_schedule", "xattn_plan_info", "xattn_plan_set_timing",
            "xattn_plan_timing")
STAGES = ("fp32", "decode", "mfma", "merge")

_lib = None


class XattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libxattn error {code}: {msg}")
        self.code = code


class ScheduleInfo(ctypes.Structure):
    _fields_ = [("num_units", ctypes.c_int32 * 3), ("chunk_tokens", ctypes.c_int32 * 3),
                ("decode_rows", ctypes.c_int32), ("num_merge_rows", ctypes.c_int32),
                ("workspace_rows", ctypes.c_int64), ("total_kv_tokens", ctypes.c_int64),
                ("visible_pairs", ctypes.c_int64), ("layout_generation", ctypes.c_int64),
                ("slot", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {"num_units": list(self.num_units), "chunk_tokens": list(self.chunk_tokens),
                "decode_rows": self.decode_rows, "num_merge_rows": self.num_merge_rows,
                "workspace_rows": self.workspace_rows, "total_kv_tokens": self.total_kv_tokens,
                "visible_pairs": self.visible_pairs, "layout_generation": self.layout_generation,
                "slot": self.slot}


def lib() -> ctypes.CDLL:
    """The loaded libxattn.so. Raises if it was not built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m ragged_attention_serving_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    P32 = ctypes.POINTER(ctypes.c_int32)
    L.xattn_plan.argtypes = [ctypes.POINTER(vp), P32, P32, P32, P32, i32, i32, i32, i32, i32, i64,
                             i32, i32, f32, i32, vp]
    L.xattn_plan.restype = ctypes.c_int
    L.xattn_plan_create.argtypes = [ctypes.POINTER(vp), i32]
    L.xattn_plan_create.restype = ctypes.c_int
    L.xattn_run.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.xattn_run.restype = ctypes.c_int
    L.xattn_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.xattn_run_noalloc.restype = ctypes.c_int
    L.xattn_write_kv.argtypes = [vp, vp, vp, vp, vp, vp]
    L.xattn_write_kv.restype = ctypes.c_int
    L.xattn_plan_ready.argtypes = [vp]
    L.xattn_plan_ready.restype = ctypes.c_int
    L.xattn_plan_destroy.argtypes = [vp]
    L.xattn_plan_destroy.restype = None
    L.xattn_last_error.argtypes = []
    L.xattn_last_error.restype = ctypes.c_char_p
    L.xattn_schedule.argtypes = [P32, P32, P32, P32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i32,
                                 ctypes.POINTER(ScheduleInfo), P32, P32]
    L.xattn_schedule.restype = ctypes.c_int
    L.xattn_plan_info.argtypes = [vp, ctypes.POINTER(ScheduleInfo)]
    L.xattn_plan_info.restype = ctypes.c_int
    L.xattn_plan_set_timing.argtypes = [vp, ctypes.c_int]
    L.xattn_plan_set_timing.restype = ctypes.c_int
    L.xattn_plan_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_double), P32]
    L.xattn_plan_timing.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> int:
    if rc < 0:
        raise XattnError(rc, xattn_last_error())
    return rc


def _i32(a):
    """Host int32 array (contiguous) and its ctypes pointer; None stays NULL."""
    if a is None:
        return None, None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _dtype_code(dtype) -> int:
    if dtype in (F32, "f32", "float32"):
        return F32
    if dtype in (BF16, "bf16", "bfloat16"):
        return BF16
    s = str(dtype)
    if s.endswith("float32"):
        return F32
    if s.endswith("bfloat16"):
        return BF16
    raise ValueError(f"unsupported dtype {dtype}")


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


# ------------------------------------------------------------------ C entry points

def xattn_last_error() -> str:
    return lib().xattn_last_error().decode()


def xattn_schedule(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
                   num_kv_heads, head_dim, page_size, num_pages, mask_mode=MASK_NONE, block_size=0,
                   dtype=BF16, force_chunk=0, want_units=True):
    """Host-only schedule: (info dict, units [n][8] int32, merges [m][4] int32)."""
    L = lib()
    qo, qo_p = _i32(qo_indptr)
    kv, kv_p = _i32(kv_indptr)
    pi, pi_p = _i32(kv_page_indices)
    lp, lp_p = _i32(kv_last_page_len)
    b = len(qo) - 1
    info = ScheduleInfo()
    _check(L.xattn_schedule(qo_p, kv_p, pi_p, lp_p, b, num_qo_heads, num_kv_heads, head_dim, page_size,
                            int(num_pages), mask_mode, block_size, _dtype_code(dtype), force_chunk,
                            ctypes.byref(info), None, None))
    units = merges = None
    if want_units:
        n = sum(info.num_units)
        units = np.zeros((max(n, 1), 8), np.int32)
        merges = np.zeros((max(info.num_merge_rows, 1), 4), np.int32)
        _check(L.xattn_schedule(qo_p, kv_p, pi_p, lp_p, b, num_qo_heads, num_kv_heads, head_dim,
                                page_size, int(num_pages), mask_mode, block_size, _dtype_code(dtype),
                                force_chunk, ctypes.byref(info),
                                units.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                merges.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        units, merges = units[:n], merges[:info.num_merge_rows]
    return info.as_dict(), units, merges


def xattn_plan(handle, qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
               num_kv_heads, head_dim, page_size, num_pages, mask_mode=MASK_NONE, block_size=0,
               sm_scale=0.0, dtype=BF16, stream=None):
    """Plans into `handle` (a ctypes.c_void_p; its value None creates one). Returns it."""
    L = lib()
    qo, qo_p = _i32(qo_indptr)
    kv, kv_p = _i32(kv_indptr)
    pi, pi_p = _i32(kv_page_indices)
    lp, lp_p = _i32(kv_last_page_len)
    if handle is None:
        handle = ctypes.c_void_p()
    _check(L.xattn_plan(ctypes.byref(handle), qo_p, kv_p, pi_p, lp_p, len(qo) - 1, num_qo_heads,
                        num_kv_heads, head_dim, page_size, int(num_pages), mask_mode, block_size,
                        float(sm_scale), _dtype_code(dtype), _stream_handle(stream)))
    return handle


def xattn_run(handle, q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, lse_ptr: int | None,
              stream=None) -> None:
    """Raw run on device pointers (ints)."""
    _check(lib().xattn_run(handle, q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr or None, _stream_handle(stream)))


def xattn_run_noalloc(handle, q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, lse_ptr: int | None,
                      stream=None) -> None:
    """Raw allocation-free run on device pointers (ints): the split workspace is the
    library's static device scratch."""
    _check(lib().xattn_run_noalloc(handle, q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr or None,
                                   _stream_handle(stream)))


PLAN_GRAPH_STABLE = 1


def xattn_plan_create(handle, flags: int = 0) -> None:
    """Creates an empty handle in `handle` (a ctypes.c_void_p holding NULL) with flags."""
    _check(lib().xattn_plan_create(ctypes.byref(handle), flags))


def xattn_write_kv(handle, k_src_ptr: int, v_src_ptr: int, k_pages_ptr: int, v_pages_ptr: int,
                   stream=None) -> None:
    """Raw context write on device pointers (ints)."""
    _check(lib().xattn_write_kv(handle, k_src_ptr, v_src_ptr, k_pages_ptr, v_pages_ptr,
                                _stream_handle(stream)))


def xattn_plan_ready(handle) -> bool:
    return bool(_check(lib().xattn_plan_ready(handle)))


def xattn_plan_info(handle) -> dict:
    info = ScheduleInfo()
    _check(lib().xattn_plan_info(handle, ctypes.byref(info)))
    return info.as_dict()


def xattn_plan_set_timing(handle, every: int) -> None:
    """Record kernel events on every `every`-th run (0 or False: off, True: every run)."""
    _check(lib().xattn_plan_set_timing(handle, int(every)))


def xattn_plan_timing(handle) -> dict:
    """{stage: (total ms, launches)} for the runs recorded since the last call."""
    ms = (ctypes.c_double * 4)()
    n = (ctypes.c_int32 * 4)()
    _check(lib().xattn_plan_timing(handle, ms, n))
    return {STAGES[i]: (float(ms[i]), int(n[i])) for i in range(4)}


def xattn_plan_destroy(handle) -> None:
    if handle is not None and handle.value:
        lib().xattn_plan_destroy(handle)
        handle.value = None


# ------------------------------------------------------------------ torch-facing wrapper

class Plan:
    """One attention handle: plan once per step, run once per layer."""

    def __init__(self, graph_stable: bool = False):
        """graph_stable: lay each slot out for HIP-graph replay across plans
        (XATTN_PLAN_GRAPH_STABLE; see xattn_plan_create)."""
        lib()
        self._h = ctypes.c_void_p()
        self.meta = None
        if graph_stable:
            xattn_plan_create(self._h, PLAN_GRAPH_STABLE)

    def plan(self, qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
             num_kv_heads, head_dim, page_size, num_pages, mask_mode=MASK_NONE, block_size=0,
             sm_scale=0.0, dtype="bf16", stream=None) -> "Plan":
        xattn_plan(self._h, qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
                   num_kv_heads, head_dim, page_size, num_pages, mask_mode, block_size, sm_scale,
                   dtype, stream)
        total_q = int(np.asarray(qo_indptr)[-1]) if len(qo_indptr) else 0
        self.meta = dict(total_q=total_q, hq=num_qo_heads, hkv=num_kv_heads, d=head_dim,
                         page_size=page_size, num_pages=int(num_pages), dtype=_dtype_code(dtype),
                         total_kv=int(xattn_plan_info(self._h)["total_kv_tokens"]))
        return self

    def run(self, q, k_pages, v_pages, out=None, lse=None, stream=None, want_lse=True):
        """Attention for one layer. q/k_pages/v_pages are CUDA tensors of the planned dtype."""
        import torch
        if self.meta is None:
            raise XattnError(XATTN_ERR_INVALID_ARG, "run before plan")
        m = self.meta
        tdt = torch.float32 if m["dtype"] == F32 else torch.bfloat16
        for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous CUDA {tdt} tensor")
        if tuple(q.shape) != (m["total_q"], m["hq"], m["d"]):
            raise ValueError(f"q has shape {tuple(q.shape)}, expected {(m['total_q'], m['hq'], m['d'])}")
        pool = (m["num_pages"], m["page_size"], m["hkv"], m["d"])
        for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
            if t.numel() != int(np.prod(pool)) or t.shape[-1] != m["d"]:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {pool}")
        if out is None:
            out = torch.empty_like(q)
        elif out.shape != q.shape or out.dtype != tdt or not out.is_contiguous():
            raise ValueError("out must match q")
        if lse is None and want_lse:
            lse = torch.empty((m["total_q"], m["hq"]), dtype=torch.float32, device=q.device)
        xattn_run(self._h, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                  lse.data_ptr() if lse is not None else None, stream)
        return out, lse

    def run_noalloc(self, q, k_pages, v_pages, out, lse=None, stream=None):
        """Attention for one layer through xattn_run_noalloc: the caller passes out (and lse,
        or None for no lse); nothing is allocated, the split workspace is the library's
        static device scratch. Runs on the stream of the latest plan only."""
        if self.meta is None:
            raise XattnError(XATTN_ERR_INVALID_ARG, "run before plan")
        self._check_run_tensors(q, k_pages, v_pages, out, lse)
        xattn_run_noalloc(self._h, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if lse is not None else None, stream)
        return out, lse

    def _check_run_tensors(self, q, k_pages, v_pages, out, lse):
        import torch
        m = self.meta
        tdt = torch.float32 if m["dtype"] == F32 else torch.bfloat16
        for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("out", out)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous CUDA {tdt} tensor")
        if tuple(q.shape) != (m["total_q"], m["hq"], m["d"]) or out.shape != q.shape:
            raise ValueError(f"q and out must have shape {(m['total_q'], m['hq'], m['d'])}")
        pool = (m["num_pages"], m["page_size"], m["hkv"], m["d"])
        for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
            if t.numel() != int(np.prod(pool)) or t.shape[-1] != m["d"]:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {pool}")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous()
                                or tuple(lse.shape) != (m["total_q"], m["hq"])):
            raise ValueError(f"lse must be a contiguous CUDA float32 tensor of shape {(m['total_q'], m['hq'])}")

    def write_kv(self, k_src, v_src, k_pages, v_pages, stream=None):
        """Writes the planned requests' packed context rows (k_src/v_src [sum kv_len, Hkv, D])
        into their page slots of k_pages/v_pages (CUDA tensors of the planned dtype)."""
        import torch
        if self.meta is None:
            raise XattnError(XATTN_ERR_INVALID_ARG, "write_kv before plan")
        m = self.meta
        tdt = torch.float32 if m["dtype"] == F32 else torch.bfloat16
        rows = m["total_kv"]
        for name, t in (("k_src", k_src), ("v_src", v_src), ("k_pages", k_pages), ("v_pages", v_pages)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous CUDA {tdt} tensor")
        for name, t in (("k_src", k_src), ("v_src", v_src)):
            if t.numel() != rows * m["hkv"] * m["d"]:
                raise ValueError(f"{name} has {t.numel()} elements, expected {rows} x {m['hkv']} x {m['d']}")
        pool = m["num_pages"] * m["page_size"] * m["hkv"] * m["d"]
        for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
            if t.numel() != pool:
                raise ValueError(f"{name} has {t.numel()} elements, expected {pool}")
        xattn_write_kv(self._h, k_src.data_ptr(), v_src.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                       stream)

    def ready(self) -> bool:
        return xattn_plan_ready(self._h)

    def info(self) -> dict:
        return xattn_plan_info(self._h)

    def set_timing(self, every: int = 1) -> None:
        xattn_plan_set_timing(self._h, every)

    def timing(self) -> dict:
        return xattn_plan_timing(self._h)

    @property
    def handle(self):
        return self._h

    def close(self) -> None:
        if self._h is not None and self._h.value:
            xattn_plan_destroy(self._h)

    def __del__(self):  # pragma: no cover - interpreter shutdown order varies
        try:
            self.close()
        except Exception:
            pass
