"""The C ABI: the library loads, exports what include/xattn.h declares, and rejects bad
arguments on the host before any GPU call (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

import ragged_attention_serving_amd as xa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "xattn.h")).read()
    return re.findall(r"XATTN_API\s+[\w\s\*]+?\b(xattn_\w+)\s*\(", text)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(xa.EXPORTED), names
    L = xa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_library_is_gfx950_code():
    out = open(xa.LIB_PATH, "rb").read()
    assert b"gfx950" in out


def _sched(**kw):
    base = dict(qo_indptr=[0, 1, 3], kv_indptr=[0, 2, 5], kv_page_indices=[4, 0, 1, 2, 3],
                kv_last_page_len=[3, 2], num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=4,
                num_pages=5, mask_mode=0, block_size=0, dtype="bf16")
    base.update(kw)
    return xa.xattn_schedule(**base)


def test_valid_schedule():
    info, units, merges = _sched()
    assert info["total_kv_tokens"] == (1 * 4 + 3) + (2 * 4 + 2)


@pytest.mark.parametrize("kw,code", [
    (dict(qo_indptr=[1, 1, 3]), xa.XATTN_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 3, 1]), xa.XATTN_ERR_INVALID_ARG),
    (dict(kv_indptr=[0, 3, 2]), xa.XATTN_ERR_INVALID_ARG),
    (dict(kv_last_page_len=[0, 2]), xa.XATTN_ERR_INVALID_ARG),
    (dict(kv_last_page_len=[5, 2]), xa.XATTN_ERR_INVALID_ARG),
    (dict(num_qo_heads=3), xa.XATTN_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), xa.XATTN_ERR_INVALID_ARG),
    (dict(head_dim=96), xa.XATTN_ERR_UNSUPPORTED),
    (dict(head_dim=16), xa.XATTN_ERR_UNSUPPORTED),
    (dict(page_size=0), xa.XATTN_ERR_INVALID_ARG),
    (dict(mask_mode=3), xa.XATTN_ERR_INVALID_ARG),
    (dict(mask_mode=2, block_size=0), xa.XATTN_ERR_INVALID_ARG),
    (dict(kv_page_indices=[4, 0, 1, 2, 5]), xa.XATTN_ERR_INVALID_ARG),
    (dict(kv_page_indices=[4, 0, -1, 2, 3]), xa.XATTN_ERR_INVALID_ARG),
    (dict(num_pages=0), xa.XATTN_ERR_INVALID_ARG),
    (dict(kv_page_indices=None, num_pages=4), xa.XATTN_ERR_INVALID_ARG),
    (dict(qo_indptr=[0, 1, 13], mask_mode=1), xa.XATTN_ERR_INVALID_ARG),  # causal qo > kv
    (dict(dtype=7), None),
])
def test_rejects(kw, code):
    if code is None:
        with pytest.raises(ValueError):
            _sched(**kw)
        return
    with pytest.raises(xa.XattnError) as e:
        _sched(**kw)
    assert e.value.code == code
    assert xa.xattn_last_error()


def test_fp32_head_dims():
    for d in (16, 32, 64, 128):
        _sched(head_dim=d, dtype="f32")
    with pytest.raises(xa.XattnError):
        _sched(head_dim=8, dtype="f32")


def test_plan_validates_before_touching_the_device():
    """An invalid plan fails in host validation: no handle is created."""
    h = ctypes.c_void_p()
    with pytest.raises(xa.XattnError) as e:
        xa.xattn_plan(h, [0, 1], [0, 1], [0], [9], 2, 2, 64, 4, 1, stream=0)
    assert e.value.code == xa.XATTN_ERR_INVALID_ARG and not h.value
    assert "kv_last_page_len" in xa.xattn_last_error()


def test_run_without_plan_is_rejected():
    rc = xa.lib().xattn_run(None, None, None, None, None, None, None)
    assert rc == xa.XATTN_ERR_INVALID_ARG


def test_destroy_null_is_a_no_op():
    xa.lib().xattn_plan_destroy(None)


def test_binding_raises_without_the_library():
    """No fallback: without libxattn.so every entry point of the binding raises."""
    import subprocess
    import sys
    code = (
        "import ragged_attention_serving_amd as xa\n"
        "xa.LIB_PATH = '/nonexistent/libxattn.so'\n"
        "xa._lib = None\n"
        "import numpy as np\n"
        "for call in (lambda: xa.lib(), lambda: xa.Plan().plan(np.array([0, 1], np.int32), np.array([0, 1], np.int32),"
        " None, None, 1, 1, 64, 16, 1)):\n"
        "    try:\n"
        "        call()\n"
        "    except RuntimeError as e:\n"
        "        assert 'missing' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('no error')\n"
        "print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0 and "raised" in r.stdout, r.stderr[-2000:]


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=root)
    assert r.returncode == 2 and "one GPU only" in r.stderr, (r.returncode, r.stderr[-2000:])


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), 3e38])
def test_plan_rejects_a_scale_that_is_not_finite(scale):
    h = ctypes.c_void_p()
    with pytest.raises(xa.XattnError) as e:
        xa.xattn_plan(h, [0, 1], [0, 1], [0], [4], 2, 2, 64, 4, 1, sm_scale=scale, stream=0)
    assert e.value.code == xa.XATTN_ERR_INVALID_ARG and not h.value
    assert "sm_scale" in xa.xattn_last_error()
