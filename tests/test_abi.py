"""The C-ABI library, on the CPU: it loads, exports every entry point the
header declares, and rejects bad configurations before touching the GPU."""
import ctypes
import os
import re

import pytest

from paged_kv_gqa_qwen3_amd import binding, build, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "qd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.QD_LIB):
        build.build_qd()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _cfg(**kw):
    c = binding.make_config(synth.TINY, 4, 8, 64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code", [
    ("page_size", 32, binding.QD_EUNSUPPORTED),
    ("head_dim", 96, binding.QD_EUNSUPPORTED),
    ("num_kv_heads", 3, binding.QD_EUNSUPPORTED),
    ("hidden", 200, binding.QD_EUNSUPPORTED),
    ("vocab", 4000, binding.QD_EUNSUPPORTED),
    ("intermediate", 700, binding.QD_EUNSUPPORTED),
    ("max_batch", 0, binding.QD_EINVAL),
    ("max_batch", 65, binding.QD_EINVAL),
    ("num_pages", 0, binding.QD_EINVAL),
    ("rms_eps", 0.0, binding.QD_EINVAL),
    ("num_layers", 0, binding.QD_EINVAL),
    ("hidden", 8256, binding.QD_EUNSUPPORTED),
    ("max_pages_per_seq", 4097, binding.QD_EUNSUPPORTED),
    ("max_prefill_rows", -1, binding.QD_EINVAL),
    ("max_prefill_rows", 16385, binding.QD_EINVAL),
    ("kv_dtype", 2, binding.QD_EINVAL),
])
def test_create_rejects_bad_config(lib, field, value, code):
    h = ctypes.c_void_p()
    cfg = _cfg(**{field: value})
    rc = lib.qd_create(ctypes.byref(cfg), None, ctypes.byref(h))
    assert rc == code
    assert h.value is None
    assert binding.qd_last_error(None) != ""


@pytest.mark.parametrize("k,v", [(0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0),
                                 (1.0, float("nan"))])
def test_create_rejects_bad_fp8_scales(lib, k, v):
    h = ctypes.c_void_p()
    cfg = _cfg(kv_dtype=1, k_scale=k, v_scale=v)
    assert lib.qd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == binding.QD_EINVAL
    assert h.value is None


def test_null_arguments(lib):
    assert lib.qd_create(None, None, None) == binding.QD_EINVAL
    h = ctypes.c_void_p()
    assert lib.qd_create(None, None, ctypes.byref(h)) == binding.QD_EINVAL
    assert lib.qd_decode_step(None, 1, None, None, None, None, None, None) == binding.QD_EINVAL
    assert lib.qd_load_weights(None, None, 0) == binding.QD_EINVAL
    assert lib.qd_sample(None, 1, None, None, None, None, None, None) == binding.QD_EINVAL
    assert lib.qd_prefill(None, 1, None, None, None, None, 0, None, None) == binding.QD_EINVAL
    assert lib.qd_prefill_prompts(None, 1, None, None, None, None, None, 0, None,
                                  None) == binding.QD_EINVAL
    lib.qd_destroy(None)
    e = ctypes.c_void_p()
    assert lib.qd_engine_create(None, None, ctypes.byref(e)) == binding.QD_EINVAL
    assert lib.qd_engine_submit(None, None) == binding.QD_EINVAL
    n = ctypes.c_int32()
    assert lib.qd_engine_step(None, 64, None, None, None, ctypes.byref(n)) == binding.QD_EINVAL
    assert lib.qd_engine_get_stats(None, None) == binding.QD_EINVAL
    lib.qd_engine_destroy(None)
