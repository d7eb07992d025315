"""CPU checks of the C ABI: the built library loads and exports every
function include/mla.h declares; calls that need no GPU behave."""

import ctypes
import os
import re

import numpy as np
import pytest

from paged_mla_attention_amd import _native
from paged_mla_attention_amd.build import build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s+(mla_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        build_library()
    return ctypes.CDLL(_native.LIB_PATH)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("mla_plan_create", "mla_plan", "mla_run", "mla_merge_state", "mla_plan_destroy",
              "mla_status_str", "mla_last_error"):
        assert n in names
    assert set(names) == set(_native.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_host_only_calls_work_without_gpu(lib):
    l2 = _native.load(_native.LIB_PATH)
    assert l2.mla_status_str(2) == b"unsupported shape"
    import paged_mla_attention_amd as pm
    s = pm.schedule([0, 1], [0, 2], [0, 1], [3], 4, 2, 16, 8, lib_path=_native.LIB_PATH)
    assert s["items"].shape[0] >= 1


def test_plan_create_rejects_shapes_before_touching_the_device(lib):
    l2 = _native.load(_native.LIB_PATH)
    h = ctypes.c_void_p()
    assert l2.mla_plan_create(ctypes.byref(h), 0, 16, 256, 64, 16) == 2
    assert b"kv_lora_rank" in l2.mla_last_error()
    assert l2.mla_plan_create(None, 0, 16, 512, 64, 16) == 1
    # NULL plan handles are rejected, not dereferenced
    assert l2.mla_run(None, None, None, None, None, None, None) == 1
    assert l2.mla_plan_stats(None, None, None, None, None) == 1
    l2.mla_plan_destroy(None)


def test_merge_state_argument_checks(lib):
    l2 = _native.load(_native.LIB_PATH)
    assert l2.mla_merge_state(None, None, None, None, None, None, 0, 16, None) == 0  # no work
    assert l2.mla_merge_state(None, None, None, None, None, None, 5, 16, None) == 1
    assert l2.mla_merge_state(None, None, None, None, None, None, -1, 16, None) == 1


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        _native.load(str(tmp_path / "missing.so"))
    assert np.int32(0) == 0


def test_noalloc_host_checks_before_touching_the_device(lib):
    """mla_run_noalloc rejects bad scalars on the host, before its first HIP
    call: a cache of more than 2^31 rows (the kernels address rows in 32
    bits) and too many heads."""
    l2 = _native.load(_native.LIB_PATH)
    args = [None] * 4 + [1, 1, 1, 1, 0.1, (1 << 29) + 1, 64, 16, 4] + [None] * 6
    assert l2.mla_run_noalloc(*args) == 2
    assert b"2^31 cache rows" in l2.mla_last_error()
    args[9], args[11] = 8, 129
    assert l2.mla_run_noalloc(*args) == 2
    assert b"num_heads" in l2.mla_last_error()
