"""Host-side checks of the C ABI library that need no GPU.

The library must load and export every function include/adam_mi355x.h
declares; adam_state_bytes is a pure host function checked against its
closed form and the memory claims of the 8-bit Adam page (about 2 bytes per
parameter plus a small scale overhead, about 4x below fp32 moments) and the
BF16-Adam page (half of fp32 moment state); argument errors must come back
before any HIP call.  No compute call is made here.
"""
import ctypes
import os
import re

import pytest

import memory_efficient_adam_amd as ma
from memory_efficient_adam_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adam_mi355x.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(adam_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"adam_state_bytes", "adam_state_create", "adam_step"} <= set(names)
    lib = ctypes.CDLL(ma.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_abi_structs_match_the_header_sizes():
    assert ctypes.sizeof(B.adam_layout) == 12
    assert ctypes.sizeof(B.adam_hparams) == 48
    assert B.adam_hparams.t.offset == 24 and B.adam_hparams.seed.offset == 40


def _pad16(n):
    return (n + 15) // 16 * 16


@pytest.mark.parametrize("storage,e,s", [("bf16", 4, 0), ("q8", 2, 8), ("q8_v_only", 5, 4)])
def test_state_bytes_closed_form(storage, e, s):
    numels = [1, 17, 2048, 2049, 6001, 0, 1048576]
    want = sum(_pad16(n) * e + -(-n // 2048) * s for n in numels)
    assert ma.adam_state_bytes(numels, storage, "f32") == want
    assert ma.adam_state_bytes([], storage, "bf16") == 0


def test_state_bytes_matches_the_pages_memory_claims():
    import workloads
    numels = workloads.numels_of(workloads.vit_base_shapes())
    n = sum(numels)
    fp32_moments = 8 * n
    q8 = ma.adam_state_bytes(numels, "q8")
    bf16 = ma.adam_state_bytes(numels, "bf16")
    # ~2 bytes per parameter plus a small overhead for the scales
    assert 2.0 <= q8 / n <= 2.01
    # ~4x smaller than two fp32 moments
    assert 3.9 <= fp32_moments / q8 <= 4.0
    # bf16 moments: half of the fp32 moment state
    assert abs(bf16 / fp32_moments - 0.5) < 1e-3


def test_state_bytes_rejects_bad_arguments():
    with pytest.raises(ma.AdamError) as e:
        ma.adam_state_bytes([-1], "q8")
    assert e.value.code == -1
    with pytest.raises(ma.AdamError):
        ma.adam_state_bytes([2 ** 32], "q8")
    with pytest.raises(ma.AdamError):
        ma.adam_state_bytes([5], 9)
    with pytest.raises(ma.AdamError) as e:
        ma.adam_state_bytes([5], "q8", block_size=1024)
    assert "block_size" in str(e.value)
    lib = ma.library()
    assert lib.adam_state_bytes(-1, None, None) == -1
    assert lib.adam_state_bytes(1, None, ctypes.byref(B._layout("q8", "f32"))) == -1


def test_create_rejects_bad_arguments_before_any_device_call():
    lib = ma.library()
    n, arr = B._numels([10])
    good = B._layout("q8", "f32")
    assert lib.adam_state_create(None, n, arr, ctypes.byref(good), None) == -1
    h = ctypes.c_void_p()
    assert lib.adam_state_create(ctypes.byref(h), n, arr, None, None) == -1
    assert lib.adam_state_create(ctypes.byref(h), -3, arr, ctypes.byref(good), None) == -1
    bad = B._layout("q8", "f32", 4096)
    assert lib.adam_state_create(ctypes.byref(h), n, arr, ctypes.byref(bad), None) == -1
    assert "block_size" in ma.adam_last_error()
    bad = B._layout("q8", 7)
    assert lib.adam_state_create(ctypes.byref(h), n, arr, ctypes.byref(bad), None) == -1
    assert h.value is None


def test_step_and_buffer_calls_reject_null_state():
    lib = ma.library()
    hp = B.adam_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 100.0, 1, 1, 0, 0)
    lay = B._layout("q8", "f32")
    assert lib.adam_step(None, None, None, ctypes.byref(hp), ctypes.byref(lay), None) == -1
    assert lib.adam_state_buffer_bytes(None, 0) == -1
    assert lib.adam_state_read(None, 0, None, 0, None) == -1
    assert lib.adam_state_write(None, 0, None, 0, None) == -1
    lib.adam_state_destroy(None)
    assert "NULL" in ma.adam_last_error()
