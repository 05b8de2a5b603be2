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
    assert ctypes.sizeof(B.adam_layout) == 16 and B.adam_layout.options.offset == 12
    assert ctypes.sizeof(B.adam_hparams) == 48
    assert B.adam_hparams.t.offset == 24 and B.adam_hparams.seed.offset == 40


def _pad16(n):
    return (n + 15) // 16 * 16


@pytest.mark.parametrize("storage,e,s,ae,as_", [("bf16", 4, 0, 2, 0), ("q8", 2, 8, 1, 4),
                                                ("q8_v_only", 5, 4, 1, 4)])
def test_state_bytes_closed_form(storage, e, s, ae, as_):
    numels = [1, 17, 2048, 2049, 6001, 0, 1048576]
    want = sum(_pad16(n) * e + -(-n // 2048) * s for n in numels)
    assert ma.adam_state_bytes(numels, storage, "f32") == want
    assert ma.adam_state_bytes([], storage, "bf16") == 0
    # AMSGrad: the running maximum of v stored as v is
    extra = sum(_pad16(n) * ae + -(-n // 2048) * as_ for n in numels)
    assert ma.adam_state_bytes(numels, storage, "f32", amsgrad=True) == want + extra


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
    n, arr = B._numels([5])
    assert lib.adam_state_bytes(n, arr, ctypes.byref(B._layout("q8", "f32", 2048, 2))) == -1
    assert "option" in ma.adam_last_error()


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


def test_create_rejects_an_oversized_state_before_building_it():
    # 17 tensors of 2^32 - 1 elements pass the per-tensor limit but exceed
    # 2^36 padded state entries in total: refused up front (no host tables
    # built, no device call)
    lib = ma.library()
    n, arr = B._numels([2 ** 32 - 1] * 17)
    h = ctypes.c_void_p()
    lay = B._layout("q8", "bf16")
    assert lib.adam_state_create(ctypes.byref(h), n, arr, ctypes.byref(lay), None) == -1
    assert "too large" in ma.adam_last_error() and h.value is None


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


# ---------------------------------------------------------------- checkpoint stream
def _stream_hash(b):
    # the stream's 64-bit multiply-xor checksum (format definition in the header)
    n = len(b)
    h = (0x9E3779B97F4A7C15 ^ n) & 0xFFFFFFFFFFFFFFFF
    i = 0
    while i + 8 <= n:
        w = int.from_bytes(b[i:i + 8], "little")
        h = ((h ^ w) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
        i += 8
    while i < n:
        h = ((h ^ b[i]) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
        i += 1
    return h ^ (h >> 32)


def _serialized(numels, storage=2, records=None, version=2, options=0, pad_word=0, draw=None):
    import struct
    pad16 = [(n + 15) // 16 * 16 for n in numels]
    blocks = sum(-(-n // 2048) for n in numels)
    if draw is None:  # default draw indices: the segment starts
        draw = [sum(pad16[:k]) for k in range(len(numels))]
    out = bytearray(b"MEAMSTAT")
    out += struct.pack("<IIiiiIiI", version, 40 + 16 * len(numels), storage, 0, 2048, options,
                       len(numels), pad_word)
    out += struct.pack(f"<{len(numels)}q", *numels)
    out += struct.pack(f"<{len(numels)}q", *draw)
    if records is None:
        P = sum(pad16)
        records = {2: [(0, P), (1, P), (2, 4 * blocks), (3, 4 * blocks)],
                   1: [(4, 2 * P), (5, 2 * P)], 3: [(1, P), (3, 4 * blocks), (6, 4 * P)]}[storage]
        if options & 1:
            records += [(9, 2 * P)] if storage == 1 else [(7, P), (8, 4 * blocks)]
    for bid, nb in records:
        out += struct.pack("<IIQ", bid, 0, nb) + bytes((nb + 7) // 8 * 8)
    out += struct.pack("<II", 0xFFFFFFFF, len(records))
    out += struct.pack("<Q", _stream_hash(bytes(out)))
    return bytes(out)


def _load_rc(buf):
    lib = ma.library()
    h = ctypes.c_void_p()
    arr = (ctypes.c_uint8 * len(buf)).from_buffer_copy(buf)
    rc = lib.adam_state_load(ctypes.byref(h), ctypes.cast(arr, ctypes.c_void_p), len(buf), None)
    return rc, h.value


@pytest.mark.parametrize("mutate", ["magic", "version", "truncate", "checksum", "payload",
                                    "record_order", "record_size", "storage", "numel",
                                    "options", "header_word", "amsgrad_records",
                                    "draw_unaligned", "draw_negative", "draw_too_large"])
def test_load_rejects_malformed_streams_before_any_device_call(mutate):
    import struct
    numels = [5000, 17]
    good = bytearray(_serialized(numels))
    if mutate == "magic":
        bad = b"XEAMSTAT" + bytes(good[8:])
    elif mutate == "version":
        bad = _serialized(numels, version=1)
    elif mutate == "options":
        bad = _serialized(numels, options=2)
    elif mutate == "header_word":
        bad = _serialized(numels, pad_word=1)
    elif mutate == "draw_unaligned":
        bad = _serialized(numels, draw=[0, 5016])
    elif mutate == "draw_negative":
        bad = _serialized(numels, draw=[-16, 5008])
    elif mutate == "draw_too_large":
        bad = _serialized(numels, draw=[0, 2 ** 62 - 16])
    elif mutate == "amsgrad_records":
        # claims the AMSGrad option but holds only the plain buffers
        P = 5008 + 32
        bad = _serialized(numels, options=1, records=[(0, P), (1, P), (2, 16), (3, 16)])
    elif mutate == "truncate":
        bad = bytes(good[:-24])
    elif mutate == "checksum":
        good[-1] ^= 0x40
        bad = bytes(good)
    elif mutate == "payload":
        good[96] ^= 1  # inside the first record's bytes, checksum now stale
        bad = bytes(good)
    elif mutate == "record_order":
        P = 5008 + 32
        bad = _serialized(numels, records=[(1, P), (0, P), (2, 16), (3, 16)])
    elif mutate == "record_size":
        P = 5008 + 32
        bad = _serialized(numels, records=[(0, P), (1, P - 16), (2, 16), (3, 16)])
    elif mutate == "storage":
        bad = bytearray(good)
        bad[16:20] = struct.pack("<i", 1)  # claims bf16 but holds 8-bit records
        bad = bytes(bad[:-8]) + struct.pack("<Q", _stream_hash(bytes(bad[:-8])))
    else:  # numel
        bad = bytearray(good)
        bad[40:48] = struct.pack("<q", -3)
        bad = bytes(bad[:-8]) + struct.pack("<Q", _stream_hash(bytes(bad[:-8])))
    rc, h = _load_rc(bytes(bad))
    assert rc == -1 and h is None, (mutate, ma.adam_last_error())


@pytest.mark.parametrize("storage,options,draw", [(2, 0, None), (1, 0, None), (3, 0, None),
                                                  (2, 1, None), (1, 1, None), (3, 1, [2 ** 40, 0])])
def test_load_of_a_valid_stream_gets_past_validation(storage, options, draw):
    # a well-formed stream passes every host check; on a machine without a GPU
    # the first device call (state creation) is what fails
    rc, h = _load_rc(_serialized([5000, 17], storage=storage, options=options, draw=draw))
    if rc == 0:
        ma.library().adam_state_destroy(h)
    else:
        assert rc in (-4, -5), ma.adam_last_error()


# ---------------------------------------------------------------- binding checks
# The torch-facing binding hands raw pointers to the kernel, which reads and
# writes numel elements through each; every tensor is checked before any
# library call (these run with no GPU and no library state).
def _fake_state(numels, grad_dtype=0):
    return B.AdamState(None, numels, B.adam_layout(2, grad_dtype, 2048, 0), device=0)


def test_step_rejects_bad_tensors_before_any_call():
    import torch
    st = _fake_state([100, 7])
    ok_p = [torch.zeros(100), torch.zeros(7)]
    ok_g = [torch.zeros(100), torch.zeros(7)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=1)
    bad_cases = [
        ([torch.zeros(100)], ok_g, "expected 2"),                                # count
        ([torch.zeros(99), torch.zeros(7)], ok_g, "numel"),                      # short param
        (ok_p, [torch.zeros(100), torch.zeros(8)], "numel"),                     # long grad
        ([torch.zeros(100, dtype=torch.float64), torch.zeros(7)], ok_g, "dtype"),
        (ok_p, [torch.zeros(100, dtype=torch.bfloat16), torch.zeros(7)], "dtype"),
        ([torch.zeros(200)[::2], torch.zeros(7)], ok_g, "contiguous"),           # strided view
        (ok_p, ok_g, "device"),                                                  # host tensors
    ]
    for params, grads, what in bad_cases:
        with pytest.raises(ValueError, match=what):
            ma.adam_step(st, params, grads, **hp)
    with pytest.raises(TypeError):
        ma.adam_step(st, [None, torch.zeros(7)], ok_g, **hp)
    # bf16 gradients for a bf16-gradient layout: fp32 ones are refused
    st16 = _fake_state([100], grad_dtype=1)
    with pytest.raises(ValueError, match="dtype"):
        ma.adam_step(st16, [torch.zeros(100)], [torch.zeros(100)], **hp)
    with pytest.raises(ValueError, match="device"):  # right dtype, still host memory
        ma.adam_step(st16, [torch.zeros(100)], [torch.zeros(100, dtype=torch.bfloat16)], **hp)
    # zero-size tensors carry no pointer the kernel uses
    st0 = _fake_state([0])
    with pytest.raises(ma.AdamError):  # reaches the library, which refuses a NULL state
        ma.adam_step(st0, [torch.zeros(0)], [torch.zeros(0)], stream=0, **hp)


def test_state_read_write_reject_wrong_sizes():
    import torch
    st = _fake_state([100])
    # buffer sizes come from the library: a NULL state fails there first, so
    # check the size rule through a stand-in that reports 112 bytes
    orig = B.adam_state_buffer_bytes
    B.adam_state_buffer_bytes = lambda state, which: 112
    try:
        with pytest.raises(ValueError, match="112 bytes"):
            ma.adam_state_read(st, "v_codes", out=torch.empty(100, dtype=torch.uint8))
        with pytest.raises(ValueError, match="112 bytes"):
            ma.adam_state_read(st, "v_codes", out=torch.empty(224, dtype=torch.uint8)[::2])
        with pytest.raises(ValueError, match="112 bytes"):
            ma.adam_state_write(st, "v_codes", torch.empty(111, dtype=torch.uint8))
    finally:
        B.adam_state_buffer_bytes = orig


def test_noalloc_limits_refused_before_any_device_call():
    # the allocation-free step's table space is fixed: 65536 tensors and 2^20
    # blocks; larger lists are refused with a message naming the limit, before
    # any HIP call (the pointers below are never dereferenced)
    lib = ma.library()
    lay = B.adam_layout(2, 0, 2048, 0)
    hp = B.adam_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 100.0, 1, 1, 0, 42)
    for numels, what in (([0] * 70000, b"65536"), ([2 ** 31 + 1], b"1048576")):
        n = len(numels)
        arr = (ctypes.c_int64 * n)(*numels)
        ptrs = (ctypes.c_void_p * n)(*([4096] * n))
        state = (ctypes.c_void_p * 10)(*([4096] * 10))
        rc = lib.adam_step_noalloc(n, arr, ctypes.byref(lay), ctypes.cast(ptrs, ctypes.c_void_p),
                                   ctypes.cast(ptrs, ctypes.c_void_p),
                                   ctypes.cast(state, ctypes.c_void_p), None, ctypes.byref(hp), None)
        assert rc == -1 and what in lib.adam_last_error(), lib.adam_last_error()


def test_step_checks_rerun_when_tensors_change(monkeypatch):
    # the binding checks a call's tensors in full when the tensor objects or
    # their data pointers differ from the last checked call on the state,
    # and only compares identities and pointers otherwise
    import torch
    st = _fake_state([100, 7])
    full = []
    monkeypatch.setattr(B, "_check_step_tensors", lambda s, p, g: full.append(1))
    ps = [torch.zeros(100), torch.zeros(7)]
    gs = [torch.zeros(100), torch.zeros(7)]
    for _ in range(3):
        B._checked_pointers(st, ps, gs)
    assert len(full) == 1
    B._checked_pointers(st, list(ps), list(gs))  # new lists, same tensors
    assert len(full) == 1
    gs2 = [gs[0], torch.zeros(7)]  # one new tensor object
    B._checked_pointers(st, ps, gs2)
    assert len(full) == 2
    ps[1].set_(torch.zeros(7).untyped_storage())  # same object, new data pointer
    P, G = B._checked_pointers(st, ps, gs2)
    assert len(full) == 3
    # the pointer arrays handed to the C call are the current ones, also when
    # they come from the remembered set
    for _ in range(2):
        assert [P[k] for k in range(2)] == [t.data_ptr() for t in ps]
        assert [G[k] for k in range(2)] == [t.data_ptr() for t in gs2]
        P, G = B._checked_pointers(st, ps, gs2)
    assert len(full) == 3
    # rotating a few gradient sets stays on the fast path
    sets = [[torch.zeros(100), torch.zeros(7)] for _ in range(4)]
    for r in range(12):
        B._checked_pointers(st, ps, sets[r % 4])
    assert len(full) == 3 + 4
    st.destroy()
    B._checked_pointers(st, ps, gs2)  # a destroyed state forgets
    assert len(full) == 8
