"""CPU oracle for the compressed-moment Adam step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``adam_oracle.c`` (plain,
scalar fp32 C; see that file's header for the sources and the pins) with
ctypes; this module only marshals numpy arrays, it does no arithmetic of the
method.  It imports nothing from the HIP implementation and shares no code
with it.

Storage modes are named by strings here: "f32" (oracle-only textbook mode
with fp32 moments), "bf16", "q8" (int8 m + uint8 v, one fp32 scale per
block each) and "q8_v_only" (fp32 m + uint8 v).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_STORAGE = {"f32": 0, "bf16": 1, "q8": 2, "q8_v_only": 3}
_lib = None

# state buffers, in the order of the C struct orc_ptrs
_PTR_FIELDS = ["m_codes", "v_codes", "vmax_codes", "m_scale", "v_scale", "vmax_scale",
               "m_bf16", "v_bf16", "vmax_bf16", "m_f32", "v_f32", "vmax_f32"]


class _OrcPtrs(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _PTR_FIELDS]

_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


def lib():
    """Load (building first if absent) the oracle's shared library.  The
    environment variable ORACLE_LIBRARY names another build of the same
    source to load instead (the sanitizer tests use it)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIBRARY") or _build.LIBRARY
    if path == _build.LIBRARY and not os.path.exists(path):
        _build.build()
    L = ctypes.CDLL(path)
    L.orc_bf16_from_f32_array.argtypes = [_f32p, _u16p, ctypes.c_int64]
    L.orc_f32_from_bf16_array.argtypes = [_u16p, _f32p, ctypes.c_int64]
    L.orc_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    L.orc_sr_draws.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_int32, _u16p]
    L.orc_percentile_rank.argtypes = [ctypes.c_float, ctypes.c_int64]
    L.orc_percentile_rank.restype = ctypes.c_int64
    L.orc_block_stat.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float]
    L.orc_block_stat.restype = ctypes.c_float
    L.orc_dequantize_block.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_float, _f32p]
    L.orc_quantize_with_stat.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_float, _u16p, _i32p]
    L.orc_quantize_with_stat.restype = ctypes.c_float
    L.orc_quantize_block.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_float, _u16p, _i32p]
    L.orc_quantize_block.restype = ctypes.c_float
    L.orc_host_scalars.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, ctypes.c_int64, ctypes.c_int32, _f32p]
    L.orc_adam_step.argtypes = (
        [ctypes.c_int32, _i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp,
         ctypes.POINTER(_OrcPtrs)]
        + [ctypes.c_float] * 6
        + [ctypes.c_int64] + [ctypes.c_int32] * 5 + [ctypes.c_uint64]
        + [_vp, _vp, _vp])
    L.orc_adam_step.restype = ctypes.c_int
    L.orc_adam_step_blocks.argtypes = (
        [ctypes.c_int64, _i64p, _i64p, _i64p, ctypes.c_int32, ctypes.c_int32, _vp, _vp,
         ctypes.POINTER(_OrcPtrs)]
        + [ctypes.c_float] * 6
        + [ctypes.c_int64] + [ctypes.c_int32] * 5 + [ctypes.c_uint64])
    L.orc_adam_step_blocks.restype = ctypes.c_int
    _lib = L
    return L


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def _vptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# --------------------------------------------------------------------------
# element-level helpers
# --------------------------------------------------------------------------
def bf16_from_f32(x):
    x = _c(x, np.float32).ravel()
    out = np.empty(x.size, np.uint16)
    lib().orc_bf16_from_f32_array(_ptr(x, _f32p), _ptr(out, _u16p), x.size)
    return out


def f32_from_bf16(h):
    h = _c(h, np.uint16).ravel()
    out = np.empty(h.size, np.float32)
    lib().orc_f32_from_bf16_array(_ptr(h, _u16p), _ptr(out, _f32p), h.size)
    return out


def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    assert c.size == 4 and k.size == 2
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c, _u32p), _ptr(k, _u32p), _ptr(out, _u32p))
    return out


def sr_draws(seed, t, gidx0, n, which):
    """16-bit stochastic-rounding draws; which=0 first moment, 1 second."""
    out = np.empty(n, np.uint16)
    lib().orc_sr_draws(seed, t, gidx0, n, which, _ptr(out, _u16p))
    return out


def percentile_rank(p, n):
    return int(lib().orc_percentile_rank(p, n))


def block_stat(a, use_pct=False, p=99.9):
    a = _c(a, np.float32).ravel()
    return float(lib().orc_block_stat(_ptr(a, _f32p), a.size, int(use_pct), p))


def dequantize_block(codes, signed, A):
    c = _c(codes, np.int32).ravel()
    out = np.empty(c.size, np.float32)
    lib().orc_dequantize_block(_ptr(c, _i32p), c.size, int(signed), A, _ptr(out, _f32p))
    return out


def quantize_with_stat(x, signed, A, draws=None):
    x = _c(x, np.float32).ravel()
    codes = np.empty(x.size, np.int32)
    d = None if draws is None else _c(draws, np.uint16).ravel()
    A_out = lib().orc_quantize_with_stat(_ptr(x, _f32p), x.size, int(signed), A,
                                         None if d is None else _ptr(d, _u16p),
                                         _ptr(codes, _i32p))
    return codes, np.float32(A_out)


def quantize_block(x, signed, use_pct=False, p=99.9, draws=None):
    x = _c(x, np.float32).ravel()
    codes = np.empty(x.size, np.int32)
    d = None if draws is None else _c(draws, np.uint16).ravel()
    A = lib().orc_quantize_block(_ptr(x, _f32p), x.size, int(signed), int(use_pct), p,
                                 None if d is None else _ptr(d, _u16p),
                                 _ptr(codes, _i32p))
    return codes, np.float32(A)


def host_scalars(lr, beta1, beta2, wd, t, decoupled=True):
    """(step, ibc2, decay, 1-beta1, 1-beta2) as fp32."""
    out = np.empty(5, np.float32)
    lib().orc_host_scalars(lr, beta1, beta2, wd, t, int(decoupled), _ptr(out, _f32p))
    return out


# --------------------------------------------------------------------------
# multi-tensor state + step
# --------------------------------------------------------------------------
def pad16(n):
    return (n + 15) // 16 * 16


class OracleState:
    """Flat, padded optimizer state held in numpy arrays (all zero at start).

    numels: element counts of the tensors, in order; block: block length.
    Buffers present per storage mode:
      f32:        m_f32, v_f32
      bf16:       m_bf16, v_bf16 (uint16 bit patterns)
      q8:         m_codes (int8), v_codes (uint8), m_scale, v_scale
      q8_v_only:  m_f32, v_codes, v_scale
    amsgrad adds the running maximum of v, stored like v: vmax_f32,
    vmax_bf16, or vmax_codes (uint8) + vmax_scale.
    """

    def __init__(self, numels, storage, block=2048, grad_bf16=False, amsgrad=False):
        self.numels = [int(n) for n in numels]
        self.storage = storage
        self.block = int(block)
        self.grad_bf16 = bool(grad_bf16)
        self.amsgrad = bool(amsgrad)
        self.total = sum(pad16(n) for n in self.numels)
        self.nblocks = sum((n + self.block - 1) // self.block for n in self.numels)
        _alloc(self, storage, self.total, self.nblocks, self.amsgrad)

    def buffers(self):
        return {k: getattr(self, k) for k in _PTR_FIELDS if getattr(self, k) is not None}

    def _ptrs(self):
        return _OrcPtrs(*[_vptr(getattr(self, f)) for f in _PTR_FIELDS])

    def step(self, params, grads, *, lr, beta1, beta2, eps, weight_decay, t,
             decoupled=True, stochastic=False, percentile=None, seed=42,
             static_scales=False, want_moments=False):
        """Advance params (list of float32 arrays, updated in place).

        grads: float32 arrays, or uint16 bf16 bit patterns if grad_bf16.
        percentile=None selects the absmax statistic; static_scales keeps
        each block's first scale.
        Returns (m_new, v_new) -- plus vmax_new with amsgrad -- flat padded
        fp32 arrays if want_moments.
        """
        n = len(self.numels)
        assert len(params) == n and len(grads) == n
        gdt = np.uint16 if self.grad_bf16 else np.float32
        for k in range(n):
            assert params[k].dtype == np.float32 and params[k].flags.c_contiguous
            assert params[k].size == self.numels[k]
            assert grads[k].dtype == gdt and grads[k].size == self.numels[k]
        numels = np.array(self.numels, np.int64)
        P = (ctypes.c_void_p * max(n, 1))(*[p.ctypes.data for p in params])
        G = (ctypes.c_void_p * max(n, 1))(*[np.ascontiguousarray(g).ctypes.data
                                             for g in grads])
        m_new = v_new = w_new = None
        if want_moments:
            m_new = np.zeros(self.total, np.float32)
            v_new = np.zeros(self.total, np.float32)
            w_new = np.zeros(self.total, np.float32)
        use_pct = percentile is not None
        ptrs = self._ptrs()
        rc = lib().orc_adam_step(
            n, _ptr(numels, _i64p), self.block, _STORAGE[self.storage], int(self.grad_bf16),
            ctypes.cast(P, _vp), ctypes.cast(G, _vp), ctypes.byref(ptrs),
            lr, beta1, beta2, eps, weight_decay, percentile if use_pct else 100.0,
            t, int(decoupled), int(stochastic), int(use_pct), int(static_scales),
            int(self.amsgrad), seed, _vptr(m_new), _vptr(v_new), _vptr(w_new))
        if rc != 0:
            raise ValueError("oracle rejected the step arguments")
        if want_moments:
            return (m_new, v_new, w_new) if self.amsgrad else (m_new, v_new)
        return None


def _alloc(obj, storage, T, B, amsgrad):
    for f in _PTR_FIELDS:
        setattr(obj, f, None)
    if storage == "f32":
        obj.m_f32 = np.zeros(T, np.float32)
        obj.v_f32 = np.zeros(T, np.float32)
        if amsgrad:
            obj.vmax_f32 = np.zeros(T, np.float32)
    elif storage == "bf16":
        obj.m_bf16 = np.zeros(T, np.uint16)
        obj.v_bf16 = np.zeros(T, np.uint16)
        if amsgrad:
            obj.vmax_bf16 = np.zeros(T, np.uint16)
    elif storage in ("q8", "q8_v_only"):
        if storage == "q8":
            obj.m_codes = np.zeros(T, np.int8)
            obj.m_scale = np.zeros(B, np.float32)
        else:
            obj.m_f32 = np.zeros(T, np.float32)
        obj.v_codes = np.zeros(T, np.uint8)
        obj.v_scale = np.zeros(B, np.float32)
        if amsgrad:
            obj.vmax_codes = np.zeros(T, np.uint8)
            obj.vmax_scale = np.zeros(B, np.float32)
    else:
        raise ValueError(storage)


class OracleBlocks:
    """State for a sample of independent blocks (full-size workloads).

    blocks: list of (n, gidx) -- element count and first padded flat index of
    each sampled block.  State for block i lives at offset off[i] of flat
    arrays sized to the sample; scale slot i.
    """

    def __init__(self, blocks, storage, grad_bf16=False, amsgrad=False):
        self.n = np.array([b[0] for b in blocks], np.int64)
        self.gidx = np.array([b[1] for b in blocks], np.int64)
        self.off = np.zeros(len(blocks), np.int64)
        if len(blocks):
            self.off[1:] = np.cumsum([pad16(int(x)) for x in self.n])[:-1]
        total = int(sum(pad16(int(x)) for x in self.n))
        self.inner = OracleState([], storage, grad_bf16=grad_bf16, amsgrad=amsgrad)
        self.storage = storage
        self.grad_bf16 = bool(grad_bf16)
        self.amsgrad = bool(amsgrad)
        _alloc(self.inner, storage, total, len(blocks), self.amsgrad)

    def buffers(self):
        return self.inner.buffers()

    def block_slice(self, i):
        o = int(self.off[i])
        return slice(o, o + int(self.n[i]))

    def step(self, params, grads, *, lr, beta1, beta2, eps, weight_decay, t,
             decoupled=True, stochastic=False, percentile=None, seed=42, static_scales=False):
        """params[i]/grads[i]: arrays of block i (params updated in place)."""
        B = len(self.n)
        gdt = np.uint16 if self.grad_bf16 else np.float32
        for i in range(B):
            assert params[i].dtype == np.float32 and params[i].size == self.n[i]
            assert grads[i].dtype == gdt and grads[i].size == self.n[i]
        P = (ctypes.c_void_p * max(B, 1))(*[p.ctypes.data for p in params])
        G = (ctypes.c_void_p * max(B, 1))(*[g.ctypes.data for g in grads])
        use_pct = percentile is not None
        ptrs = self.inner._ptrs()
        rc = lib().orc_adam_step_blocks(
            B, _ptr(self.n, _i64p), _ptr(self.gidx, _i64p), _ptr(self.off, _i64p),
            _STORAGE[self.storage], int(self.grad_bf16),
            ctypes.cast(P, _vp), ctypes.cast(G, _vp), ctypes.byref(ptrs),
            lr, beta1, beta2, eps, weight_decay, percentile if use_pct else 100.0,
            t, int(decoupled), int(stochastic), int(use_pct), int(static_scales),
            int(self.amsgrad), seed)
        if rc != 0:
            raise ValueError("oracle rejected the step arguments")
