"""ctypes marshalling for libadam_mi355x.so (names follow include/adam_mi355x.h)."""
import ctypes
import operator
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libadam_mi355x.so")

ADAM_BLOCK_SIZE = 2048
STORAGES = {"bf16": 1, "q8": 2, "q8_v_only": 3}
GRAD_DTYPES = {"f32": 0, "bf16": 1}
BUFFERS = {"m_codes": 0, "v_codes": 1, "m_scale": 2, "v_scale": 3, "m_bf16": 4,
           "v_bf16": 5, "m_f32": 6, "vmax_codes": 7, "vmax_scale": 8, "vmax_bf16": 9}
OPT_AMSGRAD = 1
_F_DECOUPLED, _F_STOCHASTIC, _F_PERCENTILE, _F_STATIC_SCALES = 1, 2, 4, 8
_STATUS = {0: "ADAM_OK", -1: "ADAM_EINVAL", -2: "ADAM_EMODE", -3: "ADAM_EALIGN",
           -4: "ADAM_ENOMEM", -5: "ADAM_EDEVICE"}


class adam_layout(ctypes.Structure):
    _fields_ = [("storage", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("options", ctypes.c_uint32)]


class adam_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("percentile", ctypes.c_float), ("t", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]


class AdamError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{_STATUS.get(code, code)}: {message}")
        self.code = code


_lib = None


def library_path():
    return _LIB_PATH


def library():
    """Load libadam_mi355x.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built (run __graft_entry__.build() or "
                           "python memory_efficient_adam_amd/build.py); there is no fallback")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
    L.adam_state_bytes.argtypes = [ctypes.c_int32, i64p, ctypes.POINTER(adam_layout)]
    L.adam_state_bytes.restype = ctypes.c_int64
    L.adam_state_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int32, i64p,
                                    ctypes.POINTER(adam_layout), vp]
    L.adam_state_create.restype = ctypes.c_int
    L.adam_step.argtypes = [vp, vp, vp, ctypes.POINTER(adam_hparams),
                            ctypes.POINTER(adam_layout), vp]
    L.adam_step.restype = ctypes.c_int
    L.adam_state_buffer_bytes.argtypes = [vp, ctypes.c_int32]
    L.adam_state_buffer_bytes.restype = ctypes.c_int64
    L.adam_state_read.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int64, vp]
    L.adam_state_read.restype = ctypes.c_int
    L.adam_state_write.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int64, vp]
    L.adam_state_write.restype = ctypes.c_int
    L.adam_state_describe.argtypes = [vp, ctypes.POINTER(adam_layout), i64p, ctypes.c_int32]
    L.adam_state_describe.restype = ctypes.c_int32
    L.adam_state_serialized_bytes.argtypes = [vp]
    L.adam_state_serialized_bytes.restype = ctypes.c_int64
    L.adam_state_save.argtypes = [vp, vp, ctypes.c_int64, vp]
    L.adam_state_save.restype = ctypes.c_int
    L.adam_state_load.argtypes = [ctypes.POINTER(vp), vp, ctypes.c_int64, vp]
    L.adam_state_load.restype = ctypes.c_int
    L.adam_state_set_draw_index.argtypes = [vp, i64p, vp]
    L.adam_state_set_draw_index.restype = ctypes.c_int
    L.adam_state_get_draw_index.argtypes = [vp, i64p, ctypes.c_int32]
    L.adam_state_get_draw_index.restype = ctypes.c_int32
    L.adam_step_noalloc.argtypes = [ctypes.c_int32, i64p, ctypes.POINTER(adam_layout), vp, vp, vp,
                                    i64p, ctypes.POINTER(adam_hparams), vp]
    L.adam_step_noalloc.restype = ctypes.c_int
    L.adam_state_destroy.argtypes = [vp]
    L.adam_state_destroy.restype = None
    L.adam_last_error.argtypes = []
    L.adam_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def adam_last_error():
    return library().adam_last_error().decode()


def _check(rc):
    if rc != 0:
        raise AdamError(rc, adam_last_error())


def _layout(storage, grad_dtype, block_size=ADAM_BLOCK_SIZE, options=0):
    return adam_layout(STORAGES.get(storage, storage) if isinstance(storage, str) else storage,
                       GRAD_DTYPES.get(grad_dtype, grad_dtype) if isinstance(grad_dtype, str)
                       else grad_dtype, block_size, options)


def _numels(numels):
    arr = (ctypes.c_int64 * max(len(numels), 1))(*[int(n) for n in numels])
    return len(numels), arr


def _current_device():
    import torch
    return torch.cuda.current_device()


_GRAD_TORCH_DTYPES = {0: ("float32",), 1: ("bfloat16", "int16", "uint16")}


def _check_step_tensors(state, params, grads):
    """The kernel reads and writes exactly numel elements through each raw
    pointer: a shorter, strided, mistyped or host tensor would make it touch
    memory that is not the tensor's.  Every tensor is checked here, before
    any pointer reaches the library."""
    import torch
    n = len(state.numels)
    if len(params) != n or len(grads) != n:
        raise ValueError(f"expected {n} params and grads, got {len(params)} and {len(grads)}")
    gdts = _GRAD_TORCH_DTYPES[state.layout.grad_dtype]
    for k, (p, g, want) in enumerate(zip(params, grads, state.numels)):
        if not isinstance(p, torch.Tensor) or not isinstance(g, torch.Tensor):
            raise TypeError(f"tensor {k}: params and grads must be torch tensors")
        if p.dtype != torch.float32:
            raise ValueError(f"param {k}: dtype {p.dtype}, expected torch.float32")
        if str(g.dtype).replace("torch.", "") not in gdts:
            raise ValueError(f"grad {k}: dtype {g.dtype}, expected one of {gdts} for this layout")
        if p.numel() != want or g.numel() != want:
            raise ValueError(f"tensor {k}: param/grad numel {p.numel()}/{g.numel()}, the state "
                             f"holds {want}")
        if not p.is_contiguous() or not g.is_contiguous():
            raise ValueError(f"tensor {k}: params and grads must be contiguous")
    for k, (p, g, want) in enumerate(zip(params, grads, state.numels)):
        if want == 0:
            continue
        if not p.is_cuda or not g.is_cuda:
            raise ValueError(f"tensor {k}: params and grads must be CUDA (HIP) device tensors")
        if state.device is not None and (p.device.index != state.device
                                         or g.device.index != state.device):
            raise ValueError(f"tensor {k}: on {p.device}/{g.device}, the state lives on "
                             f"cuda:{state.device}")


_CHECKED_SETS = 8  # tensor sets remembered per state (callers rotate gradient buffers)


def _checked_pointers(state, params, grads):
    """Device pointer arrays (ctypes) of params and grads.  The full tensor
    checks run when the (params, grads) tensor objects and their data
    pointers are not among the last few sets checked on this state: a caller
    stepping the same tensors, or rotating a few gradient buffers, pays two
    passes of data_ptr() and an identity compare (~0.25 us per tensor)
    instead of the checks (~1.5 us per tensor, which for a 150-tensor model
    outlast a step of the kernel and would leave the GPU waiting on the
    host), and reuses the set's pointer arrays.  The state holds the
    remembered tensors until they are pushed out or destroy()."""
    import torch
    ptr = torch.Tensor.data_ptr
    try:
        pp = list(map(ptr, params))
        gp = list(map(ptr, grads))
    except (TypeError, AttributeError):
        _check_step_tensors(state, params, grads)  # raises the precise error
        raise
    sets = state._checked
    for c in sets:
        if (c[2] == pp and c[3] == gp and len(c[0]) == len(params) and len(c[1]) == len(grads)
                and all(map(operator.is_, c[0], params)) and all(map(operator.is_, c[1], grads))):
            return c[4], c[5]
    _check_step_tensors(state, params, grads)
    n = max(len(state.numels), 1)
    P = (ctypes.c_void_p * n)(*pp)
    G = (ctypes.c_void_p * n)(*gp)
    sets.insert(0, (tuple(params), tuple(grads), pp, gp, P, G))
    del sets[_CHECKED_SETS:]
    return P, G


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def adam_state_bytes(numels, storage, grad_dtype="f32", block_size=ADAM_BLOCK_SIZE,
                     amsgrad=False):
    n, arr = _numels(numels)
    lay = _layout(storage, grad_dtype, block_size, OPT_AMSGRAD if amsgrad else 0)
    rc = library().adam_state_bytes(n, arr, ctypes.byref(lay))
    if rc < 0:
        raise AdamError(int(rc), adam_last_error())
    return int(rc)


class AdamState:
    """Owns one library state (freed on destroy() or garbage collection).
    device: the CUDA device index the state lives on (None: not recorded)."""

    def __init__(self, handle, numels, layout, device=None):
        self.handle = handle
        self.numels = list(numels)
        self.layout = layout
        self.device = device
        # tensor sets (held) and pointers of recent checked adam_step calls
        self._checked = []

    def __del__(self):
        self.destroy()

    def destroy(self):
        self._checked = []
        if getattr(self, "handle", None):
            library().adam_state_destroy(self.handle)
            self.handle = None

    @property
    def storage(self):
        return {v: k for k, v in STORAGES.items()}[self.layout.storage]

    @property
    def amsgrad(self):
        return bool(self.layout.options & OPT_AMSGRAD)


def adam_state_create(numels, storage, grad_dtype="f32", block_size=ADAM_BLOCK_SIZE,
                      amsgrad=False, stream=None):
    """A zero state for tensors of the given sizes; amsgrad keeps the running
    maximum of v (layout option ADAM_OPT_AMSGRAD)."""
    n, arr = _numels(numels)
    lay = _layout(storage, grad_dtype, block_size, OPT_AMSGRAD if amsgrad else 0)
    h = ctypes.c_void_p()
    _check(library().adam_state_create(ctypes.byref(h), n, arr, ctypes.byref(lay),
                                       _stream(stream)))
    return AdamState(h.value, numels, lay, _current_device())


def adam_state_destroy(state):
    state.destroy()


def adam_step(state, params, grads, *, lr, beta1, beta2, eps, weight_decay, t,
              decoupled=True, stochastic=False, percentile=None, seed=42, static_scales=False,
              stream=None, expect=None):
    """One step over all tensors.  params: fp32 device tensors (updated in
    place); grads: fp32 or bf16 device tensors; percentile=None selects the
    absmax block statistic; static_scales keeps each block's scale once set.
    expect: (storage, grad_dtype[, block_size[, options]]) the caller believes
    the state has (default: the state's own layout)."""
    P, G = _checked_pointers(state, params, grads)
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, t, decoupled, stochastic, percentile, seed,
                  static_scales)
    lay = state.layout if expect is None else _layout(*expect)
    _check(library().adam_step(state.handle, ctypes.cast(P, ctypes.c_void_p),
                               ctypes.cast(G, ctypes.c_void_p), ctypes.byref(hp),
                               ctypes.byref(lay), _stream(stream)))


def _hparams(lr, beta1, beta2, eps, weight_decay, t, decoupled, stochastic, percentile, seed,
             static_scales):
    flags = ((_F_DECOUPLED if decoupled else 0) | (_F_STOCHASTIC if stochastic else 0)
             | (_F_PERCENTILE if percentile is not None else 0)
             | (_F_STATIC_SCALES if static_scales else 0))
    return adam_hparams(lr, beta1, beta2, eps, weight_decay,
                        100.0 if percentile is None else percentile, int(t), flags, 0, int(seed))


def state_buffer_sizes(numels, storage, amsgrad=False):
    """{buffer name: bytes} of every state buffer a layout has, for caller-owned
    state (adam_step_noalloc): padded elements = sum of pad16(numel), blocks =
    sum of ceil(numel / 2048), as include/adam_mi355x.h lays them out."""
    padded = sum((int(n) + 15) // 16 * 16 for n in numels)
    blocks = sum(-(-int(n) // ADAM_BLOCK_SIZE) for n in numels)
    sizes = {"bf16": {"m_bf16": 2 * padded, "v_bf16": 2 * padded},
             "q8": {"m_codes": padded, "v_codes": padded, "m_scale": 4 * blocks,
                    "v_scale": 4 * blocks},
             "q8_v_only": {"v_codes": padded, "v_scale": 4 * blocks, "m_f32": 4 * padded}}[storage]
    if amsgrad:
        sizes.update({"vmax_bf16": 2 * padded} if storage == "bf16"
                     else {"vmax_codes": padded, "vmax_scale": 4 * blocks})
    return sizes


def adam_step_noalloc(params, grads, buffers, *, storage, grad_dtype="f32", amsgrad=False, lr,
                      beta1, beta2, eps, weight_decay, t, decoupled=True, stochastic=False,
                      percentile=None, seed=42, static_scales=False, draw_index=None,
                      stream=None):
    """The allocation-free step over caller-owned state: buffers maps each
    buffer name of the layout (state_buffer_sizes) to a contiguous device
    tensor of exactly that many bytes (zeros for a new state).  The library
    allocates nothing; its tables live in a fixed device array (calls that
    overlap on one GPU race on it)."""
    numels = [int(p.numel()) for p in params]
    lay = _layout(storage, grad_dtype, ADAM_BLOCK_SIZE, OPT_AMSGRAD if amsgrad else 0)
    _check_step_tensors(AdamState(None, numels, lay), params, grads)
    want = state_buffer_sizes(numels, storage, amsgrad)
    if set(buffers) != set(want):
        raise ValueError(f"buffers must be exactly {sorted(want)}, got {sorted(buffers)}")
    S = (ctypes.c_void_p * len(BUFFERS))()
    for name, nbytes in want.items():
        b = buffers[name]
        if b.numel() * b.element_size() != nbytes or not b.is_contiguous():
            raise ValueError(f"buffer {name}: must be a contiguous tensor of {nbytes} bytes")
        if nbytes and not b.is_cuda:
            raise ValueError(f"buffer {name}: must be a device tensor")
        S[BUFFERS[name]] = b.data_ptr()
    n, arr = _numels(numels)
    P = (ctypes.c_void_p * max(n, 1))(*[p.data_ptr() for p in params])
    G = (ctypes.c_void_p * max(n, 1))(*[g.data_ptr() for g in grads])
    D = None
    if draw_index is not None:
        if len(draw_index) != n:
            raise ValueError(f"expected {n} draw indices")
        D = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in draw_index])
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, t, decoupled, stochastic, percentile, seed,
                  static_scales)
    _check(library().adam_step_noalloc(n, arr, ctypes.byref(lay), ctypes.cast(P, ctypes.c_void_p),
                                       ctypes.cast(G, ctypes.c_void_p),
                                       ctypes.cast(S, ctypes.c_void_p), D, ctypes.byref(hp),
                                       _stream(stream)))


def adam_state_buffer_bytes(state, which):
    w = BUFFERS.get(which, which) if isinstance(which, str) else which
    rc = library().adam_state_buffer_bytes(state.handle, w)
    if rc < 0:
        raise AdamError(int(rc), adam_last_error())
    return int(rc)


_BUF_DTYPES = {"m_codes": "int8", "v_codes": "uint8", "m_scale": "float32",
               "v_scale": "float32", "m_bf16": "int16", "v_bf16": "int16", "m_f32": "float32",
               "vmax_codes": "uint8", "vmax_scale": "float32", "vmax_bf16": "int16"}


def adam_state_read(state, which, out=None, stream=None):
    """Copy a state buffer into a (new, device) torch tensor; bf16 moments
    come back as int16 bit patterns."""
    import torch
    nbytes = adam_state_buffer_bytes(state, which)
    if out is None:
        dt = getattr(torch, _BUF_DTYPES[which])
        out = torch.empty(nbytes // dt.itemsize, dtype=dt, device="cuda")
    elif out.numel() * out.element_size() != nbytes or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous tensor of exactly {nbytes} bytes, got "
                         f"{out.numel() * out.element_size()} bytes")
    _check(library().adam_state_read(state.handle, BUFFERS[which], out.data_ptr(), nbytes,
                                     _stream(stream)))
    return out


def adam_state_write(state, which, src, stream=None):
    nbytes = adam_state_buffer_bytes(state, which)
    if src.numel() * src.element_size() != nbytes or not src.is_contiguous():
        raise ValueError(f"src must be a contiguous tensor of exactly {nbytes} bytes, got "
                         f"{src.numel() * src.element_size()} bytes")
    _check(library().adam_state_write(state.handle, BUFFERS[which], src.data_ptr(), nbytes,
                                      _stream(stream)))


def adam_state_describe(state):
    """(layout, numels) of a state, as the library holds them."""
    lay = adam_layout()
    n = library().adam_state_describe(state.handle, ctypes.byref(lay), None, 0)
    if n < 0:
        raise AdamError(int(n), adam_last_error())
    arr = (ctypes.c_int64 * max(n, 1))()
    library().adam_state_describe(state.handle, ctypes.byref(lay), arr, n)
    return lay, [int(arr[i]) for i in range(n)]


def adam_state_set_draw_index(state, first_index, stream=None):
    """Per tensor: the stochastic-rounding draw index of element 0 (e.g. a
    shard slice's flat index in the unsharded state)."""
    n, arr = _numels(first_index)
    if n != len(state.numels):
        raise ValueError(f"expected {len(state.numels)} draw indices")
    _check(library().adam_state_set_draw_index(state.handle, arr, _stream(stream)))


def adam_state_get_draw_index(state):
    n = len(state.numels)
    arr = (ctypes.c_int64 * max(n, 1))()
    rc = library().adam_state_get_draw_index(state.handle, arr, n)
    if rc < 0:
        raise AdamError(int(rc), adam_last_error())
    return [int(arr[i]) for i in range(n)]


def adam_state_serialized_bytes(state):
    n = library().adam_state_serialized_bytes(state.handle)
    if n < 0:
        raise AdamError(int(n), adam_last_error())
    return int(n)


def adam_state_save(state, stream=None):
    """The serialized state as a numpy uint8 array (host memory)."""
    import numpy as np
    out = np.empty(adam_state_serialized_bytes(state), np.uint8)
    _check(library().adam_state_save(state.handle, out.ctypes.data, out.size, _stream(stream)))
    return out


def adam_state_load(buf, stream=None):
    """A new state holding the contents of a serialized state (bytes-like or
    numpy uint8 array)."""
    import numpy as np
    arr = np.ascontiguousarray(np.frombuffer(buf, np.uint8) if not isinstance(buf, np.ndarray)
                               else buf.view(np.uint8))
    h = ctypes.c_void_p()
    _check(library().adam_state_load(ctypes.byref(h), arr.ctypes.data, arr.size, _stream(stream)))
    st = AdamState(h.value, [], adam_layout(), _current_device())
    st.layout, st.numels = adam_state_describe(st)
    return st
