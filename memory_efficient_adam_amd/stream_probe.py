"""ctypes marshalling for libadam_stream_probe.so (names follow
include/adam_stream_probe.h): a measurement kernel that moves the Adam
step's bytes in the step's pattern with no arithmetic.  The step does not
use it."""
import ctypes
import os

from ._binding import STORAGES

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libadam_stream_probe.so")
_lib = None


def library():
    """Load libadam_stream_probe.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    L.adam_stream_probe.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_uint32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]
    L.adam_stream_probe.restype = ctypes.c_int
    L.adam_stream_probe_bytes.argtypes = [ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32]
    L.adam_stream_probe_bytes.restype = ctypes.c_uint64
    _lib = L
    return L


# moment bytes per element (m, v) and scales per block of each storage, with
# the AMSGrad maximum stored as v is
_LAYOUT = {"bf16": (2, 2, 0), "q8": (1, 1, 2), "q8_v_only": (4, 1, 1)}


def _grad_bytes(grad_dtype):
    return {"f32": 4, "bf16": 2}[grad_dtype]


def adam_stream_probe_bytes(n_blocks, grad_dtype, storage, amsgrad=False):
    return int(library().adam_stream_probe_bytes(n_blocks, _grad_bytes(grad_dtype),
                                                 STORAGES[storage], int(amsgrad)))


def probe_buffers_shape(n_blocks, grad_dtype, storage, amsgrad=False):
    """(elements, bytes per element) of each probe buffer (0 elements: unused)."""
    n = n_blocks * 2048
    mb, vb, ns = _LAYOUT[storage]
    return {"param": (n, 4), "grad": (n, _grad_bytes(grad_dtype)), "m": (n, mb), "v": (n, vb),
            "w": (n if amsgrad else 0, vb),
            "scales": ((ns + (1 if amsgrad else 0)) * n_blocks if ns else 0, 4)}


def probe_buffers(n_blocks, grad_dtype, storage, amsgrad=False, device="cuda"):
    """Uninitialised device buffers of one probe launch (the caller fills
    them if it checks values)."""
    import torch
    n = n_blocks * 2048
    mb, vb, ns = _LAYOUT[storage]
    bytes_dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
    return {
        "param": torch.empty(n, dtype=torch.float32, device=device),
        "grad": torch.empty(n, dtype=torch.float32 if grad_dtype == "f32" else torch.bfloat16,
                            device=device),
        "m": torch.empty(n, dtype=bytes_dt[mb], device=device),
        "v": torch.empty(n, dtype=bytes_dt[vb], device=device),
        "w": torch.empty(n, dtype=bytes_dt[vb], device=device) if amsgrad else None,
        "scales": (torch.empty((ns + (1 if amsgrad else 0)) * n_blocks, dtype=torch.float32,
                               device=device) if ns else None),
    }


def adam_stream_probe(bufs, n_blocks, grad_dtype, storage, amsgrad=False, resident_per_cu=8,
                      stream=None):
    """One probe launch over the buffers of probe_buffers(), enqueued on
    `stream` (default: torch's current stream)."""
    import torch
    # the kernel reads and writes n_blocks * 2048 elements of each buffer:
    # check every size here (the C ABI cannot)
    want = probe_buffers_shape(n_blocks, grad_dtype, storage, amsgrad)
    for name, (numel, elem) in want.items():
        t = bufs.get(name)
        if numel == 0:
            continue
        if (t is None or not t.is_cuda or not t.is_contiguous() or t.numel() != numel
                or t.element_size() != elem):
            raise ValueError(f"probe buffer {name}: want a contiguous device tensor of {numel} "
                             f"elements of {elem} bytes")
    if stream is None:
        stream = torch.cuda.current_stream()
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    rc = library().adam_stream_probe(ptr(bufs["param"]), ptr(bufs["grad"]), ptr(bufs["m"]),
                                     ptr(bufs["v"]), ptr(bufs["w"]), ptr(bufs["scales"]),
                                     n_blocks, _grad_bytes(grad_dtype), STORAGES[storage],
                                     int(amsgrad), resident_per_cu, stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"adam_stream_probe returned {rc}")
