"""Host-side checks of the stream-probe library (no GPU): it loads and
exports every function include/adam_stream_probe.h declares, its byte count
has the closed form the header states and matches the step's algorithmic
bytes on full blocks, and bad arguments come back before any HIP call."""
import ctypes
import os
import re

import pytest

from memory_efficient_adam_amd import stream_probe as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adam_stream_probe.h")


def test_probe_library_exports_every_declared_function():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(adam_[a-z_]+)\s*\(", src)))
    assert names == ["adam_stream_probe", "adam_stream_probe_bytes"]
    lib = ctypes.CDLL(sp._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


# per element: param 4 + 4, grad, each moment read and written; per block:
# each scale read and written
@pytest.mark.parametrize("storage,grad,ams,per_elem,per_block", [
    ("bf16", "f32", False, 8 + 4 + 4 + 4, 0),
    ("bf16", "bf16", True, 8 + 2 + 4 + 4 + 4, 0),
    ("q8", "f32", False, 8 + 4 + 2 + 2, 16),
    ("q8", "bf16", True, 8 + 2 + 2 + 2 + 2, 24),
    ("q8_v_only", "bf16", False, 8 + 2 + 8 + 2, 8),
    ("q8_v_only", "f32", True, 8 + 4 + 8 + 2 + 2, 16),
])
def test_probe_bytes_closed_form(storage, grad, ams, per_elem, per_block):
    for nb in (1, 7, 42334):
        assert sp.adam_stream_probe_bytes(nb, grad, storage, ams) == nb * (2048 * per_elem + per_block)


def test_probe_bytes_equal_the_steps_on_full_blocks():
    import bench
    import workloads
    for name in ("vit_bf16", "vit_q8", "gpt1p3b_q8_sr", "llama7b_mf32_vq8_pct"):
        cfg = workloads.CONFIGS[name]
        one = type("C", (), dict(numels=lambda self: [2048 * 5], grad_dtype=cfg.grad_dtype,
                                 storage=cfg.storage, amsgrad=cfg.amsgrad))()
        assert sp.adam_stream_probe_bytes(5, cfg.grad_dtype, cfg.storage) == bench.algorithmic_bytes(one)


def test_probe_rejects_bad_arguments_before_any_device_call():
    L = sp.library()
    buf = ctypes.c_void_p(1 << 20)  # never dereferenced: every case fails its checks first
    ok = dict(param=buf, grad=buf, m=buf, v=buf, w=None, scales=buf, n_blocks=4, grad_bytes=4,
              storage=2, amsgrad=0, cap=8)

    def call(**kw):
        a = dict(ok, **kw)
        return L.adam_stream_probe(a["param"], a["grad"], a["m"], a["v"], a["w"], a["scales"],
                                   a["n_blocks"], a["grad_bytes"], a["storage"], a["amsgrad"],
                                   a["cap"], None)

    assert call(storage=0) == -1 and call(storage=4) == -1
    assert call(grad_bytes=3) == -1
    assert call(n_blocks=0) == -1 and call(n_blocks=1 << 24) == -1
    assert call(cap=1) == -1 and call(cap=9) == -1
    assert call(param=None) == -1 and call(m=ctypes.c_void_p((1 << 20) + 8)) == -1
    assert call(scales=None) == -1          # 8-bit moments need their scales
    assert call(amsgrad=1) == -1            # ... and AMSGrad its maximum
    assert sp.adam_stream_probe_bytes(4, "f32", "q8") > 0
    assert L.adam_stream_probe_bytes(4, 3, 2, 0) == 0 and L.adam_stream_probe_bytes(4, 4, 9, 0) == 0
