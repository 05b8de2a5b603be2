"""The stream probe on the GPU: one launch stores exactly what the header
states in every element of every buffer (each block visited once, in the
XCD order over 300 blocks: two full runs of 128 and a tail of 44), for
each storage, grad width and AMSGrad, at a capped and an uncapped
residency."""
import numpy as np
import pytest
import torch

from memory_efficient_adam_amd import stream_probe as sp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only"])
@pytest.mark.parametrize("grad", ["f32", "bf16"])
@pytest.mark.parametrize("ams", [False, True])
@pytest.mark.parametrize("cap", [3, 8])
def test_probe_stores_what_it_states(storage, grad, ams, cap):
    nb = 300
    print(f"stream probe {storage} grads={grad} amsgrad={ams} cap={cap}", flush=True)
    rng = np.random.default_rng([nb, cap])
    bufs = sp.probe_buffers(nb, grad, storage, ams)
    host = {}
    for name, t in bufs.items():
        if t is None:
            continue
        if name in ("param", "grad", "scales"):
            x = rng.standard_normal(t.numel()).astype(np.float32)
            src = torch.from_numpy(x)
            if t.dtype == torch.bfloat16:
                src = src.to(torch.bfloat16)
            t.copy_(src)
            host[name] = src.float().numpy() if t.dtype == torch.bfloat16 else x
        else:
            raw = rng.integers(0, 256, t.numel() * t.element_size(), dtype=np.uint8)
            t.copy_(torch.from_numpy(raw).view(t.dtype))
            host[name] = raw
    sp.adam_stream_probe(bufs, nb, grad, storage, ams, cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bufs["param"].cpu().numpy(), host["param"] + host["grad"])
    for name in ("m", "v", "w"):
        if bufs[name] is None:
            continue
        got = bufs[name].cpu().contiguous().view(torch.uint8).numpy()
        np.testing.assert_array_equal(got, host[name] ^ np.uint8(1))
    if bufs["scales"] is not None:
        got = bufs["scales"].cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got, host["scales"].view(np.uint32) + np.uint32(1))
