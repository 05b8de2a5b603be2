"""The allocation-free step (adam_step_noalloc) against adam_step.

adam_step_noalloc runs the same kernels over caller-owned state buffers, with
the library's tables in a fixed device array instead of a state object.  Its
results must equal adam_step's on the same inputs bit for bit (params and
every state buffer), over two calls in a row on different tensor lists, the
second list smaller than the first (so the tables of the first call are still
in the array when the second call rewrites part of them).
"""
import sys

import numpy as np
import pytest
import torch

import memory_efficient_adam_amd as ma
import workloads

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
BIG = [3000, 2048, 17, 12289, 0, 5000, 1, 4096 * 3 + 5]
SMALL = [100, 2049]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _grads(cfg_id, numels, t, gdt):
    host = workloads.host_grads(cfg_id, numels, t, dtype=gdt)
    if gdt == "bf16":
        return [torch.from_numpy(g.view(np.int16)).cuda().view(torch.bfloat16) for g in host]
    return [torch.from_numpy(g).cuda() for g in host]


def _run_pair(numels, storage, gdt, ams, flags, cfg_id, draw_index=None, steps=2):
    """Steps both entry points from a zero state on the same inputs and
    compares everything after every step."""
    params = workloads.host_params(cfg_id, numels)
    p_ref = [torch.from_numpy(p.copy()).cuda() for p in params]
    p_new = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, gdt, amsgrad=ams)
    if draw_index is not None:
        ma.adam_state_set_draw_index(st, draw_index)
    bufs = {name: torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
            for name, nbytes in ma.state_buffer_sizes(numels, storage, ams).items()}
    for t in range(1, steps + 1):
        g = _grads(cfg_id, numels, t, gdt)
        ma.adam_step(st, p_ref, g, t=t, **HP, **flags)
        ma.adam_step_noalloc(p_new, g, bufs, storage=storage, grad_dtype=gdt, amsgrad=ams, t=t,
                             draw_index=draw_index, **HP, **flags)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            a = p_ref[k].view(torch.int32).cpu().numpy()
            b = p_new[k].view(torch.int32).cpu().numpy()
            assert np.array_equal(a, b), f"t={t} tensor {k}: params differ"
        for name, buf in bufs.items():
            want = ma.adam_state_read(st, name).view(torch.uint8).cpu().numpy()
            got = buf.cpu().numpy()
            assert np.array_equal(want, got), f"t={t}: buffer {name} differs"
    st.destroy()
    return sum(numels)


CASES = [
    # storage, grad dtype, amsgrad, flags
    ("q8", "f32", False, dict(stochastic=True, seed=11)),
    ("q8", "bf16", False, dict()),
    ("q8", "f32", False, dict(percentile=99.0)),
    ("q8_v_only", "bf16", True, dict(percentile=99.9, stochastic=True)),
    ("bf16", "f32", False, dict()),
    ("bf16", "bf16", True, dict(decoupled=False)),
    ("q8", "f32", True, dict(static_scales=True, stochastic=True)),
]


@pytest.mark.parametrize("storage,gdt,ams,flags", CASES)
def test_noalloc_matches_adam_step_on_two_calls(storage, gdt, ams, flags):
    log(f"noalloc vs adam_step: {storage} grads {gdt} amsgrad={ams} {flags}")
    n1 = _run_pair(BIG, storage, gdt, ams, flags, cfg_id=61)
    n2 = _run_pair(SMALL, storage, gdt, ams, flags, cfg_id=62)
    log(f"  bit-exact on {n1} then {n2} params")


def test_noalloc_draw_index_and_more_tensors_than_one_fill_launch():
    # 150 tensors (three fill launches of up to 64) with shard-style draw indices
    rng = np.random.default_rng(5)
    numels = [int(x) for x in rng.integers(1, 6000, 150)]
    first = []
    at = 1 << 40
    for n in numels:
        first.append(at)
        at += (n + 15) // 16 * 16 + 16 * int(rng.integers(0, 4))
    _run_pair(numels, "q8", "bf16", False, dict(stochastic=True, seed=3), cfg_id=63,
              draw_index=first)
    _run_pair([7, 9000], "q8", "bf16", False, dict(stochastic=True, seed=3), cfg_id=64)


def test_noalloc_refuses_beyond_its_limits():
    bufs = {}
    with pytest.raises(ma.AdamError) as e:
        z = torch.zeros(16, device="cuda")
        ma.adam_step_noalloc([z] * 70000, [z] * 70000, {
            n: torch.zeros(b, dtype=torch.uint8, device="cuda")
            for n, b in ma.state_buffer_sizes([16] * 70000, "q8").items()},
            storage="q8", t=1, **HP)
    assert e.value.code == -1 and "65536" in str(e.value)
    del bufs
