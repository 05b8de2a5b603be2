"""Pins for the oracle's AMSGrad mode (running maximum of the second moment).

References used here, none of them the oracle's own code:
  * torch.optim.AdamW / torch.optim.Adam with amsgrad=True (foreach=False)
    on the CPU in fp32, for the oracle's fp32-moment mode, on gradients that
    shrink so that the running maximum and v part ways;
  * the first step from a zero state: the maximum equals v, so AMSGrad
    reproduces the plain step (pinned in test_oracle_adam.py) bit for bit;
  * PyTorch's header-only Philox engine for the maximum's own draws;
  * every 8-bit step of a 6-step run composed from pinned parts: the
    dequantized state (m, v and the maximum) fed to torch AdamW with
    amsgrad, then brute-force nearest codes of the new maximum (or, under
    stochastic rounding, the codes its pinned draws give).
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
U = 2.0 ** -24
# beta2 = 0.9: v follows the shrinking gradients within a few steps, so the
# running maximum parts from it early
HP = dict(lr=1e-3, beta1=0.9, beta2=0.9, eps=1e-8, weight_decay=0.01)
HP32 = {k: float(np.float32(v)) for k, v in HP.items()}


def _tol(p_ref, p0, steps, lr):
    scale = np.maximum(np.abs(p_ref.astype(np.float64)), np.abs(p0.astype(np.float64)))
    return steps * (2 * U * scale + 16 * U * lr)


def _shrinking_grads(seed, n, steps):
    # the gradient scale falls by 30% a step, so v decays below its maximum
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(n) * 0.7 ** t).astype(np.float32) for t in range(steps)]


@pytest.mark.parametrize("decoupled", [True, False])
def test_fp32_mode_matches_torch_amsgrad(orc, decoupled):
    n, steps = 3000, 12
    p0 = workloads.host_params(301, [n])[0]
    gs = _shrinking_grads(301, n, steps)
    tp = torch.tensor(p0.copy(), requires_grad=True)
    cls = torch.optim.AdamW if decoupled else torch.optim.Adam
    opt = cls([tp], lr=HP32["lr"], betas=(HP32["beta1"], HP32["beta2"]), eps=HP32["eps"],
              weight_decay=HP32["weight_decay"], amsgrad=True, foreach=False)
    st = orc.OracleState([n], "f32", amsgrad=True)
    plain = orc.OracleState([n], "f32")
    pp, pq = [p0.copy()], [p0.copy()]
    for t, g in enumerate(gs, start=1):
        tp.grad = torch.tensor(g)
        opt.step()
        st.step(pp, [g], t=t, decoupled=decoupled, **HP)
        plain.step(pq, [g], t=t, decoupled=decoupled, **HP)
    want = tp.detach().numpy()
    assert np.all(np.abs(pp[0].astype(np.float64) - want) <= _tol(want, p0, steps, HP["lr"]))
    tw = opt.state[tp]["max_exp_avg_sq"].numpy()
    assert np.max(np.abs(st.vmax_f32[:n] - tw)) <= 1e-6 * np.abs(tw).max()
    # the maximum really parted from v, and the parameters with it
    assert np.mean(st.vmax_f32[:n] > st.v_f32[:n]) > 0.9
    assert np.max(np.abs(pp[0] - pq[0])) > 100 * np.max(_tol(want, p0, steps, HP["lr"]))


@pytest.mark.parametrize("storage", ["f32", "bf16", "q8", "q8_v_only"])
@pytest.mark.parametrize("grad_bf16", [False, True])
def test_first_step_equals_the_plain_step(orc, storage, grad_bf16):
    numels = workloads.numels_of(workloads.ragged_shapes())
    p0 = workloads.host_params(302, numels)
    g = workloads.host_grads(302, numels, 1, dtype="bf16" if grad_bf16 else "f32")
    a = orc.OracleState(numels, storage, grad_bf16=grad_bf16, amsgrad=True)
    b = orc.OracleState(numels, storage, grad_bf16=grad_bf16)
    pa = [p.copy() for p in p0]
    pb = [p.copy() for p in p0]
    a.step(pa, g, t=1, **HP)
    b.step(pb, g, t=1, **HP)
    for x, y in zip(pa, pb):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    for k, v in b.buffers().items():
        assert np.array_equal(a.buffers()[k], v), k
    # with nearest rounding the maximum is stored exactly as v is
    src = {"f32": ("vmax_f32", "v_f32"), "bf16": ("vmax_bf16", "v_bf16")}.get(
        storage, ("vmax_codes", "v_codes"))
    assert np.array_equal(getattr(a, src[0]), getattr(a, src[1]))
    if storage in ("q8", "q8_v_only"):
        assert np.array_equal(a.vmax_scale, a.v_scale)


@pytest.fixture(scope="module")
def philox_ref(tmp_path_factory):
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc,
                    os.path.join(HERE, "philox_ref.cpp"), "-o", exe], check=True)

    def run(triples):
        inp = "".join(f"{s} {u} {o}\n" for s, u, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
        return np.array([[int(w, 16) for w in line.split()] for line in
                         out.stdout.strip().splitlines()], dtype=np.uint32)

    return run


def test_maximum_draws_use_the_second_counter_stream(orc, philox_ref):
    # element i at step t: half (i mod 2) of word ((i/2) mod 4) of
    # philox(seed, subsequence=t, offset=i/8 + 2^63): one call per 8 elements
    for seed, t, gidx0 in [(42, 1, 0), (1234, 5, 2 ** 33 + 12), (7, 3, 2046)]:
        n = 40
        idx = np.arange(gidx0, gidx0 + n, dtype=np.uint64)
        groups = sorted(set(int(i) >> 3 for i in idx))
        words = dict(zip(groups, philox_ref([(seed, t, g + 2 ** 63) for g in groups])))
        got = orc.sr_draws(seed, t, gidx0, n, 2)
        for j, i in enumerate(idx):
            i = int(i)
            assert got[j] == (int(words[i >> 3][(i >> 1) & 3]) >> (16 * (i & 1))) & 0xFFFF
        # and it is not the first stream's, in either half
        assert not np.array_equal(got, orc.sr_draws(seed, t, gidx0, n, 0))
        assert not np.array_equal(got, orc.sr_draws(seed, t, gidx0, n, 1))


@pytest.mark.parametrize("storage", ["q8", "q8_v_only"])
@pytest.mark.parametrize("stochastic", [False, True])
def test_every_quantized_step_composes_pinned_parts(orc, storage, stochastic):
    # every step of a 6-step run, each from the state the oracle holds
    # before it: decoded, one torch AdamW(amsgrad=True) step, the running
    # maximum re-encoded by the pinned rules
    n = 2048 * 2 + 700
    p = workloads.host_params(303, [n])[0]
    gs = _shrinking_grads(303, n, 6)
    st = orc.OracleState([n], storage, amsgrad=True)
    pp = [p.copy()]
    blocks = [(0, 2048), (2048, 4096), (4096, n)]
    alphabet = np.arange(0, 256)
    for t in range(1, 7):
        g = gs[t - 1]
        deq = {k: np.empty(n, np.float32) for k in ("m", "v", "w")}
        for b, (s, e) in enumerate(blocks):
            if storage == "q8":
                deq["m"][s:e] = orc.dequantize_block(st.m_codes[s:e], True, float(st.m_scale[b]))
            else:
                deq["m"][s:e] = st.m_f32[s:e]
            deq["v"][s:e] = orc.dequantize_block(st.v_codes[s:e], False, float(st.v_scale[b]))
            deq["w"][s:e] = orc.dequantize_block(st.vmax_codes[s:e], False,
                                                 float(st.vmax_scale[b]))
        tp = torch.tensor(pp[0].copy(), requires_grad=True)
        opt = torch.optim.AdamW([tp], lr=HP32["lr"], betas=(HP32["beta1"], HP32["beta2"]),
                                eps=HP32["eps"], weight_decay=HP32["weight_decay"], amsgrad=True,
                                foreach=False)
        opt.state[tp] = {"step": torch.tensor(float(t - 1)), "exp_avg": torch.tensor(deq["m"]),
                         "exp_avg_sq": torch.tensor(deq["v"]),
                         "max_exp_avg_sq": torch.tensor(deq["w"])}
        tp.grad = torch.tensor(g)
        opt.step()
        p_before = pp[0].copy()
        m_new, v_new, w_new = (a[:n] for a in st.step(pp, [g], t=t, stochastic=stochastic, seed=9,
                                                        want_moments=True, **HP))
        want = tp.detach().numpy().astype(np.float64)
        # a few roundings of |p| and of the update itself
        tol = _tol(want, p_before, 1, HP["lr"]) + 8 * U * np.abs(want - p_before.astype(np.float64))
        assert np.all(np.abs(pp[0].astype(np.float64) - want) <= tol), t
        tw = opt.state[tp]["max_exp_avg_sq"].numpy()
        assert np.max(np.abs(w_new - tw)) <= 1e-6 * np.abs(tw).max(), t
        assert np.all(w_new >= v_new), t
        for b, (s, e) in enumerate(blocks):
            A = st.vmax_scale[b]
            assert A == w_new[s:e].max(), t
            codes = st.vmax_codes[s:e].astype(np.int64)
            vals = orc.dequantize_block(alphabet, False, float(A)).astype(np.float64)
            dist = np.abs(vals[None, :] - w_new[s:e].astype(np.float64)[:, None])
            if stochastic:
                # one of the two codes around the value, from the maximum's draws
                lo = np.floor(w_new[s:e].astype(np.float64) * 255 / float(A))
                assert np.all((codes >= lo - 1) & (codes <= lo + 2)), t
                draws = orc.sr_draws(9, t, s, e - s, 2)
                want_codes, _ = orc.quantize_with_stat(w_new[s:e], False, float(A), draws)
                assert np.array_equal(codes, want_codes), t
            else:
                chosen = dist[np.arange(e - s), codes]
                assert np.all(chosen <= dist.min(axis=1) + 4 * U * float(A)), t
    # the shrinking gradients leave the maximum above v for most elements
    assert np.mean(w_new > v_new) > 0.5
