"""Pins for the oracle's Adam/AdamW step.

References used here, none of them the oracle's own code:
  * the t=1 closed form (from a zero state the bias-corrected moments are g
    and g^2, so the update is lr*g/(|g|+eps)), evaluated in fp64;
  * g = 0 (the step reduces to the weight decay alone) and lr = 0;
  * torch.optim.AdamW / torch.optim.Adam (foreach=False) on the CPU in fp32,
    and a textbook fp64 Adam, for the oracle's fp32-moment mode;
  * one 8-bit step from a non-zero state composed from pinned parts: the
    dequantized state fed to torch.optim.AdamW, then brute-force nearest
    codes of the new moments; the same check on every step of 8-step
    trajectories (bf16, 8-bit and fp32-m modes, nearest and stochastic
    rounding);
  * structural invariants (code ranges, exact block maxima, tensor-order
    permutation, per-tensor independence).
"""
import numpy as np
import pytest
import torch

import workloads

U = 2.0 ** -24
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
f32 = np.float32
# the step takes its hyperparameters as fp32; torch gets the same values
HP32 = {k: float(np.float32(v)) for k, v in HP.items()}


def _f(x):
    return float(np.float32(x))


def _trajectory_tol(p_ref, p0, steps, lr):
    # two fp32 evaluations of the same steps in different operation orders
    # drift apart by a few roundings of |p| and of the update (~lr) per step
    scale = np.maximum(np.abs(p_ref.astype(np.float64)), np.abs(p0.astype(np.float64)))
    return steps * (2 * U * scale + 16 * U * lr)


def _fresh(orc, numels, storage, grad_bf16=False):
    return orc.OracleState(numels, storage, grad_bf16=grad_bf16)


def _closed_form_t1(p, g, decoupled, lr, eps, wd):
    p64 = p.astype(np.float64)
    g64 = g.astype(np.float64)
    lr64, eps64, wd64 = float(f32(lr)), float(f32(eps)), float(f32(wd))
    if decoupled:
        decay = float(f32(1.0 - lr64 * wd64))
        upd = lr64 * g64 / (np.abs(g64) + eps64)
        return p64 * decay - upd, upd, p64 * decay
    g2 = g64 + wd64 * p64
    upd = lr64 * g2 / (np.abs(g2) + eps64)
    return p64 - upd, upd, p64


@pytest.mark.parametrize("storage", ["f32", "bf16", "q8", "q8_v_only"])
@pytest.mark.parametrize("decoupled", [True, False])
@pytest.mark.parametrize("grad_bf16", [False, True])
def test_first_step_closed_form(orc, storage, decoupled, grad_bf16):
    numels = workloads.numels_of(workloads.ragged_shapes())
    params = workloads.host_params(101, numels)
    grads = workloads.host_grads(101, numels, 1, dtype="bf16" if grad_bf16 else "f32")
    st = _fresh(orc, numels, storage, grad_bf16)
    p0 = [p.copy() for p in params]
    st.step(params, grads, t=1, decoupled=decoupled, stochastic=(storage == "q8"),
            percentile=99.9 if storage == "q8_v_only" else None, **HP)
    for k in range(len(numels)):
        g = grads[k]
        if grad_bf16:
            g = (g.astype(np.uint32) << 16).view(np.float32)
        want, upd, base = _closed_form_t1(p0[k], g, decoupled, HP["lr"], HP["eps"],
                                          HP["weight_decay"])
        got = params[k].astype(np.float64)
        tol = 8 * U * (np.abs(upd) + np.abs(base) + np.abs(got))
        assert np.all(np.abs(got - want) <= tol), k


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only", "f32"])
def test_zero_gradient_is_decay_only(orc, storage):
    numels = [5, 2048, 3000]
    params = workloads.host_params(102, numels)
    grads = [np.zeros(n, np.float32) for n in numels]
    st = _fresh(orc, numels, storage)
    p0 = [p.copy() for p in params]
    st.step(params, grads, t=1, **HP)
    decay = f32(1.0 - float(f32(HP["lr"])) * float(f32(HP["weight_decay"])))
    for k in range(len(numels)):
        assert np.array_equal(params[k], p0[k] * decay)
    for name, buf in st.buffers().items():
        assert not buf.any(), name
    # wd = 0: params unchanged
    st2 = _fresh(orc, numels, storage)
    p1 = [p.copy() for p in p0]
    st2.step(p1, grads, t=1, **dict(HP, weight_decay=0.0))
    for k in range(len(numels)):
        assert np.array_equal(p1[k], p0[k])


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only"])
def test_zero_learning_rate_keeps_params_moves_moments(orc, storage):
    numels = [100, 4100]
    params = workloads.host_params(103, numels)
    grads = workloads.host_grads(103, numels, 1)
    st = _fresh(orc, numels, storage)
    p0 = [p.copy() for p in params]
    m_new, v_new = st.step(params, grads, t=1, want_moments=True, **dict(HP, lr=0.0))
    for k in range(len(numels)):
        assert np.array_equal(params[k], p0[k])
    omb1 = f32(1.0 - float(f32(0.9)))
    g = np.concatenate([grads[0], np.zeros(12, np.float32), grads[1],
                        np.zeros(12, np.float32)])
    assert np.array_equal(m_new, omb1 * g)
    assert np.all(v_new >= 0) and v_new.max() > 0


def _torch_run(params0, grads_seq, decoupled, **hp):
    p = torch.tensor(params0, dtype=torch.float32, requires_grad=True)
    cls = torch.optim.AdamW if decoupled else torch.optim.Adam
    hp = {k: float(np.float32(v)) for k, v in hp.items()}
    opt = cls([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
              weight_decay=hp["weight_decay"], foreach=False, fused=False)
    for g in grads_seq:
        p.grad = torch.tensor(g, dtype=torch.float32)
        opt.step()
    s = opt.state[p]
    return p.detach().numpy(), s["exp_avg"].numpy(), s["exp_avg_sq"].numpy()


@pytest.mark.parametrize("decoupled", [True, False])
def test_fp32_moment_mode_matches_torch_optim(orc, decoupled):
    n = 6001
    p = workloads.host_params(104, [n])[0]
    gs = [workloads.host_grads(104, [n], t)[0] for t in range(1, 11)]
    tp, tm, tv = _torch_run(p.copy(), gs, decoupled, **HP)
    st = _fresh(orc, [n], "f32")
    pp = [p.copy()]
    for t, g in enumerate(gs, start=1):
        st.step(pp, [g], t=t, decoupled=decoupled, **HP)
    assert np.all(np.abs(pp[0].astype(np.float64) - tp) <= _trajectory_tol(tp, p, 10, HP["lr"]))
    # moments: m changes sign (cancels), so compare at the array's scale
    assert np.max(np.abs(st.m_f32[:n] - tm)) <= 1e-6 * np.abs(tm).max()
    assert np.max(np.abs(st.v_f32[:n] - tv) / tv) <= 1e-5


def test_fp32_moment_mode_matches_fp64_textbook_adam(orc):
    n = 4096
    p = workloads.host_params(105, [n])[0]
    gs = [workloads.host_grads(105, [n], t)[0] for t in range(1, 11)]
    lr, b1, b2, eps, wd = (float(f32(HP[k])) for k in
                           ("lr", "beta1", "beta2", "eps", "weight_decay"))
    x = p.astype(np.float64)
    m = np.zeros(n)
    v = np.zeros(n)
    for t, g in enumerate(gs, start=1):
        g = g.astype(np.float64)
        x = x * (1 - lr * wd)
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh = m / (1 - b1 ** t)
        vh = v / (1 - b2 ** t)
        x = x - lr * mh / (np.sqrt(vh) + eps)
    st = _fresh(orc, [n], "f32")
    pp = [p.copy()]
    for t, g in enumerate(gs, start=1):
        st.step(pp, [g], t=t, **HP)
    assert np.all(np.abs(pp[0] - x) <= _trajectory_tol(x, p, 10, HP["lr"]))


@pytest.mark.parametrize("storage", ["q8", "q8_v_only"])
def test_one_quantized_step_composes_pinned_parts(orc, storage):
    # Build a non-zero compressed state with a few oracle steps, then check
    # the next step against (dequantized state -> torch AdamW -> nearest code).
    n = 2048 * 3 + 700
    p = workloads.host_params(106, [n])[0]
    st = _fresh(orc, [n], storage)
    pp = [p.copy()]
    for t in range(1, 5):
        st.step(pp, workloads.host_grads(106, [n], t), t=t, **HP)
    t = 5
    g = workloads.host_grads(106, [n], t)[0]
    blocks = [(0, 2048), (2048, 4096), (4096, 6144), (6144, n)]
    m_old = np.empty(n, np.float32)
    v_old = np.empty(n, np.float32)
    for b, (s, e) in enumerate(blocks):
        if storage == "q8":
            m_old[s:e] = orc.dequantize_block(st.m_codes[s:e], True, float(st.m_scale[b]))
        else:
            m_old[s:e] = st.m_f32[s:e]
        v_old[s:e] = orc.dequantize_block(st.v_codes[s:e], False, float(st.v_scale[b]))
    tp = torch.tensor(pp[0].copy(), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=HP32["lr"], betas=(HP32["beta1"], HP32["beta2"]),
                            eps=HP32["eps"], weight_decay=HP32["weight_decay"], foreach=False)
    opt.state[tp] = {"step": torch.tensor(float(t - 1)),
                     "exp_avg": torch.tensor(m_old), "exp_avg_sq": torch.tensor(v_old)}
    tp.grad = torch.tensor(g)
    opt.step()
    m_new, v_new = st.step(pp, [g], t=t, want_moments=True, **HP)
    m_new, v_new = m_new[:n], v_new[:n]
    want_p = tp.detach().numpy()
    assert np.all(np.abs(pp[0].astype(np.float64) - want_p) <=
                  _trajectory_tol(want_p, pp[0], 1, HP["lr"]))
    tm = opt.state[tp]["exp_avg"].numpy()
    tv = opt.state[tp]["exp_avg_sq"].numpy()
    assert np.max(np.abs(m_new - tm)) <= 1e-6 * np.abs(tm).max()
    assert np.max(np.abs(v_new - tv)) <= 1e-6 * np.abs(tv).max()
    # stored scales are the exact block maxima; codes are nearest in alphabet
    for b, (s, e) in enumerate(blocks):
        checks = [(v_new[s:e], st.v_codes[s:e].astype(np.int64), st.v_scale[b], False)]
        if storage == "q8":
            checks.append((m_new[s:e], st.m_codes[s:e].astype(np.int64), st.m_scale[b], True))
        else:
            assert np.array_equal(st.m_f32[s:e], m_new[s:e])
        for x, codes, A, signed in checks:
            assert A == np.abs(x).max()
            qmax = 127 if signed else 255
            alphabet = np.arange(-qmax if signed else 0, qmax + 1)
            vals = orc.dequantize_block(alphabet, signed, float(A)).astype(np.float64)
            dist = np.abs(vals[None, :] - x.astype(np.float64)[:, None])
            chosen = dist[np.arange(x.size), codes - alphabet[0]]
            assert np.all(chosen <= dist.min(axis=1) + 4 * U * float(A))


def _decoded_state(orc, st, n, blocks):
    """The oracle's stored moments of a one-tensor state, decoded to fp32."""
    if st.storage == "bf16":
        return (orc.f32_from_bf16(st.m_bf16[:n]).astype(np.float32),
                orc.f32_from_bf16(st.v_bf16[:n]).astype(np.float32))
    m = np.empty(n, np.float32)
    v = np.empty(n, np.float32)
    for b, (s, e) in enumerate(blocks):
        if st.storage == "q8":
            m[s:e] = orc.dequantize_block(st.m_codes[s:e], True, float(st.m_scale[b]))
        else:
            m[s:e] = st.m_f32[s:e]
        v[s:e] = orc.dequantize_block(st.v_codes[s:e], False, float(st.v_scale[b]))
    return m, v


@pytest.mark.parametrize("storage,stochastic", [("bf16", False), ("q8", False), ("q8", True),
                                                ("q8_v_only", False), ("q8_v_only", True)])
def test_every_step_of_a_trajectory_composes_pinned_parts(orc, storage, stochastic):
    # Eight steps from a zero state; each one checked from the state the
    # oracle actually holds before it: that state decoded, one
    # torch.optim.AdamW step, and the stored result re-encoded by the pinned
    # rules (bf16: PyTorch's cast; 8-bit: the block maximum as scale and the
    # nearest code of the whole alphabet by brute force, or under stochastic
    # rounding a code whose value lies within one step of the moment).  So
    # every step of a multi-step trajectory is pinned, not only the first.
    n = 2048 * 2 + 700
    blocks = [(0, 2048), (2048, 4096), (4096, n)]
    p0 = workloads.host_params(108, [n])[0]
    st = _fresh(orc, [n], storage)
    pp = [p0.copy()]
    for t in range(1, 9):
        g = workloads.host_grads(108, [n], t)[0]
        m_old, v_old = _decoded_state(orc, st, n, blocks)
        tp = torch.tensor(pp[0].copy(), requires_grad=True)
        opt = torch.optim.AdamW([tp], lr=HP32["lr"], betas=(HP32["beta1"], HP32["beta2"]),
                                eps=HP32["eps"], weight_decay=HP32["weight_decay"], foreach=False)
        opt.state[tp] = {"step": torch.tensor(float(t - 1)),
                         "exp_avg": torch.tensor(m_old), "exp_avg_sq": torch.tensor(v_old)}
        tp.grad = torch.tensor(g)
        opt.step()
        p_before = pp[0].copy()
        m_new, v_new = st.step(pp, [g], t=t, stochastic=stochastic, seed=9, want_moments=True, **HP)
        m_new, v_new = m_new[:n], v_new[:n]
        want_p = tp.detach().numpy().astype(np.float64)
        # the two fp32 evaluations differ by a few roundings of |p| and of
        # the update itself (which can exceed lr where a decoded v is 0 and
        # the fp32 first moment is not)
        upd = np.abs(want_p - p_before.astype(np.float64))
        tol = _trajectory_tol(want_p, p_before, 1, HP["lr"]) + 8 * U * upd
        assert np.all(np.abs(pp[0].astype(np.float64) - want_p) <= tol), t
        tm = opt.state[tp]["exp_avg"].numpy()
        tv = opt.state[tp]["exp_avg_sq"].numpy()
        assert np.max(np.abs(m_new - tm)) <= 1e-6 * np.abs(tm).max(), t
        assert np.max(np.abs(v_new - tv)) <= 1e-6 * np.abs(tv).max(), t
        if storage == "bf16":
            for x, h in ((m_new, st.m_bf16[:n]), (v_new, st.v_bf16[:n])):
                want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(h, want), t
            continue
        for b, (s, e) in enumerate(blocks):
            checks = [(v_new[s:e], st.v_codes[s:e].astype(np.int64), st.v_scale[b], False)]
            if storage == "q8":
                checks.append((m_new[s:e], st.m_codes[s:e].astype(np.int64), st.m_scale[b], True))
            else:
                assert np.array_equal(st.m_f32[s:e], m_new[s:e]), t
            for x, codes, A, signed in checks:
                assert A == np.abs(x).max(), t
                qmax = 127 if signed else 255
                if stochastic:
                    got = orc.dequantize_block(codes, signed, float(A)).astype(np.float64)
                    assert np.all(np.abs(got - x.astype(np.float64)) <= float(A) / qmax * (1 + 8 * U)), t
                    continue
                alphabet = np.arange(-qmax if signed else 0, qmax + 1)
                vals = orc.dequantize_block(alphabet, signed, float(A)).astype(np.float64)
                dist = np.abs(vals[None, :] - x.astype(np.float64)[:, None])
                chosen = dist[np.arange(x.size), codes - alphabet[0]]
                assert np.all(chosen <= dist.min(axis=1) + 4 * U * float(A)), t


@pytest.mark.parametrize("stochastic", [False, True])
def test_state_invariants_over_steps(orc, stochastic):
    numels = workloads.numels_of(workloads.ragged_shapes())
    params = workloads.host_params(107, numels)
    st = _fresh(orc, numels, "q8")
    for t in range(1, 6):
        m_new, v_new = st.step(params, workloads.host_grads(107, numels, t), t=t,
                               stochastic=stochastic, want_moments=True, **HP)
        assert st.m_codes.min() >= -127 and st.v_codes.max() <= 255
        assert np.all(st.m_scale >= 0) and np.all(st.v_scale >= 0)
        b = 0
        seg = 0
        for n in numels:
            for s in range(0, n, 2048):
                e = min(n, s + 2048)
                assert st.m_scale[b] == np.abs(m_new[seg + s:seg + e]).max()
                assert st.v_scale[b] == v_new[seg + s:seg + e].max()
                b += 1
            # padding stays untouched (zero)
            pad = orc.pad16(n)
            assert not st.m_codes[seg + n:seg + pad].any()
            assert not st.v_codes[seg + n:seg + pad].any()
            seg += pad


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only"])
def test_tensor_order_permutes_results(orc, storage):
    numels = [3000, 17, 2048, 5000]
    params = workloads.host_params(108, numels)
    grads = [workloads.host_grads(108, numels, t) for t in (1, 2, 3)]
    perm = [2, 0, 3, 1]
    pa = [p.copy() for p in params]
    pb = [params[i].copy() for i in perm]
    sa = _fresh(orc, numels, storage)
    sb = _fresh(orc, [numels[i] for i in perm], storage)
    for t in (1, 2, 3):
        sa.step(pa, grads[t - 1], t=t, **HP)
        sb.step(pb, [grads[t - 1][i] for i in perm], t=t, **HP)
    for j, i in enumerate(perm):
        assert np.array_equal(pa[i], pb[j])


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only"])
def test_multi_tensor_equals_separate_tensors(orc, storage):
    numels = [4097, 1, 2048]
    params = workloads.host_params(109, numels)
    grads = workloads.host_grads(109, numels, 1)
    together = [p.copy() for p in params]
    st = _fresh(orc, numels, storage)
    st.step(together, grads, t=1, **HP)
    for k, n in enumerate(numels):
        alone = [params[k].copy()]
        s1 = _fresh(orc, [n], storage)
        s1.step(alone, [grads[k]], t=1, **HP)
        assert np.array_equal(alone[0], together[k])


def test_block_sample_api_matches_full_step(orc):
    numels = [5000, 2048, 77]
    params = workloads.host_params(110, numels)
    st = _fresh(orc, numels, "q8", grad_bf16=True)
    full = [p.copy() for p in params]
    # blocks: (tensor, local start, n, gidx)
    blocks = []
    seg = 0
    for k, n in enumerate(numels):
        for s in range(0, n, 2048):
            blocks.append((k, s, min(2048, n - s), seg + s))
        seg += orc.pad16(n)
    ob = orc.OracleBlocks([(b[2], b[3]) for b in blocks], "q8", grad_bf16=True)
    sample = [params[k][s:s + n].copy() for k, s, n, _ in blocks]
    for t in (1, 2, 3):
        grads = workloads.host_grads(110, numels, t, dtype="bf16")
        st.step(full, grads, t=t, stochastic=True, seed=1234, **HP)
        ob.step(sample, [grads[k][s:s + n].copy() for k, s, n, _ in blocks], t=t,
                stochastic=True, seed=1234, **HP)
    for i, (k, s, n, gidx) in enumerate(blocks):
        assert np.array_equal(sample[i], full[k][s:s + n])
        sl = ob.block_slice(i)
        assert np.array_equal(ob.inner.m_codes[sl], st.m_codes[gidx:gidx + n])
        assert ob.inner.v_scale[i] == st.v_scale[i]


def test_host_scalars_at_t1(orc):
    s = orc.host_scalars(1e-3, 0.9, 0.999, 0.01, 1, True)
    # at t = 1, 1 - beta^t equals 1 - beta, so step = lr / (1 - beta1)
    assert s[0] == f32(float(f32(1e-3)) / (1.0 - float(f32(0.9))))
    assert s[3] == f32(1.0) - f32(0.9) and s[4] == f32(1.0) - f32(0.999)
    s_big = orc.host_scalars(1e-3, 0.9, 0.999, 0.01, 10 ** 9, False)
    assert s_big[0] == f32(1e-3) and s_big[1] == f32(1.0) and s_big[2] == f32(1.0)
