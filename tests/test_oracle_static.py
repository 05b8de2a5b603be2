"""Pins for the oracle's static-scale mode of the 8-bit state.

The 8-bit Adam page's options class has a switch for dynamic quantization,
on by default, under which each block's scales follow the moments.  With the
switch off we read: a block's scale is set the first time the block is
quantized with a usable statistic (stored scale still 0) and then kept;
later moment values at or beyond it take the end code of the alphabet.

References used here, none of them the oracle's step code:
  * the first step from a zero state must equal the dynamic step, which is
    pinned in test_oracle_adam.py;
  * the stored scales must not move after they are set (a block whose first
    statistic is below the encodable range keeps scale 0 until a later step
    sets it);
  * codes of a later step are the nearest entries of the codebook scaled by
    the kept scale (brute-force search over all codes), so values beyond the
    scale saturate; with stochastic rounding they match the pinned quantizer
    fed the kept scale and the pinned draws;
  * the parameter update from that state matches torch.optim.AdamW fed the
    dequantized moments.
"""
import numpy as np
import pytest
import torch

import workloads

U = 2.0 ** -24
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
HP32 = {k: float(np.float32(v)) for k, v in HP.items()}
SEED = 77


def _buffers(st):
    return {k: getattr(st, k).copy() for k in ("m_f32", "m_codes", "v_codes", "m_scale",
                                                "v_scale") if getattr(st, k) is not None}


def _blocks(numels):
    """(segment start, block start, block end, block index) in state order."""
    out, seg, b = [], 0, 0
    for n in numels:
        for s in range(0, n, 2048):
            out.append((seg, s, min(n, s + 2048), b))
            b += 1
        seg += (n + 15) // 16 * 16
    return out


@pytest.mark.parametrize("storage", ["q8", "q8_v_only"])
@pytest.mark.parametrize("stochastic", [False, True])
@pytest.mark.parametrize("percentile", [None, 99.9])
def test_first_step_equals_the_dynamic_step(orc, storage, stochastic, percentile):
    numels = workloads.numels_of(workloads.ragged_shapes())
    p0 = workloads.host_params(201, numels)
    g = workloads.host_grads(201, numels, 1)
    out = []
    for static in (False, True):
        st = orc.OracleState(numels, storage)
        pp = [p.copy() for p in p0]
        st.step(pp, g, t=1, stochastic=stochastic, percentile=percentile, seed=SEED,
                static_scales=static, **HP)
        out.append((pp, _buffers(st)))
    (pd, bd), (ps, bs) = out
    for a, b in zip(pd, ps):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for k in bd:
        assert np.array_equal(bd[k], bs[k]), k


@pytest.mark.parametrize("storage", ["q8", "q8_v_only"])
@pytest.mark.parametrize("percentile", [None, 99.9])
def test_scales_are_kept_once_set(orc, storage, percentile):
    numels = [3000, 17, 2048, 5000]
    p0 = workloads.host_params(202, numels)
    st = orc.OracleState(numels, storage)
    pp = [p.copy() for p in p0]
    first = None
    for t in range(1, 7):
        g = workloads.host_grads(202, numels, t)
        if t <= 2:
            g[1] = np.zeros_like(g[1])  # tensor 1's block stays unscaled for two steps
        st.step(pp, g, t=t, percentile=percentile, static_scales=True, **HP)
        if t == 1:
            first = (None if st.m_scale is None else st.m_scale.copy(), st.v_scale.copy())
            assert first[1][2] == 0.0 and np.all(np.delete(first[1], 2) > 0)
        elif t <= 2:
            assert st.v_scale[2] == 0.0
        else:
            assert st.v_scale[2] > 0.0
        keep = np.arange(st.v_scale.size) != 2
        assert np.array_equal(st.v_scale[keep], first[1][keep])
        if first[0] is not None:
            assert np.array_equal(st.m_scale[keep], first[0][keep])
        if t == 3:
            tensor1 = (st.m_scale[2] if st.m_scale is not None else None, st.v_scale[2])
        if t > 3:
            assert st.v_scale[2] == tensor1[1]
            if tensor1[0] is not None:
                assert st.m_scale[2] == tensor1[0]


def _nearest_ok(orc, x, codes, A, signed):
    qmax = 127 if signed else 255
    alphabet = np.arange(-qmax if signed else 0, qmax + 1)
    vals = orc.dequantize_block(alphabet, signed, float(A)).astype(np.float64)
    dist = np.abs(vals[None, :] - x.astype(np.float64)[:, None])
    chosen = dist[np.arange(x.size), codes.astype(np.int64) - alphabet[0]]
    return np.all(chosen <= dist.min(axis=1) + 4 * U * float(A))


@pytest.mark.parametrize("storage", ["q8", "q8_v_only"])
def test_later_codes_are_nearest_with_the_kept_scale(orc, storage):
    n = 2048 * 3 + 700
    p = workloads.host_params(203, [n])[0]
    st = orc.OracleState([n], storage)
    pp = [p.copy()]
    for t in range(1, 5):
        st.step(pp, workloads.host_grads(203, [n], t), t=t, static_scales=True, **HP)
    kept = _buffers(st)
    t = 5
    g = workloads.host_grads(203, [n], t)[0]
    blocks = [(0, 2048), (2048, 4096), (4096, 6144), (6144, n)]
    m_old = np.empty(n, np.float32)
    v_old = np.empty(n, np.float32)
    for b, (s, e) in enumerate(blocks):
        if storage == "q8":
            m_old[s:e] = orc.dequantize_block(kept["m_codes"][s:e], True, float(kept["m_scale"][b]))
        else:
            m_old[s:e] = kept["m_f32"][s:e]
        v_old[s:e] = orc.dequantize_block(kept["v_codes"][s:e], False, float(kept["v_scale"][b]))
    tp = torch.tensor(pp[0].copy(), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=HP32["lr"], betas=(HP32["beta1"], HP32["beta2"]),
                            eps=HP32["eps"], weight_decay=HP32["weight_decay"], foreach=False)
    opt.state[tp] = {"step": torch.tensor(float(t - 1)),
                     "exp_avg": torch.tensor(m_old), "exp_avg_sq": torch.tensor(v_old)}
    tp.grad = torch.tensor(g)
    opt.step()
    m_new, v_new = st.step(pp, [g], t=t, static_scales=True, want_moments=True, **HP)
    m_new, v_new = m_new[:n], v_new[:n]
    want = tp.detach().numpy().astype(np.float64)
    scale = np.maximum(np.abs(want), np.abs(p.astype(np.float64)))
    assert np.all(np.abs(pp[0] - want) <= 2 * U * scale + 16 * U * HP["lr"])
    saturated = 0
    for b, (s, e) in enumerate(blocks):
        A = kept["v_scale"][b]
        assert st.v_scale[b] == A
        assert _nearest_ok(orc, v_new[s:e], st.v_codes[s:e], A, False)
        saturated += int(np.sum(v_new[s:e] >= A))
        assert np.all(st.v_codes[s:e][v_new[s:e] >= A] == 255)
        if storage == "q8":
            A = kept["m_scale"][b]
            assert st.m_scale[b] == A
            assert _nearest_ok(orc, m_new[s:e], st.m_codes[s:e], A, True)
            big = np.abs(m_new[s:e]) >= A
            assert np.all(st.m_codes[s:e][big] == np.where(m_new[s:e][big] < 0, -127, 127))
        else:
            assert np.array_equal(st.m_f32[s:e], m_new[s:e])
    # the second moment grows from its first value, so the kept scale clips
    assert saturated > 0


def test_stochastic_codes_use_the_kept_scale_and_the_draws(orc):
    numels = [2048 + 300, 17]
    p0 = workloads.host_params(204, numels)
    st = orc.OracleState(numels, "q8")
    pp = [p.copy() for p in p0]
    for t in range(1, 4):
        st.step(pp, workloads.host_grads(204, numels, t), t=t, stochastic=True, seed=SEED,
                static_scales=True, **HP)
    kept = _buffers(st)
    t = 4
    m_new, v_new = st.step(pp, workloads.host_grads(204, numels, t), t=t, stochastic=True,
                           seed=SEED, static_scales=True, want_moments=True, **HP)
    for seg, s, e, b in _blocks(numels):
        gidx = seg + s
        dm = orc.sr_draws(SEED, t, gidx, e - s, 0)
        dv = orc.sr_draws(SEED, t, gidx, e - s, 1)
        cm, Am = orc.quantize_with_stat(m_new[gidx:seg + e], True, float(kept["m_scale"][b]), dm)
        cv, Av = orc.quantize_with_stat(v_new[gidx:seg + e], False, float(kept["v_scale"][b]), dv)
        assert Am == st.m_scale[b] == kept["m_scale"][b]
        assert Av == st.v_scale[b] == kept["v_scale"][b]
        assert np.array_equal(cm, st.m_codes[gidx:seg + e].astype(np.int32))
        assert np.array_equal(cv, st.v_codes[gidx:seg + e].astype(np.int32))
