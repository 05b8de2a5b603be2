"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every test runs the library's kernels on the same seeded inputs the oracle
gets and compares element by element (criteria in tests/parity.py):
  * every storage mode x grad dtype x rounding x statistic on a ragged
    multi-tensor set (16 tensors from 1 to 12289 elements: several blocks,
    every tail shape), 10 steps, checked after every step;
  * the 1,048,576-parameter single tensor (8-bit, nearest-even), 10 steps;
  * the full-size ViT-Base, GPT-1.3B and Llama-7B shaped sets in the
    benchmark's launch configuration, on a sample of blocks that includes
    every tail block;
  * static scales (kept once set) on the ragged set, mixed with dynamic
    steps, and on the full-size Llama-7B set;
  * ZeRO-1 shard states (block-aligned slices, draw indices set) against one
    state over the whole set, bit for bit;
  * AMSGrad (running maximum of v) in every storage mode on the ragged set,
    on the full-size GPT-1.3B set with stochastic rounding, and through a
    checkpoint;
  * the percentile statistic's two paths (top walks, radix select): tied
    moments, outliers, a wave's largest values in one lane (short lane
    lists run empty), and percentiles either side of the switch;
  * seeded random configurations (mode, flags, percentile, hyperparameters,
    start step, ragged lists, gradient law);
  * edge cases: empty lists and zero-size tensors, a 2^32-1 element tensor,
    injected non-zero states, degenerate hyperparameters, pointer changes,
    a side stream, a refused step under graph capture, and the error paths.
"""
import ctypes
import dataclasses
import sys

import numpy as np
import pytest
import torch

import memory_efficient_adam_amd as ma
import oracle
import workloads
from parity import (Stats, compare_buffer, compare_params, read_state, run_full_parity,
                    run_sampled_parity, to_device_grads)

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
RAGGED = workloads.numels_of(workloads.ragged_shapes())


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


MODES = [
    # storage, grad dtype, stochastic, percentile, decoupled
    ("bf16", "f32", False, None, True),
    ("bf16", "bf16", False, None, True),
    ("bf16", "f32", False, None, False),
    ("q8", "f32", False, None, True),
    ("q8", "bf16", False, None, True),
    ("q8", "f32", True, None, True),
    ("q8", "bf16", True, None, True),
    ("q8", "f32", False, 99.9, True),
    ("q8", "bf16", True, 99.9, True),
    ("q8", "f32", False, None, False),
    ("q8", "f32", True, 50.0, False),
    ("q8", "f32", False, 0.0, True),
    ("q8", "f32", False, 100.0, True),
    ("q8_v_only", "f32", False, None, True),
    ("q8_v_only", "bf16", False, 99.9, True),
    ("q8_v_only", "bf16", True, 99.9, True),
    ("q8_v_only", "f32", True, None, False),
    ("q8_v_only", "bf16", True, None, True),
]


@pytest.mark.parametrize("storage,gdt,sr,pct,dec", MODES)
def test_ragged_set_every_mode(storage, gdt, sr, pct, dec):
    log(f"ragged {storage} grads={gdt} sr={sr} pct={pct} decoupled={dec}")
    hp = dict(HP, stochastic=sr, percentile=pct, decoupled=dec, seed=1234)
    for dist in ("normal", "student_t3"):
        stats = run_full_parity(RAGGED, storage, gdt, 10, hp, cfg_id=11, grad_dist=dist)
        log(f"  {dist}: {stats}")


STATIC_MODES = [
    # storage, grad dtype, stochastic, percentile
    ("q8", "f32", False, None),
    ("q8", "bf16", True, None),
    ("q8", "f32", False, 99.9),
    ("q8", "bf16", True, 99.9),
    ("q8_v_only", "f32", False, None),
    ("q8_v_only", "bf16", True, 99.9),
]


@pytest.mark.parametrize("storage,gdt,sr,pct", STATIC_MODES)
def test_ragged_set_static_scales(storage, gdt, sr, pct):
    log(f"ragged static scales {storage} grads={gdt} sr={sr} pct={pct}")
    hp = dict(HP, stochastic=sr, percentile=pct, static_scales=True, seed=99)
    for dist in ("normal", "student_t3"):
        stats = run_full_parity(RAGGED, storage, gdt, 10, hp, cfg_id=12, grad_dist=dist)
        log(f"  {dist}: {stats}")


@pytest.mark.parametrize("storage", ["q8", "q8_v_only"])
def test_static_scales_set_late_and_mixed_with_dynamic_steps(storage):
    # tensor 1 sees zero gradients for two steps (its blocks stay unscaled),
    # and static and dynamic steps alternate on one state
    numels = RAGGED
    log(f"static/dynamic mix {storage}")
    params = workloads.host_params(13, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, "f32")
    ost = oracle.OracleState(numels, storage)
    stats = Stats()
    for t, static in enumerate([True, True, True, False, True, True, False, False, True], start=1):
        grads = workloads.host_grads(13, numels, t)
        if t <= 2:
            grads[1] = np.zeros_like(grads[1])
        hp = dict(HP, static_scales=static, stochastic=(t % 3 == 0), seed=5)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, hp["stochastic"], stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


@pytest.mark.parametrize("ams", [False, True])
@pytest.mark.parametrize("pct", [99.0, 50.0])
def test_static_scales_radix_select_with_one_moment_kept(ams, pct):
    # the radix select runs the moments' selects side by side; with static
    # scales a block may keep one moment's scale while another still needs
    # its statistic: tiny gradients (1e-20) give tensor 1 a first-moment
    # scale at step 1 while its v underflows (no scale) until step 4, and
    # tensor 2 starts from zero gradients (no scale for either)
    numels = RAGGED
    log(f"static scales, radix percentile {pct}, one moment kept, amsgrad={ams}")
    params = workloads.host_params(16, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, "q8", "f32", amsgrad=ams)
    ost = oracle.OracleState(numels, "q8", amsgrad=ams)
    stats = Stats()
    for t in range(1, 7):
        grads = workloads.host_grads(16, numels, t)
        if t <= 3:
            grads[1] = (grads[1] * np.float32(1e-17)).astype(np.float32)
        if t <= 2:
            grads[2] = np.zeros_like(grads[2])
        hp = dict(HP, static_scales=True, percentile=pct, stochastic=(t % 2 == 0), seed=17)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, hp["stochastic"], stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


# percentiles whose full-block rank lands near the top: need = 2048 - rank
# keys at or above the statistic, with rank = floor(p/100 * 2047).  Up to
# need 4 the kernel walks down the top values, beyond it it takes the radix
# select; 2044.5 (need 4) and 2043.5 (need 5) sit on either side of that
# switch, 2032.5 and 2031.5 (need 16, 17) further into the radix select.
NEAR_TOP = [100.0, 99.9, 100.0 * 2044.5 / 2047, 100.0 * 2043.5 / 2047, 99.5,
            100.0 * 2032.5 / 2047, 100.0 * 2031.5 / 2047]


@pytest.mark.parametrize("pct", NEAR_TOP)
@pytest.mark.parametrize("storage,gdt,sr,ams", [("q8", "f32", False, False),
                                                ("q8", "bf16", True, True),
                                                ("q8_v_only", "f32", False, True)])
def test_percentile_near_the_top_with_ties(pct, storage, gdt, sr, ams):
    # gradients of five values tie the moments of a block in large groups,
    # so the top values come with counts far above need; the outlier set
    # puts a few isolated large values above the rest
    log(f"percentile {pct:.6f} {storage} grads={gdt} sr={sr} amsgrad={ams}")
    hp = dict(HP, beta2=0.9, stochastic=sr, percentile=pct, seed=5)
    for dist in ("few_levels", "normal_outliers"):
        stats = run_full_parity(RAGGED, storage, gdt, 4, hp, cfg_id=15, grad_dist=dist,
                                amsgrad=ams)
        log(f"  {dist}: {stats}")


def _far_below_grads(seed, numels, t):
    """Gradients whose moments put a block's low percentiles 15 or more
    binades below its maximum: per block a few values 1e8 times the rest,
    whole stretches of exact zeros (moments exactly 0), and values spread
    over 60 binades."""
    rng = np.random.default_rng([seed, t])
    out = []
    for n in numels:
        g = rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
        kind = rng.integers(0, 3, (n + 2047) // 2048)
        for b, k in enumerate(kind):
            blk = g[2048 * b:2048 * (b + 1)]
            if k == 0:
                blk[rng.integers(0, blk.size, 3)] *= np.float32(1e8)
            elif k == 1:
                blk[:blk.size * 2 // 3] = 0.0
            else:
                blk *= (np.float32(10.0) ** rng.uniform(-30, 0, blk.size)).astype(np.float32)
        out.append(g)
    return out


@pytest.mark.parametrize("pct", [0.0, 10.0, 50.0, 90.0, 99.0])
@pytest.mark.parametrize("storage,sr,ams", [("q8", False, False), ("q8", True, True),
                                            ("q8_v_only", False, True)])
def test_radix_select_far_below_the_maximum(pct, storage, sr, ams):
    # the radix select's coarse pass resolves the 15 binades under the block
    # maximum; an answer further down (exact zeros, tiny values) is found by
    # bisection on the key value: both paths against the oracle
    numels = RAGGED + [2048 * 6]
    log(f"radix select far below the maximum: percentile {pct} {storage} sr={sr} amsgrad={ams}")
    params = workloads.host_params(19, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, "f32", amsgrad=ams)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    stats = Stats()
    hp = dict(HP, beta2=0.9, stochastic=sr, percentile=pct, seed=23)
    for t in range(1, 4):
        grads = _far_below_grads(19, numels, t)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, sr, stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


def _sparse_grads(seed, numels, t):
    """Gradients that are zero except at 0-5 positions per block (the same
    positions every step, so the moments stay exactly zero elsewhere), with
    values over eight decades: the need-th largest key is then often 0, and
    the statistic falls back to the block maximum."""
    out = []
    for k, n in enumerate(numels):
        g = np.zeros(n, np.float32)
        for b in range((n + 2047) // 2048):
            lo, hi = 2048 * b, min(n, 2048 * (b + 1))
            pos_rng = np.random.default_rng([seed, k, b])
            nz = int(pos_rng.integers(0, 6))
            pos = lo + pos_rng.choice(hi - lo, min(nz, hi - lo), replace=False)
            val_rng = np.random.default_rng([seed, k, b, t])
            g[pos] = (val_rng.standard_normal(pos.size) *
                      10.0 ** val_rng.uniform(-6, 2, pos.size)).astype(np.float32)
        out.append(g)
    return out


@pytest.mark.parametrize("pct", [100.0, 99.9, 99.8])
@pytest.mark.parametrize("storage,sr,ams", [("q8", False, False), ("q8", True, True),
                                            ("q8_v_only", False, True)])
def test_percentile_on_sparse_blocks(pct, storage, sr, ams):
    # blocks with fewer non-zero moments than need: the need-th largest key
    # is 0, so the scale is the block maximum, which the walks' merge finds
    # (100 and 99.9: need 1 and 4) or the radix select's max reduction (99.8:
    # need 6)
    numels = RAGGED + [2048 * 6]
    log(f"percentile on sparse blocks: percentile {pct} {storage} sr={sr} amsgrad={ams}")
    params = workloads.host_params(29, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, "f32", amsgrad=ams)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    stats = Stats()
    hp = dict(HP, stochastic=sr, percentile=pct, seed=31)
    for t in range(1, 4):
        grads = _sparse_grads(29, numels, t)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, sr, stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


def _stage_grads(seed, numels, t):
    """Gradients that send the radix select down each of its paths, per
    block: keys a few hundred ulps apart with repeats (the answer's bin needs
    both fine passes), values spread over three decades (bins of one or two
    keys: the end pick after the coarse or the first fine pass), two thirds
    exact zeros (bisection at low percentiles), plain normal."""
    rng = np.random.default_rng([seed, t])
    out = []
    for n in numels:
        g = rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
        kinds = rng.integers(0, 4, (n + 2047) // 2048)
        for b, k in enumerate(kinds):
            blk = g[2048 * b:2048 * (b + 1)]
            if k == 0:
                near = np.float32(1e-3).view(np.uint32) + rng.integers(0, 600, blk.size).astype(np.uint32)
                blk[:] = near.view(np.float32) * np.where(rng.random(blk.size) < 0.5, -1, 1).astype(np.float32)
            elif k == 1:
                blk *= (np.float32(10.0) ** rng.uniform(-3, 0, blk.size)).astype(np.float32)
            elif k == 2:
                blk[:blk.size * 2 // 3] = 0.0
        out.append(g)
    return out


@pytest.mark.parametrize("pct", [10.0, 50.0, 99.0])
@pytest.mark.parametrize("storage,sr,ams", [("q8", False, False), ("q8", False, True), ("q8", True, False),
                                            ("q8", True, True), ("q8_v_only", False, True)])
def test_radix_select_every_stage(pct, storage, sr, ams):
    # beta1 = beta2 = 0: m = g and v = fl(g^2) exactly, so the constructed
    # gradients fix the keys of the select (a host model of its decisions
    # puts blocks of these gradients on the end pick after the coarse pass
    # and after the first fine pass, on both fine passes, and on the
    # bisection); two moments, and three with AMSGrad
    numels = RAGGED + [2048 * 8]
    log(f"radix select, every stage: percentile {pct} {storage} sr={sr} amsgrad={ams}")
    params = workloads.host_params(31, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, "f32", amsgrad=ams)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    stats = Stats()
    hp = dict(HP, beta1=0.0, beta2=0.0, stochastic=sr, percentile=pct, seed=37)
    for t in range(1, 4):
        grads = _stage_grads(31, numels, t)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, sr, stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


def _one_lane_top_grads(seed, numels, t):
    # in every full block one lane of one wave (lane 5 of wave b mod 4: block
    # elements 256w + 20 .. + 23 and 1024 + 256w + 20 .. + 23) holds the eight
    # largest gradients of its wave, distinct and alternating in sign
    gs = workloads.host_grads(seed, numels, t)
    for g in gs:
        for b in range(g.size // 2048):
            w, lane = b % 4, 5
            idx = [2048 * b + 256 * w + 4 * lane + k for k in range(4)]
            idx += [2048 * b + 1024 + 256 * w + 4 * lane + k for k in range(4)]
            for j, e in enumerate(idx):
                g[e] = np.float32((-1) ** j * 1e-2 * (1.0 + 0.1 * j + 0.01 * t))
    return gs


@pytest.mark.parametrize("pct", [100.0, 99.9, 99.8, 99.5, 100.0 * 2032.5 / 2047])
@pytest.mark.parametrize("storage,ams", [("q8", False), ("q8_v_only", True)])
def test_percentile_walk_lane_lists_run_empty(pct, storage, ams):
    # the lane holding its wave's largest values empties its short list
    # (two or four keys) before need is reached in that wave, which then
    # redoes the full walk; statistic and codes must not change
    log(f"percentile {pct:.4f} one-lane tops {storage} amsgrad={ams}")
    numels = [2048 * 4, 3000]
    hp = dict(HP, beta2=0.9, percentile=pct)
    params = workloads.host_params(62, numels)
    dev_p = [torch.from_numpy(x.copy()).cuda() for x in params]
    st = ma.adam_state_create(numels, storage, amsgrad=ams)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    stats = Stats()
    for t in range(1, 5):
        grads = _one_lane_top_grads(62, numels, t)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, False, stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


AMSGRAD_MODES = [
    # storage, grad dtype, stochastic, percentile, static scales, decoupled, beta2
    ("bf16", "f32", False, None, False, True, 0.9),
    ("bf16", "bf16", False, None, False, False, 0.999),
    ("q8", "f32", False, None, False, True, 0.9),
    ("q8", "bf16", True, None, False, True, 0.9),
    ("q8", "f32", False, 99.9, False, False, 0.9),
    ("q8", "bf16", True, 99.9, True, True, 0.9),
    ("q8_v_only", "f32", True, None, False, True, 0.999),
    ("q8_v_only", "bf16", False, 99.9, False, True, 0.9),
    ("q8_v_only", "f32", False, None, True, True, 0.9),
]


@pytest.mark.parametrize("storage,gdt,sr,pct,static,dec,b2", AMSGRAD_MODES)
def test_ragged_set_amsgrad(storage, gdt, sr, pct, static, dec, b2):
    # beta2 = 0.9 lets v fall below its running maximum within a few steps
    log(f"ragged AMSGrad {storage} grads={gdt} sr={sr} pct={pct} static={static} "
        f"decoupled={dec} beta2={b2}")
    hp = dict(HP, beta2=b2, stochastic=sr, percentile=pct, static_scales=static, decoupled=dec,
              seed=4321)
    for dist in ("normal", "student_t3"):
        stats = run_full_parity(RAGGED, storage, gdt, 10, hp, cfg_id=14, grad_dist=dist,
                                amsgrad=True)
        log(f"  {dist}: {stats}")


def test_full_size_sampled_blocks_amsgrad():
    cfg = dataclasses.replace(workloads.CONFIGS["gpt1p3b_q8_sr"], steps=3, amsgrad=True)
    log(f"full-size {cfg.name} AMSGrad: {sum(cfg.numels())} params, {cfg.steps} steps")
    stats = run_sampled_parity(cfg, log=log)
    assert stats.codes >= stats.params >= cfg.steps * 800 * 1024


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only"])
@pytest.mark.parametrize("eps", [1e-8, 2.0 ** -40, 1e-13, 1.0, 2.0 ** 20, 1e7])
def test_mixed_magnitudes_in_one_block(storage, eps):
    # within each block some waves hold only ordinary values and others tiny
    # (1e-20), zero or huge (1e15) gradients, and eps sits inside, on and
    # beyond the range where the update's short exact sqrt/divide applies:
    # every element must still match the oracle
    numels = [2048 * 3, 5000, 300]
    log(f"mixed magnitudes {storage} eps={eps}")
    params = workloads.host_params(31, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, "f32")
    ost = oracle.OracleState(numels, storage)
    hp = dict(HP, eps=eps)
    stats = Stats()
    for t in range(1, 6):
        grads = workloads.host_grads(31, numels, t)
        for g in grads:
            g[64:128] = 1e-20                 # one wave's lanes of the first group
            g[1024 + 256:1024 + 300] = 0.0     # part of another wave
            g[700:710] *= 1e18                 # |m| beyond 2^40
            g[1600:1602] = 1e-30
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, False, stats, f"t={t}")
    log(f"  {stats}")
    assert stats.params_exact == stats.params
    st.destroy()


@pytest.mark.parametrize("storage,ams,static", [("q8", False, False), ("q8", True, False),
                                                ("q8_v_only", True, False), ("q8", False, True)])
def test_stochastic_rounding_at_extreme_block_scales(storage, ams, static):
    # stochastic rounding on blocks whose reciprocal r = qmax / A sits far
    # from a training run's: moments up to ~1000 (r below 1/2), scales near
    # 2^-101 (r above 2^100), r near 1/2, a zero block, and subnormal moments
    # beside large ones (their scaled magnitudes underflow): every code must
    # match the oracle's, bit for bit
    numels = [2048 * 6, 1000]
    rng = np.random.default_rng(77)
    log(f"stochastic rounding at extreme scales {storage} amsgrad={ams} static={static}")
    params = workloads.host_params(33, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, "f32", amsgrad=ams)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    hp = dict(HP, stochastic=True, seed=99, static_scales=static)
    stats = Stats()
    for t in range(1, 6):
        grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in numels]
        g = grads[0]
        g[2048:2048 + 8] = 3000.0 * rng.choice([-1.0, 1.0], 8)  # A_m ~ 300, A_v ~ 9000: r < 1/2
        g[2048 + 100:2048 + 140] = np.float32(1e-44)           # subnormal m beside them
        g[2048 + 300:2048 + 340] = np.float32(3e-21)           # subnormal v
        g[4096:6144] = (rng.standard_normal(2048) * 1e-30).astype(np.float32)  # A_m ~ 2^-101: r > 2^100
        g[6144:6144 + 4] = 700.0                               # A_m ~ 70, A_v ~ 490: r just above 1/2
        g[6144 + 10:6144 + 60] = np.float32(1e-44)
        g[6144 + 60:6144 + 110] = np.float32(3e-21)
        g[8192:8192 + 4] = 714.0                               # A_v ~ 510: r near 1/2
        g[8192 + 10:8192 + 60] = np.float32(-1e-44)
        g[10240:12288] = np.float32(0.0)                       # zero block: r = 0
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, True, stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


def _random_case(i):
    rng = np.random.default_rng([4242, i])
    storage = ["bf16", "q8", "q8_v_only"][i % 3]
    q8 = storage != "bf16"
    case = dict(
        storage=storage,
        grad_dtype=["f32", "bf16"][int(rng.integers(2))],
        amsgrad=bool(rng.integers(2)),
        numels=[int(x) for x in rng.choice([0, 1, 15, 16, 17, 2047, 2048, 2049, 4100, 6144, 9001],
                                           size=int(rng.integers(1, 5)))],
        t0=int(rng.choice([1, 2, 1000, 100000])),
        dist=["normal", "student_t3", "normal_outliers", "few_levels"][int(rng.integers(4))],
        hp=dict(lr=float(rng.choice([1e-4, 1e-3, 1e-1])), beta1=float(rng.choice([0.0, 0.5, 0.9, 0.99])),
                beta2=float(rng.choice([0.9, 0.99, 0.999, 0.9999])),
                eps=float(rng.choice([1e-8, 1e-6, 1e-12, 1e-3])),
                weight_decay=float(rng.choice([0.0, 0.01, 0.1])), decoupled=bool(rng.integers(2)),
                stochastic=q8 and bool(rng.integers(2)),
                percentile=(float(rng.choice([0.0, 50.0, 99.0, 99.3, 99.5, 99.8, 99.9, 100.0]))
                            if q8 and rng.integers(2) else None),
                static_scales=q8 and bool(rng.integers(3) == 0), seed=int(rng.integers(2 ** 63))))
    return case


@pytest.mark.parametrize("i", range(36))
def test_random_configurations(i):
    c = _random_case(i)
    numels, hp, gdt = c["numels"], c["hp"], c["grad_dtype"]
    log(f"random case {i}: {c}")
    params = workloads.host_params(500 + i, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, c["storage"], gdt, amsgrad=c["amsgrad"])
    ost = oracle.OracleState(numels, c["storage"], grad_bf16=(gdt == "bf16"), amsgrad=c["amsgrad"])
    stats = Stats()
    for t in range(c["t0"], c["t0"] + 4):
        grads = workloads.host_grads(500 + i, numels, t, dist=c["dist"], dtype=gdt)
        ma.adam_step(st, dev_p, to_device_grads(grads, gdt), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
        if sum(numels):
            got = read_state(st)
            for nm, want in ost.buffers().items():
                compare_buffer(nm, got[nm], want, hp["stochastic"], stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()


def _slices(shard):
    """(tensor index, start, stop) of each slice named 't<k>[start:stop]'."""
    out = []
    for name, _ in shard:
        base, rng = name.split("[")
        lo, hi = (int(x) for x in rng.rstrip("]").split(":"))
        out.append((int(base[1:]), lo, hi))
    return out


@pytest.mark.parametrize("storage,gdt,sr,ams,pct", [("q8", "bf16", True, False, None),
                                                    ("q8_v_only", "f32", True, True, 99.9),
                                                    ("bf16", "f32", False, True, None)])
def test_zero1_shards_reproduce_the_unsharded_step(storage, gdt, sr, ams, pct):
    # three states, each holding one rank's block-aligned slices of the set
    # with their draw indices set to the slices' flat indices in the whole
    # state, step to the same bits as one state over the whole set
    sizes = [9001, 2048 * 3, 17, 4100, 6001, 2048]
    shapes = [(f"t{k}", (n,)) for k, n in enumerate(sizes)]
    log(f"ZeRO-1 shards x3 {storage} sr={sr} amsgrad={ams} pct={pct}")
    seg = np.concatenate([[0], np.cumsum([oracle.pad16(n) for n in sizes])])
    blk0 = np.concatenate([[0], np.cumsum([-(-n // 2048) for n in sizes])])
    hp = dict(HP, stochastic=sr, percentile=pct, seed=2024)
    p0 = workloads.host_params(41, sizes)
    whole_p = [torch.from_numpy(x.copy()).cuda() for x in p0]
    shard_p = [torch.from_numpy(x.copy()).cuda() for x in p0]
    whole = ma.adam_state_create(sizes, storage, gdt, amsgrad=ams)
    shards = []
    for r in range(3):
        sl = _slices(workloads.zero1_shard_shapes(shapes, r, 3))
        st = ma.adam_state_create([b - a for _, a, b in sl], storage, gdt, amsgrad=ams)
        ma.adam_state_set_draw_index(st, [int(seg[k]) + a for k, a, _ in sl])
        assert ma.adam_state_get_draw_index(st) == [int(seg[k]) + a for k, a, _ in sl]
        shards.append((sl, st))
    for t in range(1, 5):
        g = to_device_grads(workloads.host_grads(41, sizes, t, dtype=gdt), gdt)
        ma.adam_step(whole, whole_p, g, t=t, **hp)
        for sl, st in shards:
            ma.adam_step(st, [shard_p[k][a:b] for k, a, b in sl], [g[k][a:b] for k, a, b in sl],
                         t=t, **hp)
    torch.cuda.synchronize()
    for a_, b_ in zip(whole_p, shard_p):
        assert torch.equal(a_.view(torch.int32), b_.view(torch.int32))
    want = read_state(whole)
    for sl, st in shards:
        got = read_state(st)
        sseg, sblk = 0, 0
        for k, a, b in sl:
            for nm, w in want.items():
                if nm.endswith("scale"):
                    nb = -(-(b - a) // 2048)
                    g0 = blk0[k] + a // 2048
                    assert np.array_equal(got[nm][sblk:sblk + nb].view(np.uint32),
                                          w[g0:g0 + nb].view(np.uint32)), (nm, k, a)
                else:
                    gv = got[nm][sseg:sseg + b - a]
                    wv = w[seg[k] + a:seg[k] + b]
                    assert np.array_equal(gv.view(np.uint8), wv.view(np.uint8)), (nm, k, a)
            sseg += oracle.pad16(b - a)
            sblk += -(-(b - a) // 2048)
        st.destroy()
    whole.destroy()


def test_draw_index_validation_and_checkpoint():
    numels = [5000, 17]
    st = ma.adam_state_create(numels, "q8", "f32")
    assert ma.adam_state_get_draw_index(st) == [0, 5008]
    for bad in ([8, 5008], [-16, 5008], [0, 2 ** 62 - 16]):
        with pytest.raises(ma.AdamError) as e:
            ma.adam_state_set_draw_index(st, bad)
        assert e.value.code == -1, bad
    assert ma.adam_state_get_draw_index(st) == [0, 5008]
    ma.adam_state_set_draw_index(st, [2 ** 40, 16])
    params = workloads.host_params(42, numels)
    dev_p = [torch.from_numpy(x.copy()).cuda() for x in params]
    hp = dict(HP, stochastic=True, seed=3)
    grads = [to_device_grads(workloads.host_grads(42, numels, t), "f32") for t in range(1, 5)]
    for t in (1, 2):
        ma.adam_step(st, dev_p, grads[t - 1], t=t, **hp)
    st2 = ma.adam_state_load(ma.adam_state_save(st))
    assert ma.adam_state_get_draw_index(st2) == [2 ** 40, 16]
    p2 = [x.clone() for x in dev_p]
    for t in (3, 4):
        ma.adam_step(st, dev_p, grads[t - 1], t=t, **hp)
        ma.adam_step(st2, p2, grads[t - 1], t=t, **hp)
    torch.cuda.synchronize()
    a, b = read_state(st), read_state(st2)
    for nm in a:
        assert np.array_equal(a[nm].view(np.uint8), b[nm].view(np.uint8)), nm
    for x, y in zip(dev_p, p2):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    # the draws did move: the default indices give other codes
    st3 = ma.adam_state_create(numels, "q8", "f32")
    p3 = [torch.from_numpy(x.copy()).cuda() for x in params]
    for t in (1, 2, 3, 4):
        ma.adam_step(st3, p3, grads[t - 1], t=t, **hp)
    torch.cuda.synchronize()
    assert not np.array_equal(read_state(st3)["m_codes"], a["m_codes"])
    for x in (st, st2, st3):
        x.destroy()


_GOLDEN = None


def _golden():
    global _GOLDEN
    if _GOLDEN is None:
        import json
        import os
        with open(os.path.join(os.path.dirname(__file__), "golden", "step_examples.json")) as f:
            _GOLDEN = json.load(f)
    return _GOLDEN


def _f32(hexes):
    return np.array([int(h, 16) for h in hexes], np.uint32).view(np.float32)


@pytest.mark.parametrize("name", ["bf16", "bf16_amsgrad_l2", "q8_rne", "q8_sr", "q8_sr_amsgrad",
                                  "q8_pct50", "q8_v_only_sr_pct"])
def test_stored_step_examples(name):
    # the stored examples (written from the oracle, kept in the repository)
    G = _golden()
    case = G["cases"][name]
    numels = G["numels"]
    st = ma.adam_state_create(numels, case["storage"], "f32", amsgrad=case["amsgrad"])
    dev_p = [torch.from_numpy(_f32(p).copy()).cuda() for p in G["params0"]]
    stats = Stats()
    for t, want in enumerate(case["steps"], start=1):
        grads = [_f32(g) for g in G["grads"][t - 1]]
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, stochastic=case["stochastic"],
                     percentile=case["percentile"], seed=G["seed"], decoupled=case["decoupled"],
                     **G["hparams"])
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), _f32(want["params"][k]), stats, f"t={t} tensor {k}")
        got = read_state(st)
        for nm, ref in want.items():
            if nm == "params":
                continue
            ref = _f32(ref) if got[nm].dtype == np.float32 else np.array(ref, got[nm].dtype)
            compare_buffer(nm, got[nm], ref, case["stochastic"], stats, f"t={t}")
    assert stats.params_exact == stats.params
    st.destroy()


@pytest.mark.parametrize("storage,gdt,sr,pct,static,ams", [("q8", "bf16", True, None, False, False),
                                                          ("q8_v_only", "f32", False, 99.9, False, False),
                                                          ("bf16", "f32", False, None, False, False),
                                                          ("q8", "f32", True, None, True, True)])
def test_hundred_steps_stay_bit_exact(storage, gdt, sr, pct, static, ams):
    # a long run: every element, every 10th step, params bit for bit
    numels = RAGGED
    log(f"100 steps {storage} grads={gdt} sr={sr} pct={pct} static={static} amsgrad={ams}")
    hp = dict(HP, stochastic=sr, percentile=pct, static_scales=static, seed=7)
    params = workloads.host_params(43, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, gdt, amsgrad=ams)
    ost = oracle.OracleState(numels, storage, grad_bf16=(gdt == "bf16"), amsgrad=ams)
    stats = Stats()
    for t in range(1, 101):
        grads = workloads.host_grads(43, numels, t, dist="student_t3", dtype=gdt)
        ma.adam_step(st, dev_p, to_device_grads(grads, gdt), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        if t % 10 == 0:
            torch.cuda.synchronize()
            for k in range(len(numels)):
                compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
            got = read_state(st)
            for nm, want in ost.buffers().items():
                compare_buffer(nm, got[nm], want, sr, stats, f"t={t}")
    log(f"  {stats}")
    assert stats.params_exact == stats.params
    st.destroy()


def test_single_tensor_1m_q8_ten_steps():
    cfg = workloads.CONFIGS["single_q8"]
    log("single 1M q8 nearest-even, 10 steps")
    stats = run_full_parity(cfg.numels(), cfg.storage, cfg.grad_dtype, cfg.steps, cfg.hp,
                            cfg_id=cfg.cfg_id)
    log(f"  {stats}")
    assert stats.params == 10 * 1048576


def test_full_size_sampled_blocks_static_scales():
    cfg = dataclasses.replace(workloads.CONFIGS["llama7b_mf32_vq8_pct"], steps=4)
    cfg.hp = dict(cfg.hp, static_scales=True)
    log(f"full-size {cfg.name} static scales: {sum(cfg.numels())} params, {cfg.steps} steps")
    stats = run_sampled_parity(cfg, log=log)
    assert stats.codes >= stats.params >= cfg.steps * 800 * 1024


@pytest.mark.parametrize("name", ["vit_bf16", "vit_q8", "gpt1p3b_q8_sr",
                                  "llama7b_mf32_vq8_pct", "llama7b_shard8_mf32_vq8_pct",
                                  "vit_q8@99.0", "vit_q8@50.0", "vit_q8@99.9",
                                  "gpt1p3b_q8_sr@99.9", "vit_q8+sr", "vit_q8+sr@99.9"])
def test_full_size_sampled_blocks(name):
    # name@p: the same set with the percentile-p block statistic (the top
    # walks serve 99.85 and above, the radix select the rest); name+sr: with
    # stochastic rounding (fp32 grads); in the benchmark's launch
    # configuration (XCD block order included)
    base, _, pct = name.partition("@")
    base, _, sr = base.partition("+")
    cfg = workloads.CONFIGS[base]
    if sr:
        cfg = dataclasses.replace(cfg, hp=dict(cfg.hp, stochastic=True), name=f"{base}_sr")
    if pct:
        cfg = dataclasses.replace(cfg, hp=dict(cfg.hp, percentile=float(pct)),
                                  name=f"{cfg.name}_percentile{pct}")
    log(f"full-size {name}: {sum(cfg.numels())} params, {cfg.steps} steps")
    stats = run_sampled_parity(cfg, log=log)
    # every step compared at least the sampled blocks' params (and codes)
    assert stats.params >= cfg.steps * 800 * 1024
    if cfg.storage != "bf16":
        assert stats.codes >= stats.params


def test_empty_and_zero_size_tensors():
    st = ma.adam_state_create([], "q8")
    ma.adam_step(st, [], [], t=1, **HP)
    st.destroy()
    numels = [0, 5, 0, 3000, 0]
    run_full_parity(numels, "q8", "f32", 3, dict(HP, stochastic=True), cfg_id=12)
    run_full_parity(numels, "bf16", "bf16", 3, HP, cfg_id=12)
    st = ma.adam_state_create([0, 0], "bf16")
    z = torch.empty(0, device="cuda")
    ma.adam_step(st, [z, z], [z, z], t=1, **HP)
    st.destroy()


def test_largest_tensor_last_blocks():
    # numel 2^32 - 1: the largest tensor the descriptor format takes
    n = 2 ** 32 - 1
    log("2^32-1 element tensor, q8 with bf16 grads, 2 steps (last 3 blocks checked)")
    p = torch.empty(n, dtype=torch.float32, device="cuda")
    g = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    p.normal_(0, 0.02, generator=gen)
    tail = 2048 * 2 + (n % 2048)
    lo = n - tail
    host_p = [p[lo:].cpu().numpy()]
    st = ma.adam_state_create([n], "q8", "bf16")
    first_block = lo // 2048
    ob = oracle.OracleBlocks([(2048, lo), (2048, lo + 2048), (n % 2048, lo + 4096)], "q8",
                             grad_bf16=True)
    stats = Stats()
    for t in (1, 2):
        g.normal_(0, 1e-3, generator=gen)
        hg = g[lo:].view(torch.int16).cpu().numpy().view(np.uint16)
        ma.adam_step(st, [p], [g], t=t, stochastic=True, seed=99, **HP)
        blocks_p = [host_p[0][0:2048], host_p[0][2048:4096], host_p[0][4096:]]
        ob.step(blocks_p, [hg[0:2048], hg[2048:4096], hg[4096:]], t=t, stochastic=True,
                seed=99, **HP)
        host_p = [np.concatenate(blocks_p)]
        torch.cuda.synchronize()
        compare_params(p[lo:].cpu().numpy(), host_p[0], stats, f"t={t}")
        codes = ma.adam_state_read(st, "m_codes")
        compare_buffer("m_codes", codes[lo:n].cpu().numpy(),
                       np.concatenate([ob.inner.m_codes[ob.block_slice(i)] for i in range(3)]),
                       True, stats, f"t={t}")
        del codes
        sc = ma.adam_state_read(st, "v_scale")[first_block:].cpu().numpy()
        compare_buffer("v_scale", sc, ob.inner.v_scale, True, stats, f"t={t}")
    log(f"  {stats}")
    st.destroy()
    del p, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("storage", ["bf16", "q8", "q8_v_only"])
@pytest.mark.parametrize("ams", [False, True])
def test_step_from_injected_state(storage, ams):
    # arbitrary (non-trajectory) state: extreme codes, tiny / huge / zero scales
    numels = [2048, 5000, 17]
    rng = np.random.default_rng(21)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    for name, buf in ost.buffers().items():
        if name == "m_codes":
            buf[:] = rng.integers(-127, 128, buf.size)
        elif name in ("v_codes", "vmax_codes"):
            buf[:] = rng.integers(0, 256, buf.size)
        elif name.endswith("scale"):
            buf[:] = (10.0 ** rng.uniform(-30, 2, buf.size)).astype(np.float32)
            buf[0] = 0.0
            buf[-1] = np.float32(2.0 ** -112)
        elif name.endswith("bf16"):
            x = (rng.standard_normal(buf.size) * 1e-3).astype(np.float32)
            buf[:] = oracle.bf16_from_f32(x if name == "m_bf16" else np.abs(x))
        elif name == "m_f32":
            buf[:] = (rng.standard_normal(buf.size) * 1e-3).astype(np.float32)
    # The oracle's padding entries are zero, as its layout keeps them; the
    # GPU state gets the same buffers with non-zero padding.  A step ignores
    # padding and stores it back as zero, so after it the two must agree
    # everywhere (padding included).
    seg = 0
    gpu_bufs = {}
    for n in numels:
        for name, buf in ost.buffers().items():
            if not name.endswith("scale"):
                buf[seg + n:seg + oracle.pad16(n)] = 0
        seg += oracle.pad16(n)
    for name, buf in ost.buffers().items():
        b = buf.copy()
        if not name.endswith("scale"):
            seg = 0
            for n in numels:
                pad = slice(seg + n, seg + oracle.pad16(n))
                if name.endswith("bf16"):
                    b[pad] = oracle.bf16_from_f32(np.full(b[pad].size, 0.5, np.float32))
                elif name == "m_f32":
                    b[pad] = np.float32(-0.5)
                else:
                    b[pad] = 127 if name == "m_codes" else 255
                seg += oracle.pad16(n)
        gpu_bufs[name] = b
    st = ma.adam_state_create(numels, storage, amsgrad=ams)
    for name, buf in gpu_bufs.items():
        src = torch.from_numpy(buf.view(np.int16) if name.endswith("bf16") else buf).cuda()
        ma.adam_state_write(st, name, src)
    params = workloads.host_params(22, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    stats = Stats()
    for t in (7, 8):
        grads = workloads.host_grads(22, numels, t)
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **HP)
        ost.step(params, grads, t=t, **HP)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats)
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, False, stats, f"t={t}")
    st.destroy()


@pytest.mark.parametrize("case", ["beta1_zero", "lr_zero", "wd_zero", "late_step", "big_eps",
                                  "zero_grads", "constant_grads", "tiny_grads"])
def test_degenerate_hyperparameters(case):
    hp = dict(HP)
    numels = [4100, 2048, 31]
    params = workloads.host_params(23, numels)
    t0 = 1
    if case == "beta1_zero":
        hp["beta1"] = 0.0
    elif case == "lr_zero":
        hp["lr"] = 0.0
    elif case == "wd_zero":
        hp["weight_decay"] = 0.0
    elif case == "late_step":
        t0 = 10 ** 6
    elif case == "big_eps":
        hp["eps"] = 1.0
    for storage, sr in (("bf16", False), ("q8", False), ("q8", True), ("q8_v_only", False)):
        p = [x.copy() for x in params]
        dev_p = [torch.from_numpy(x.copy()).cuda() for x in p]
        st = ma.adam_state_create(numels, storage)
        ost = oracle.OracleState(numels, storage)
        stats = Stats()
        for t in range(t0, t0 + 3):
            if case == "zero_grads":
                grads = [np.zeros(n, np.float32) for n in numels]
            elif case == "constant_grads":
                grads = [np.full(n, np.float32(3e-4 * (-1) ** t), np.float32) for n in numels]
            elif case == "tiny_grads":
                grads = [(g * np.float32(1e-20)).astype(np.float32)
                         for g in workloads.host_grads(23, numels, t)]
            else:
                grads = workloads.host_grads(23, numels, t)
            ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, stochastic=sr, **hp)
            ost.step(p, grads, t=t, stochastic=sr, **hp)
            torch.cuda.synchronize()
            for k in range(len(numels)):
                compare_params(dev_p[k].cpu().numpy(), p[k], stats, f"{case} {storage} t={t}")
            got = read_state(st)
            for nm, want in ost.buffers().items():
                compare_buffer(nm, got[nm], want, sr, stats, f"{case} {storage} t={t}")
        st.destroy()


def test_pointer_change_and_side_stream():
    numels = [3000, 2048]
    params = workloads.host_params(24, numels)
    st = ma.adam_state_create(numels, "q8")
    ost = oracle.OracleState(numels, "q8")
    side = torch.cuda.Stream()
    stats = Stats()
    dev_p = [torch.from_numpy(x.copy()).cuda() for x in params]
    for t in range(1, 5):
        grads = workloads.host_grads(24, numels, t)
        if t == 3:  # move the params to new allocations
            dev_p = [x.clone() for x in dev_p]
        dg = to_device_grads(grads, "f32")
        if t % 2:
            ma.adam_step(st, dev_p, dg, t=t, **HP)
        else:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                ma.adam_step(st, dev_p, dg, t=t, **HP)
            torch.cuda.current_stream().wait_stream(side)
        ost.step(params, grads, t=t, **HP)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats)
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, False, stats)
    st.destroy()


def test_two_states_interleaved():
    a_n, b_n = [5000], [2049, 7]
    pa = workloads.host_params(25, a_n)
    pb = workloads.host_params(26, b_n)
    sa, sb = ma.adam_state_create(a_n, "q8"), ma.adam_state_create(b_n, "bf16", "bf16")
    oa, ob = oracle.OracleState(a_n, "q8"), oracle.OracleState(b_n, "bf16", grad_bf16=True)
    da = [torch.from_numpy(x.copy()).cuda() for x in pa]
    db = [torch.from_numpy(x.copy()).cuda() for x in pb]
    for t in (1, 2, 3):
        ga = workloads.host_grads(25, a_n, t)
        gb = workloads.host_grads(26, b_n, t, dtype="bf16")
        ma.adam_step(sa, da, to_device_grads(ga, "f32"), t=t, **HP)
        ma.adam_step(sb, db, to_device_grads(gb, "bf16"), t=t, **HP)
        oa.step(pa, ga, t=t, **HP)
        ob.step(pb, gb, t=t, **HP)
    torch.cuda.synchronize()
    stats = Stats()
    for d, h in zip(da + db, pa + pb):
        compare_params(d.cpu().numpy(), h, stats)
    for st, o in ((sa, oa), (sb, ob)):
        got = read_state(st)
        for nm, want in o.buffers().items():
            compare_buffer(nm, got[nm], want, False, stats)
    sa.destroy()
    sb.destroy()


def test_states_stepped_from_concurrent_threads_and_streams():
    # different states are independent: four host threads, each with its own
    # state, stream and rotating gradient buffers (so the pointer-table cache
    # and staging ring are exercised), step concurrently without any host
    # synchronization between them; each result must equal its oracle run
    import threading
    specs = [([3000, 17], "q8", "f32", True), ([2049, 5000], "bf16", "bf16", False),
             ([6001], "q8_v_only", "bf16", True), ([4096, 1, 300], "q8", "bf16", False)]
    runs, errors = [], []
    for i, (numels, storage, gdt, sr) in enumerate(specs):
        params = workloads.host_params(60 + i, numels)
        grads = [workloads.host_grads(60 + i, numels, t, dtype=gdt) for t in range(1, 13)]
        runs.append(dict(numels=numels, storage=storage, gdt=gdt, sr=sr, params=params, grads=grads,
                         dev_p=[torch.from_numpy(x.copy()).cuda() for x in params],
                         dev_g=[to_device_grads(g, gdt) for g in grads],
                         stream=torch.cuda.Stream(),
                         st=ma.adam_state_create(numels, storage, gdt)))
    torch.cuda.synchronize()

    def work(r):
        try:
            for t in range(1, 13):
                ma.adam_step(r["st"], r["dev_p"], r["dev_g"][t - 1], t=t, stochastic=r["sr"], seed=11,
                             stream=r["stream"], **HP)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(r,)) for r in runs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    stats = Stats()
    for r in runs:
        o = oracle.OracleState(r["numels"], r["storage"], grad_bf16=(r["gdt"] == "bf16"))
        for t in range(1, 13):
            o.step(r["params"], r["grads"][t - 1], t=t, stochastic=r["sr"], seed=11, **HP)
        for d, h in zip(r["dev_p"], r["params"]):
            compare_params(d.cpu().numpy(), h, stats)
        got = read_state(r["st"])
        for nm, want in o.buffers().items():
            compare_buffer(nm, got[nm], want, r["sr"], stats)
        r["st"].destroy()
    assert stats.params_exact == stats.params


def test_error_paths_enqueue_nothing():
    numels = [100]
    st = ma.adam_state_create(numels, "q8")
    p = torch.zeros(104, device="cuda")
    g = torch.zeros(104, device="cuda")
    before = p.clone()
    with pytest.raises(ma.AdamError) as e:  # layout drift
        ma.adam_step(st, [p[:100]], [g[:100]], t=1, expect=("bf16", "f32"), **HP)
    assert e.value.code == -2
    with pytest.raises(ma.AdamError) as e:  # AMSGrad option drift
        ma.adam_step(st, [p[:100]], [g[:100]], t=1, expect=("q8", "f32", 2048, 1), **HP)
    assert e.value.code == -2
    with pytest.raises(ma.AdamError):  # absent buffer
        ma.adam_state_read(st, "vmax_codes")
    with pytest.raises(ma.AdamError) as e:  # 4-byte offset pointer
        ma.adam_step(st, [p[1:101]], [g[:100]], t=1, **HP)
    assert e.value.code == -3
    for bad in (dict(t=0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(lr=-1.0),
                dict(weight_decay=float("nan")), dict(percentile=101.0)):
        kw = dict(HP, t=1)
        kw.update(bad)
        with pytest.raises(ma.AdamError) as e:
            ma.adam_step(st, [p[:100]], [g[:100]], **kw)
        assert e.value.code == -1, bad
    bst = ma.adam_state_create(numels, "bf16")
    with pytest.raises(ma.AdamError):
        ma.adam_step(bst, [p[:100]], [g[:100]], t=1, stochastic=True, **HP)
    with pytest.raises(ma.AdamError) as e:
        ma.adam_step(bst, [p[:100]], [g[:100]], t=1, static_scales=True, **HP)
    assert e.value.code == -1
    with pytest.raises(ma.AdamError):
        ma.adam_state_read(bst, "m_codes")
    lib = ma.library()
    buf = torch.empty(10, dtype=torch.uint8, device="cuda")
    assert lib.adam_state_read(ctypes.c_void_p(st.handle), 1, ctypes.c_void_p(buf.data_ptr()), 10,
                               None) == -1
    torch.cuda.synchronize()
    assert torch.equal(p, before)
    st.destroy()
    bst.destroy()


def test_alternating_gradient_buffers_beyond_the_table_cache():
    # six gradient buffer sets in rotation (more than the resident pointer
    # tables), params moved twice: every step must still read the right tensors
    numels = [3000, 2048, 77]
    params = workloads.host_params(27, numels)
    dev_p = [torch.from_numpy(x.copy()).cuda() for x in params]
    bufs = [[torch.empty(n, device="cuda") for n in numels] for _ in range(6)]
    st = ma.adam_state_create(numels, "q8")
    ost = oracle.OracleState(numels, "q8")
    stats = Stats()
    order = [0, 1, 2, 3, 4, 5, 0, 2, 4, 1, 3, 5, 5, 0]
    for t, b in enumerate(order, start=1):
        grads = workloads.host_grads(27, numels, t)
        for k in range(len(numels)):
            bufs[b][k].copy_(torch.from_numpy(grads[k]))
        if t in (5, 11):
            dev_p = [x.clone() for x in dev_p]
        ma.adam_step(st, dev_p, bufs[b], t=t, stochastic=True, seed=5, **HP)
        ost.step(params, grads, t=t, stochastic=True, seed=5, **HP)
        torch.cuda.synchronize()
        for k in range(len(numels)):
            compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            compare_buffer(nm, got[nm], want, True, stats, f"t={t}")
    st.destroy()


def test_step_refuses_a_capturing_stream():
    # a captured launch would replay one call's t with a pointer table later
    # calls may re-use: the step is refused while the stream captures, it
    # records nothing (the capture stays valid and replays its own work),
    # and eager steps go on as before
    log("graph capture refused")
    numels = [4100, 17]
    params = workloads.host_params(61, numels)
    dev_p = [torch.from_numpy(x.copy()).cuda() for x in params]
    grads = [workloads.host_grads(61, numels, t) for t in (1, 2)]
    dev_g = [[torch.from_numpy(x.copy()).cuda() for x in gs] for gs in grads]
    st = ma.adam_state_create(numels, "q8")
    ost = oracle.OracleState(numels, "q8")
    ma.adam_step(st, dev_p, dev_g[0], t=1, **HP)  # eager: the pointer table is resident
    ost.step(params, grads[0], t=1, **HP)
    torch.cuda.synchronize()
    before_p = [x.clone() for x in dev_p]
    before_s = read_state(st)
    x = torch.zeros(64, device="cuda")
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        try:
            x.add_(1.0)
            with pytest.raises(ma.AdamError) as e:
                ma.adam_step(st, dev_p, dev_g[1], t=2, stream=side, **HP)
            assert e.value.code == -1
            assert "graph" in ma.adam_last_error()
        finally:
            graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(x, torch.full_like(x, 3.0))
    for a, b in zip(dev_p, before_p):
        assert torch.equal(a, b)
    after_s = read_state(st)
    for nm, want in before_s.items():
        assert np.array_equal(after_s[nm], want), nm
    ma.adam_step(st, dev_p, dev_g[1], t=2, **HP)
    ost.step(params, grads[1], t=2, **HP)
    torch.cuda.synchronize()
    stats = Stats()
    for k in range(len(numels)):
        compare_params(dev_p[k].cpu().numpy(), params[k], stats, "t=2")
    got = read_state(st)
    for nm, want in ost.buffers().items():
        compare_buffer(nm, got[nm], want, False, stats, "t=2")
    del graph
    st.destroy()


@pytest.mark.parametrize("storage,gdt,sr,pct,ams", [("bf16", "f32", False, None, False),
                                                    ("q8", "bf16", True, None, False),
                                                    ("q8_v_only", "bf16", False, 99.9, False),
                                                    ("bf16", "bf16", False, None, True),
                                                    ("q8", "f32", True, 99.9, True)])
def test_checkpoint_resume_is_bit_exact(storage, gdt, sr, pct, ams):
    # 4 steps, save; continue 3 steps (A); load the checkpoint into a new
    # state and run the same 3 steps from the saved params (B).  A == B bit
    # for bit, and both equal the oracle after 7 uninterrupted steps.
    numels = RAGGED
    hp = dict(HP, stochastic=sr, percentile=pct, seed=77)
    params = workloads.host_params(28, numels)
    dev_p = [torch.from_numpy(x.copy()).cuda() for x in params]
    st = ma.adam_state_create(numels, storage, gdt, amsgrad=ams)
    ost = oracle.OracleState(numels, storage, grad_bf16=(gdt == "bf16"), amsgrad=ams)
    grads = [workloads.host_grads(28, numels, t, dtype=gdt) for t in range(1, 8)]
    for t in range(1, 5):
        ma.adam_step(st, dev_p, to_device_grads(grads[t - 1], gdt), t=t, **hp)
    blob = ma.adam_state_save(st)
    assert blob.size == ma.adam_state_serialized_bytes(st)
    saved_p = [x.clone() for x in dev_p]
    # the stream's records are the state buffers, verbatim
    got = read_state(st)
    off = 40 + 16 * len(numels)
    names = {"bf16": ["m_bf16", "v_bf16"], "q8": ["m_codes", "v_codes", "m_scale", "v_scale"],
             "q8_v_only": ["v_codes", "v_scale", "m_f32"]}[storage]
    if ams:
        names += ["vmax_bf16"] if storage == "bf16" else ["vmax_codes", "vmax_scale"]
    for name in names:
        nb = int(np.frombuffer(blob[off + 8:off + 16].tobytes(), np.uint64)[0])
        assert nb == got[name].nbytes
        assert np.array_equal(blob[off + 16:off + 16 + nb], got[name].view(np.uint8)), name
        off += 16 + (nb + 7) // 8 * 8
    for t in range(5, 8):
        ma.adam_step(st, dev_p, to_device_grads(grads[t - 1], gdt), t=t, **hp)
    st2 = ma.adam_state_load(blob)
    assert st2.numels == list(numels) and st2.storage == storage and st2.amsgrad == ams
    for t in range(5, 8):
        ma.adam_step(st2, saved_p, to_device_grads(grads[t - 1], gdt), t=t, **hp)
    for t in range(1, 8):
        ost.step(params, grads[t - 1], t=t, **hp)
    torch.cuda.synchronize()
    a, b = read_state(st), read_state(st2)
    stats = Stats()
    for nm, want in ost.buffers().items():
        assert np.array_equal(a[nm].view(np.uint8), b[nm].view(np.uint8)), nm
        compare_buffer(nm, a[nm], want, sr, stats)
    for k in range(len(numels)):
        pa, pb = dev_p[k].cpu().numpy(), saved_p[k].cpu().numpy()
        assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))
        compare_params(pa, params[k], stats)
    st.destroy()
    st2.destroy()


def test_checkpoint_rejects_a_corrupted_stream():
    st = ma.adam_state_create([5000, 3], "q8")
    blob = ma.adam_state_save(st)
    bad = blob.copy()
    bad[100] ^= 0x01
    with pytest.raises(ma.AdamError) as e:
        ma.adam_state_load(bad)
    assert e.value.code == -1 and "checksum" in str(e.value)
    with pytest.raises(ma.AdamError):
        ma.adam_state_load(blob[:-8])
    # a destination of the wrong size is refused before any copy
    rc = ma.library().adam_state_save(ctypes.c_void_p(st.handle), ctypes.c_void_p(blob.ctypes.data),
                                      blob.size - 8, None)
    assert rc == -1
    empty = ma.adam_state_create([], "bf16")
    again = ma.adam_state_load(ma.adam_state_save(empty))
    assert again.numels == []
    st.destroy()
    empty.destroy()
    again.destroy()


# ---------------------------------------------------------------- exact rounding ties
# Nearest rounding breaks ties to even (reading S8; the 8-bit Adam page names
# only the stochastic option).  With beta1 = beta2 = 0 the new moments are
# m = g and v = fl(g*g) exactly, so gradients can be placed on exact ties:
#   first moment: block maximum 127 * 2^-12 gives r = fl(127 / A) = 2^12, and
#     |g| = (k + 1/2) * 2^-12 gives y = k + 1/2 exactly;
#   second moment: for a block maximum g_max (A = fl(g_max^2), r = fl(255/A)),
#     a host search finds fp32 g with fl(fl(g*g) * r) = k + 1/2 exactly (six
#     block scales between them reach 247 of the 255 half-integers).
# Codes must then match the oracle bit for bit (not within +-1), and the tie
# codes must be the even neighbours.
_TIE_GMAX = [2.0 ** -10 * f for f in (1.0, 1.5, 1.25, 1.75, 1.125, 1.375)]


def _v_tie_blocks():
    """[(g_max, [(k, g), ...]) per block]: fp32 gradients whose squares land
    on y = k + 1/2 in a block whose maximum gradient is g_max."""
    cover = {}
    blocks = []
    for gm in _TIE_GMAX:
        gm = np.float32(gm)
        r = np.float32(255.0) / (gm * gm)
        ties = []
        for k in range(255):
            if k in cover:
                continue
            yt = np.float32(k + 0.5)
            g0 = np.float32(np.sqrt(float(yt) / float(r)))
            cand = (g0.view(np.uint32).astype(np.int64) + np.arange(-64, 65)).astype(
                np.uint32).view(np.float32)
            hit = np.nonzero(((cand * cand) * r == yt) & (cand < gm))[0]
            if hit.size:
                cover[k] = True
                ties.append((k, cand[hit[0]]))
        blocks.append((gm, ties))
    assert sum(len(t) for _, t in blocks) >= 240
    return blocks


def _tie_inputs():
    """Two tensors: m ties (3 blocks, the last ragged) and v ties (one block
    per block scale, the last ragged).  Returns grads, and per tensor the
    expected (index, code) of every tie element for m and for v."""
    rng = np.random.default_rng(77)
    # first-moment ties
    n0 = 2 * 2048 + 700
    k = rng.integers(0, 127, n0)
    sgn = np.where(rng.random(n0) < 0.5, -1, 1)
    g0 = (sgn * (k + 0.5) * 2.0 ** -12).astype(np.float32)
    maxpos = [0, 2048, 4096]
    for b, i in enumerate(maxpos):
        g0[i] = np.float32((1 if b % 2 == 0 else -1) * 127 * 2.0 ** -12)
    m_ties = [(i, int(sgn[i]) * int(k[i] + (k[i] & 1))) for i in range(n0) if i not in maxpos]
    # second-moment ties
    vblocks = _v_tie_blocks()
    n1 = 2048 * (len(vblocks) - 1) + 1500
    g1 = np.zeros(n1, np.float32)
    v_ties = []
    for b, (gm, ties) in enumerate(vblocks):
        base = 2048 * b
        length = min(2048, n1 - base)
        g1[base] = gm
        for j in range(1, length):
            kk, g = ties[(j - 1) % len(ties)]
            g1[base + j] = g if rng.random() < 0.5 else -g
            v_ties.append((base + j, kk + (kk & 1)))
    return [g0, g1], m_ties, v_ties


@pytest.mark.parametrize("storage,ams,pct", [("q8", False, None), ("q8", True, None),
                                             ("q8", False, 100.0), ("q8_v_only", False, None),
                                             ("q8_v_only", True, 100.0)])
def test_nearest_rounding_ties_to_even(storage, ams, pct):
    grads, m_ties, v_ties = _tie_inputs()
    numels = [g.size for g in grads]
    hp = dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.01, percentile=pct)
    params = workloads.host_params(31, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, amsgrad=ams)
    ost = oracle.OracleState(numels, storage, amsgrad=ams)
    seg1 = oracle.pad16(numels[0])
    stats = Stats()
    for t in (1, 2):
        ma.adam_step(st, dev_p, to_device_grads(grads, "f32"), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        torch.cuda.synchronize()
        for i in range(2):
            compare_params(dev_p[i].cpu().numpy(), params[i], stats, f"t={t} tensor {i}")
        got = read_state(st)
        for nm, want in ost.buffers().items():
            # bit-exact codes, not the +-1 allowance of nearest rounding
            compare_buffer(nm, got[nm], want, True, stats, f"t={t}")
        if storage == "q8":
            mc = got["m_codes"].astype(np.int64)
            idx = np.array([i for i, _ in m_ties])
            assert np.array_equal(mc[idx], np.array([c for _, c in m_ties])), "m tie codes"
        vidx = seg1 + np.array([i for i, _ in v_ties])
        vwant = np.array([c for _, c in v_ties])
        assert np.array_equal(got["v_codes"][vidx].astype(np.int64), vwant), "v tie codes"
        if ams:  # the running maximum equals v here (w_old <= v at both steps)
            assert np.array_equal(got["vmax_codes"][vidx].astype(np.int64), vwant)
    log(f"ties to even, {storage} ams={ams} pct={pct}: {len(m_ties)} m and {len(v_ties)} v "
        f"tie elements; {stats}")
    st.destroy()
