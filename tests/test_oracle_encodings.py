"""Pins for the oracle's encodings: bf16 packing and the Philox stream.

bf16 is checked against PyTorch's CPU float->bfloat16 cast (round to nearest,
ties to even) on every upper-half bit pattern combined with the lower halves
that decide rounding (0, 1, just below / at / just above one half, all ones,
plus random ones).  Philox4x32-10 and the stochastic-rounding draw mapping
are checked against PyTorch's header-only philox_engine, compiled here with
g++ (a separate implementation of the SC'11 definition).
"""
import os
import subprocess

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_cast_on_all_upper_halves(orc):
    upper = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(7)
    lowers = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF] + list(
        rng.integers(0, 1 << 16, size=6))
    for lo in lowers:
        bits = upper | np.uint32(lo)
        x = bits.view(np.float32)
        got = orc.bf16_from_f32(x)
        want = _torch_bf16_bits(x)
        nan_in = np.isnan(x)
        # NaN inputs: both must produce a NaN pattern
        got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
        want_nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x007F) != 0)
        assert np.all(got_nan[nan_in]) and np.all(want_nan[nan_in])
        assert np.array_equal(got[~nan_in], want[~nan_in]), hex(lo)


def test_bf16_widening_is_exact(orc):
    h = np.arange(1 << 16, dtype=np.uint16)
    x = orc.f32_from_bf16(h)
    assert np.array_equal(x.view(np.uint32), h.astype(np.uint32) << 16)
    t = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    finite = np.isfinite(t)
    assert np.array_equal(x[finite].view(np.uint32), t[finite].view(np.uint32))


def test_bf16_ties_go_to_even(orc):
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)
    got = orc.bf16_from_f32(x)
    assert list(got) == [0x3F80, 0x3F82, 0xBF80]


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


def test_philox_block_matches_torch_engine(orc, philox_ref):
    rng = np.random.default_rng(11)
    triples = [(0, 0, 0), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1), (42, 1, 0), (1234, 5, 7)]
    triples += [tuple(int(v) for v in rng.integers(0, 2 ** 63, size=3, dtype=np.uint64))
                for _ in range(60)]
    want = philox_ref(triples)
    for (seed, sub, off), w in zip(triples, want):
        ctr = [off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        got = orc.philox4x32_10(ctr, key)
        assert np.array_equal(got, w), (seed, sub, off)


def test_sr_draws_follow_the_counter_mapping(orc, philox_ref):
    # element i at step t uses word (i mod 4) of philox(seed, subsequence=t,
    # offset=i/4); low half for the first moment, high half for the second
    for seed, t, gidx0 in [(42, 1, 0), (1234, 5, 2 ** 33 + 12), (7, 3, 2046)]:
        n = 40
        idx = np.arange(gidx0, gidx0 + n, dtype=np.uint64)
        groups = sorted(set(int(i) >> 2 for i in idx))
        words = dict(zip(groups, philox_ref([(seed, t, g) for g in groups])))
        lo = orc.sr_draws(seed, t, gidx0, n, 0)
        hi = orc.sr_draws(seed, t, gidx0, n, 1)
        for j, i in enumerate(idx):
            w = int(words[int(i) >> 2][int(i) & 3])
            assert lo[j] == (w & 0xFFFF) and hi[j] == (w >> 16)


def test_sr_draws_are_uniform(orc):
    d = orc.sr_draws(99, 1, 0, 1 << 18, 0).astype(np.int64)
    counts = np.bincount(d >> 12, minlength=16)
    expected = d.size / 16
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    assert chi2 < 45.0  # 15 dof, p ~ 1e-4
