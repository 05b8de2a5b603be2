"""The stored step examples (tests/golden/step_examples.json, written by
tests/golden/make_golden.py from the oracle) are reproduced bit for bit by
the oracle as it stands: any change of its arithmetic shows here and must
come with a regenerated fixture and the reading that justifies it."""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "step_examples.json")))


def f32(hexes):
    return np.array([int(h, 16) for h in hexes], np.uint32).view(np.float32)


@pytest.mark.parametrize("name", sorted(GOLDEN["cases"]))
def test_oracle_reproduces_the_stored_examples(orc, name):
    case = GOLDEN["cases"][name]
    numels = GOLDEN["numels"]
    st = orc.OracleState(numels, case["storage"], amsgrad=case["amsgrad"])
    params = [f32(p).copy() for p in GOLDEN["params0"]]
    for t, want in enumerate(case["steps"], start=1):
        grads = [f32(g) for g in GOLDEN["grads"][t - 1]]
        st.step(params, grads, t=t, stochastic=case["stochastic"], percentile=case["percentile"],
                seed=GOLDEN["seed"], decoupled=case["decoupled"], **GOLDEN["hparams"])
        for k, p in enumerate(params):
            assert np.array_equal(p.view(np.uint32), f32(want["params"][k]).view(np.uint32)), (t, k)
        bufs = st.buffers()
        assert set(bufs) == set(want) - {"params"}
        for nm, buf in bufs.items():
            ref = f32(want[nm]) if buf.dtype == np.float32 else np.array(want[nm], buf.dtype)
            assert np.array_equal(buf.view(np.uint8), ref.view(np.uint8)), (t, nm)
