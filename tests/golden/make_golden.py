"""Writes tests/golden/step_examples.json: small self-contained examples of
the step (inputs and the oracle's outputs after each of three steps) for
every storage mode, rounding and AMSGrad setting.  Calls only oracle/.

The pages print no worked example, so these are not page values: they pin
the oracle's outputs against silent change (tests/test_golden.py re-derives
them on the CPU) and give the GPU path expected bits stored in the
repository (tests/test_gpu_parity.py).  Regenerate only for a change of the
oracle's arithmetic that a reading of the pages justifies."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402

NUMELS = [19, 45, 5]
STEPS = 3
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
CASES = [  # name, storage, stochastic, percentile, amsgrad, decoupled
    ("bf16", "bf16", False, None, False, True),
    ("bf16_amsgrad_l2", "bf16", False, None, True, False),
    ("q8_rne", "q8", False, None, False, True),
    ("q8_sr", "q8", True, None, False, True),
    ("q8_sr_amsgrad", "q8", True, None, True, True),
    ("q8_pct50", "q8", False, 50.0, False, True),
    ("q8_v_only_sr_pct", "q8_v_only", True, 99.9, False, True),
]


def hexs(a):
    return [format(int(x), "08x") for x in np.asarray(a, np.float32).view(np.uint32)]


def inputs():
    rng = np.random.default_rng(20250101)
    p0 = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in NUMELS]
    gs = [[(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in NUMELS] for _ in range(STEPS)]
    return p0, gs


def main():
    p0, gs = inputs()
    out = {"numels": NUMELS, "hparams": HP, "seed": 42,
           "params0": [hexs(p) for p in p0], "grads": [[hexs(g) for g in step] for step in gs],
           "cases": {}}
    for name, storage, sr, pct, ams, dec in CASES:
        st = oracle.OracleState(NUMELS, storage, amsgrad=ams)
        params = [p.copy() for p in p0]
        steps = []
        for t in range(1, STEPS + 1):
            st.step(params, gs[t - 1], t=t, stochastic=sr, percentile=pct, seed=42, decoupled=dec, **HP)
            rec = {"params": [hexs(p) for p in params]}
            for k, buf in st.buffers().items():
                rec[k] = hexs(buf) if buf.dtype == np.float32 else [int(x) for x in buf]
            steps.append(rec)
        out["cases"][name] = {"storage": storage, "stochastic": sr, "percentile": pct,
                              "amsgrad": ams, "decoupled": dec, "steps": steps}
    with open(os.path.join(HERE, "step_examples.json"), "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
