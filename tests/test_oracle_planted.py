"""Planted mistakes: each test builds a copy of the oracle with one plausible
error written into it (on the CPU, in a temporary directory) and runs the
oracle's pin suite against that copy through ORACLE_LIBRARY.  The pins must
catch every one of them: a pin set that passes a broken oracle pins nothing.

Mistakes planted (one per build):
  tie_away      nearest rounding with ties away from zero (roundf) instead of
                ties to even
  recip_128     codebook step 1/128 instead of 1/qmax
  draw_halves   first and second moment take each other's 16-bit draw halves
  max_draw_word the AMSGrad maximum's draws from word i mod 4 instead of
                (i / 2) mod 4
  eps_in_root   eps added under the square root instead of after it
  rank_ceil     percentile entry ceil(p/100 (n-1)) instead of floor
  no_omb1       first-moment EMA without the (1 - beta1) factor
  bf16_ties_up  bf16 packing rounds exact halves up instead of to even
  weyl_key      Philox key bumped with the wrong Weyl constant
  v_signed      the 8-bit step decodes its stored v codes in the signed
                alphabet (step 1 is right, every later step is not)
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(ROOT, "oracle", "adam_oracle.c")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")

PIN_TESTS = ["tests/test_oracle_encodings.py", "tests/test_oracle_quant.py",
             "tests/test_oracle_adam.py", "tests/test_oracle_amsgrad.py", "tests/test_golden.py"]

# (name, exact source text, replacement)
MUTATIONS = [
    ("tie_away", "k = (int32_t)rintf(y);", "k = (int32_t)roundf(y);"),
    ("recip_128", "const float R = 1.0f / qmax;", "const float R = 1.0f / 128.0f;"),
    ("draw_halves", "half_hi = which == 1;", "half_hi = which != 1;"),
    ("max_draw_word", "word = w[(i >> 1) & 3u];", "word = w[i & 3u];"),
    ("eps_in_root", "fmaf(sqrtf(w), ibc2, h->eps)", "fmaf(sqrtf(w + h->eps), ibc2, 0.0f)"),
    ("rank_ceil", "return (int64_t)floor(frac * (double)(n - 1));",
     "return (int64_t)ceil(frac * (double)(n - 1));"),
    ("no_omb1", "fmaf(h->beta1, m_old, omb1 * g)", "fmaf(h->beta1, m_old, g)"),
    ("bf16_ties_up", "(dropped == 0x8000u && (upper & 1u))", "(dropped == 0x8000u)"),
    ("weyl_key", "k[0] += 0x9E3779B9u;", "k[0] += 0x9E3779B7u;"),
    ("v_signed", "m_old = orc_dequantize(q->mq[j], q->ms[0], 1);\n            v_old = orc_dequantize(q->vq[j], q->vs[0], 0);",
     "m_old = orc_dequantize(q->mq[j], q->ms[0], 1);\n            v_old = orc_dequantize(q->vq[j], q->vs[0], 1);"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    with open(SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"{name}: the line to mutate is not unique or is gone"
    mutated = tmp_path / f"oracle_{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"liboracle_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-o", str(lib), str(mutated), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIBRARY=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_TESTS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode != 0 and " failed" in r.stdout, (
        f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}")
