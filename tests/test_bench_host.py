"""Host-side checks of bench.py (no GPU): the refusal of more than one GPU, the
algorithmic bytes the roofline divides by, and the CPU-baseline record."""
import dataclasses
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    # the step needs no exchange between GPUs and the benchmark measures one:
    # --gpus 2 exits with status 2 and a message, printing no bench line
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


# What one step must move, per parameter and per 2048-element block, written
# out from the storage of each set: params read and written (4 + 4), grads read
# (fp32 4, bf16 2), each moment read and written (bf16 2 + 2, 8-bit 1 + 1, fp32
# 4 + 4), and each 8-bit moment's block scale read and written (4 + 4).
#   name, AMSGrad, bytes per parameter, bytes per block
EXPECTED = [
    ("vit_bf16", False, 8 + 4 + (2 + 2) + (2 + 2), 0),
    ("vit_bf16", True, 8 + 4 + (2 + 2) + (2 + 2) + (2 + 2), 0),
    ("vit_q8", False, 8 + 4 + (1 + 1) + (1 + 1), 8 + 8),
    ("gpt1p3b_q8_sr", False, 8 + 2 + (1 + 1) + (1 + 1), 8 + 8),
    ("gpt1p3b_q8_sr", True, 8 + 2 + (1 + 1) + (1 + 1) + (1 + 1), 8 + 8 + 8),
    ("llama7b_mf32_vq8_pct", False, 8 + 2 + (4 + 4) + (1 + 1), 8),
    ("llama7b_mf32_vq8_pct", True, 8 + 2 + (4 + 4) + (1 + 1) + (1 + 1), 8 + 8),
]


@pytest.mark.parametrize("name,ams,per_param,per_block", EXPECTED,
                         ids=[f"{e[0]}{'-amsgrad' if e[1] else ''}" for e in EXPECTED])
def test_algorithmic_bytes(name, ams, per_param, per_block):
    cfg = workloads.CONFIGS[name]
    if ams:
        cfg = dataclasses.replace(cfg, amsgrad=True)
    numels = cfg.numels()
    blocks = sum((n + 2047) // 2048 for n in numels)
    assert bench.algorithmic_bytes(cfg) == sum(numels) * per_param + blocks * per_block


def test_cpu_baseline_record():
    # a few blocks of the 8-bit ViT-Base set: the record the bench line
    # carries, timed on one thread and on the host threads the process may use
    cfg = workloads.CONFIGS["vit_q8"]
    rec = bench.cpu_baseline(cfg, dict(cfg.hp), max_blocks=6, min_seconds=0.01, max_steps=2)
    assert rec["kind"] == "oracle" and rec["unit"] == "Gparams/s"
    assert rec["cores"] == bench.host_threads() >= 1
    assert rec["value"] > 0 and rec["single_thread"]["value"] > 0
    assert rec["single_thread"]["cores"] == 1
    assert "6 of the vit_q8 set's blocks" in rec["sample"]
