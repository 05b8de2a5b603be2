"""Seeded synthetic workloads for the compressed-moment Adam step.

This module holds parameter-set shapes, hyperparameters and seeded random
draws only -- none of the optimizer's arithmetic -- and is the one piece of
code that both the oracle side and the HIP side of the tests and benchmark
use (they feed the same arrays to both).

Parameter sets:
  single    one fp32 tensor of 1,048,576 params
  vit_base  ViT-B/16 as the BF16-Adam page measures it (86.5M params): patch
            embedding, class token, position table, 12 encoder blocks,
            final LayerNorm and a 1000-way head -- 152 tensors, 86,567,656
            params
  gpt_1p3b  GPT-style, 24 layers, hidden 2048, MLP 8192, vocab 50304, context
            2048, tied head (1,315,819,520 params) plus a set of ragged 1-D
            tensors {1, 17, 1000, 2047, 2049, 6001} so that tail blocks occur
  llama_7b  32 layers, hidden 4096, MLP 11008, vocab 32000, untied head
            (6,738,415,616 params)
  ragged    small multi-tensor set spanning several blocks and every tail
            shape the kernels treat specially

Value recipes: params ~ N(0, 0.02) fp32; grads fp32 N(0, 1e-3), or bf16
(round-to-nearest-even cast) of Student-t(3)*1e-3 (gpt_1p3b), or of
N(0, 1e-3) with a uniform 0.1% of entries multiplied by 100 (llama_7b).
Host draws use numpy's default_rng seeded with [config id, step]; device
draws (full-size sets) use a torch CUDA generator seeded from the same pair.
"""
from dataclasses import dataclass, field

import numpy as np


# --------------------------------------------------------------------------
# parameter-set shapes
# --------------------------------------------------------------------------
def single_shapes():
    return [("w", (1048576,))]


def vit_base_shapes():
    d, mlp, heads_out = 768, 3072, 1000
    s = [("patch_embed.weight", (d, 3, 16, 16)), ("patch_embed.bias", (d,)),
         ("cls_token", (1, 1, d)), ("pos_embed", (1, 197, d))]
    for i in range(12):
        b = f"blocks.{i}."
        s += [(b + "norm1.weight", (d,)), (b + "norm1.bias", (d,)),
              (b + "attn.qkv.weight", (3 * d, d)), (b + "attn.qkv.bias", (3 * d,)),
              (b + "attn.proj.weight", (d, d)), (b + "attn.proj.bias", (d,)),
              (b + "norm2.weight", (d,)), (b + "norm2.bias", (d,)),
              (b + "mlp.fc1.weight", (mlp, d)), (b + "mlp.fc1.bias", (mlp,)),
              (b + "mlp.fc2.weight", (d, mlp)), (b + "mlp.fc2.bias", (d,))]
    s += [("norm.weight", (d,)), ("norm.bias", (d,)),
          ("head.weight", (heads_out, d)), ("head.bias", (heads_out,))]
    return s


GPT_TAIL_SIZES = (1, 17, 1000, 2047, 2049, 6001)


def gpt_1p3b_shapes(with_tail_set=True):
    d, mlp, vocab, ctx = 2048, 8192, 50304, 2048
    s = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(24):
        b = f"h.{i}."
        s += [(b + "ln_1.weight", (d,)), (b + "ln_1.bias", (d,)),
              (b + "attn.c_attn.weight", (d, 3 * d)), (b + "attn.c_attn.bias", (3 * d,)),
              (b + "attn.c_proj.weight", (d, d)), (b + "attn.c_proj.bias", (d,)),
              (b + "ln_2.weight", (d,)), (b + "ln_2.bias", (d,)),
              (b + "mlp.c_fc.weight", (d, mlp)), (b + "mlp.c_fc.bias", (mlp,)),
              (b + "mlp.c_proj.weight", (mlp, d)), (b + "mlp.c_proj.bias", (d,))]
    s += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    if with_tail_set:
        s += [(f"tail.{n}", (n,)) for n in GPT_TAIL_SIZES]
    return s


def llama_7b_shapes():
    d, mlp, vocab = 4096, 11008, 32000
    s = [("embed_tokens.weight", (vocab, d))]
    for i in range(32):
        b = f"layers.{i}."
        s += [(b + "self_attn.q_proj.weight", (d, d)), (b + "self_attn.k_proj.weight", (d, d)),
              (b + "self_attn.v_proj.weight", (d, d)), (b + "self_attn.o_proj.weight", (d, d)),
              (b + "mlp.gate_proj.weight", (mlp, d)), (b + "mlp.up_proj.weight", (mlp, d)),
              (b + "mlp.down_proj.weight", (d, mlp)),
              (b + "input_layernorm.weight", (d,)),
              (b + "post_attention_layernorm.weight", (d,))]
    s += [("norm.weight", (d,)), ("lm_head.weight", (vocab, d))]
    return s


def zero1_shard_shapes(shapes, rank, n_ranks, block=2048):
    """Rank `rank`'s share of a parameter set under ZeRO-1 block sharding:
    the blocks of all tensors, in order, split into n_ranks contiguous runs of
    (nearly) equal length; a tensor cut by a run boundary contributes the
    1-D slice of its flattened elements that lies in the run (cuts fall on
    block boundaries, so every block of the shard is a block of the set)."""
    sizes = [int(np.prod(shp)) for _, shp in shapes]
    total = sum((n + block - 1) // block for n in sizes)
    lo, hi = total * rank // n_ranks, total * (rank + 1) // n_ranks
    out, first = [], 0  # first: global index of the tensor's first block
    for (name, _), n in zip(shapes, sizes):
        nb = (n + block - 1) // block
        b0, b1 = max(lo, first) - first, min(hi, first + nb) - first
        if b0 < b1:
            s0, s1 = b0 * block, min(n, b1 * block)
            out.append((f"{name}[{s0}:{s1}]", (s1 - s0,)))
        first += nb
    return out


def llama_7b_shard8_shapes():
    return zero1_shard_shapes(llama_7b_shapes(), 0, 8)


RAGGED_SIZES = (1, 3, 4, 5, 16, 17, 1000, 1023, 1024, 1025, 2047, 2048, 2049,
                4096, 6001, 12289)


def ragged_shapes():
    return [(f"r{i}", (n,)) for i, n in enumerate(RAGGED_SIZES)]


def numels_of(shapes):
    return [int(np.prod(s)) for _, s in shapes]


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclass
class Config:
    cfg_id: int
    name: str
    shapes_fn: object
    storage: str            # "bf16" | "q8" | "q8_v_only"
    grad_dtype: str         # "f32" | "bf16"
    grad_dist: str          # "normal" | "student_t3" | "normal_outliers" (| "few_levels", host only)
    steps: int
    hp: dict = field(default_factory=dict)
    amsgrad: bool = False   # the state keeps the running maximum of v

    def shapes(self):
        return self.shapes_fn()

    def numels(self):
        return numels_of(self.shapes())


_ADAMW = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
              decoupled=True, stochastic=False, percentile=None, seed=42)

CONFIGS = {
    "single_q8": Config(1, "single_q8", single_shapes, "q8", "f32", "normal", 10,
                        dict(_ADAMW)),
    "vit_bf16": Config(2, "vit_bf16", vit_base_shapes, "bf16", "f32", "normal", 10,
                       dict(_ADAMW)),
    "vit_q8": Config(3, "vit_q8", vit_base_shapes, "q8", "f32", "normal", 10,
                     dict(_ADAMW)),
    "gpt1p3b_q8_sr": Config(4, "gpt1p3b_q8_sr", gpt_1p3b_shapes, "q8", "bf16", "student_t3",
                            5, dict(_ADAMW, weight_decay=0.1, stochastic=True, seed=1234)),
    "llama7b_mf32_vq8_pct": Config(5, "llama7b_mf32_vq8_pct", llama_7b_shapes, "q8_v_only",
                                   "bf16", "normal_outliers", 3,
                                   dict(_ADAMW, percentile=99.9)),
    # one GPU's share of the Llama-7B set under 8-way ZeRO-1 block sharding
    "llama7b_shard8_mf32_vq8_pct": Config(6, "llama7b_shard8_mf32_vq8_pct", llama_7b_shard8_shapes,
                                          "q8_v_only", "bf16", "normal_outliers", 3,
                                          dict(_ADAMW, percentile=99.9)),
}


# --------------------------------------------------------------------------
# host draws (numpy)
# --------------------------------------------------------------------------
def bf16_bits_of(x32):
    """Round-to-nearest-even bf16 bit patterns of a float32 array, via the
    PyTorch CPU cast (input preparation only)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_params(cfg_id, numels):
    rng = np.random.default_rng([cfg_id, 0])
    out = []
    for n in numels:
        out.append(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    return out


def host_grads(cfg_id, numels, t, dist="normal", dtype="f32"):
    rng = np.random.default_rng([cfg_id, t])
    out = []
    for n in numels:
        if dist == "normal":
            g = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
        elif dist == "student_t3":
            g = (rng.standard_t(3, size=n) * 1e-3).astype(np.float32)
        elif dist == "normal_outliers":
            g = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
            hit = rng.random(n) < 1e-3
            g[hit] *= np.float32(100.0)
        elif dist == "few_levels":
            # five gradient values: the moments of a block tie in large groups
            g = (rng.integers(-2, 3, size=n) * 1e-3).astype(np.float32)
        else:
            raise ValueError(dist)
        out.append(bf16_bits_of(g) if dtype == "bf16" else g)
    return out


# --------------------------------------------------------------------------
# device draws (torch, for the full-size sets)
# --------------------------------------------------------------------------
def _gen(cfg_id, t, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(cfg_id) * 1_000_003 + int(t))
    return g


def device_params(cfg_id, numels, device="cuda"):
    """List of fp32 device tensors ~N(0, 0.02)."""
    import torch
    gen = _gen(cfg_id, 0, device)
    return [torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(0.02)
            for n in numels]


def device_grads(cfg_id, numels, t, dist="normal", dtype="f32", device="cuda", out=None):
    """List of device grad tensors (fp32 or bf16) for step t; fills `out` in
    place when given."""
    import torch
    gen = _gen(cfg_id, t, device)
    res = []
    for k, n in enumerate(numels):
        if dist == "normal":
            g = torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(1e-3)
        elif dist == "student_t3":
            z = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
            c = torch.zeros(n, device=device, dtype=torch.float32)
            for _ in range(3):
                w = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
                c.addcmul_(w, w)
            g = z.div_(c.div_(3.0).sqrt_()).mul_(1e-3)
            del c
        elif dist == "normal_outliers":
            g = torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(1e-3)
            hit = torch.rand(n, generator=gen, device=device) < 1e-3
            g = torch.where(hit, g * 100.0, g)
            del hit
        else:
            raise ValueError(dist)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        if out is not None:
            out[k].copy_(g)
            res.append(out[k])
        else:
            res.append(g.to(tdt) if tdt != torch.float32 else g)
        del g
    return res
