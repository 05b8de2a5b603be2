"""GPU-vs-oracle comparison helpers for the parity tests (not a test module).

Criteria (per element, after every step):
  bf16 moments ........ bit-exact
  8-bit codes ......... stochastic rounding: bit-exact; nearest-even: at
                        least 99.99% exact and every code within +-1
  scales .............. bit-exact
  fp32 first moment ... bit-exact (same operation order on both sides)
  params .............. |p_gpu - p_ref| / max(|p_ref|, 1e-6) <= 1e-5
The kernels and the oracle perform the same fp32 operations in the same
order with correctly rounded division and square root, so in practice every
quantity is expected to match bit for bit; the counts of exact matches are
reported alongside the assertions.
"""
import numpy as np
import torch

import memory_efficient_adam_amd as ma
import oracle
import workloads

PARAM_RTOL = 1e-5
PARAM_FLOOR = 1e-6
RNE_CODE_EXACT_FRACTION = 0.9999


def to_device_grads(host_grads, grad_dtype):
    out = []
    for g in host_grads:
        if grad_dtype == "bf16":
            out.append(torch.from_numpy(g.view(np.int16)).cuda().view(torch.bfloat16))
        else:
            out.append(torch.from_numpy(g).cuda())
    return out


def read_state(st):
    """All state buffers as numpy arrays named like the oracle's."""
    names = {"bf16": ["m_bf16", "v_bf16"], "q8": ["m_codes", "v_codes", "m_scale", "v_scale"],
             "q8_v_only": ["m_f32", "v_codes", "v_scale"]}[st.storage]
    if st.amsgrad:
        names += ["vmax_bf16"] if st.storage == "bf16" else ["vmax_codes", "vmax_scale"]
    out = {}
    for nm in names:
        t = ma.adam_state_read(st, nm)
        a = t.cpu().numpy()
        if nm.endswith("bf16"):
            a = a.view(np.uint16)
        out[nm] = a
    return out


class Stats:
    def __init__(self):
        self.params = 0
        self.params_exact = 0
        self.max_rel = 0.0
        self.codes = 0
        self.codes_exact = 0

    def __repr__(self):
        return (f"params exact {self.params_exact}/{self.params} (max rel {self.max_rel:.3g}), "
                f"codes exact {self.codes_exact}/{self.codes}")


def compare_params(got, want, stats, where=""):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    rel = np.abs(got.astype(np.float64) - want) / np.maximum(np.abs(want), PARAM_FLOOR)
    stats.params += got.size
    stats.params_exact += int(np.sum(got.view(np.uint32) == want.view(np.uint32)))
    if got.size:
        stats.max_rel = max(stats.max_rel, float(rel.max()))
    assert np.all(rel <= PARAM_RTOL), f"{where}: param rel err {rel.max():.3g}"


def compare_buffer(name, got, want, stochastic, stats, where=""):
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if name.endswith("codes"):
        g = got.astype(np.int32)
        w = want.astype(np.int32)
        stats.codes += g.size
        exact = int(np.sum(g == w))
        stats.codes_exact += exact
        if stochastic:
            assert exact == g.size, f"{where}: {name} {g.size - exact} codes differ (SR: must be exact)"
        else:
            assert np.all(np.abs(g - w) <= 1), f"{where}: {name} code off by more than 1"
            assert exact >= RNE_CODE_EXACT_FRACTION * g.size, f"{where}: {name} {exact}/{g.size} exact"
    else:
        # bf16 moments, fp32 first moment and scales: bit-exact
        gv = got.view(f"u{got.itemsize}")
        wv = want.astype(got.dtype).view(f"u{got.itemsize}")
        diff = np.nonzero(gv != wv)[0]
        assert diff.size == 0, (f"{where}: {name} differs at {diff.size} entries, first "
                                f"{diff[:6]} got {got[diff[:3]]} want {want[diff[:3]]}")


def run_full_parity(numels, storage, grad_dtype, steps, hp, cfg_id=1, stats=None,
                    grad_dist="normal", check_every_step=True, params=None, amsgrad=False):
    """Full element-by-element comparison over `steps` steps from zero state."""
    stats = stats or Stats()
    params = params if params is not None else workloads.host_params(cfg_id, numels)
    dev_p = [torch.from_numpy(p.copy()).cuda() for p in params]
    st = ma.adam_state_create(numels, storage, grad_dtype, amsgrad=amsgrad)
    ost = oracle.OracleState(numels, storage, grad_bf16=(grad_dtype == "bf16"), amsgrad=amsgrad)
    for t in range(1, steps + 1):
        grads = workloads.host_grads(cfg_id, numels, t, dist=grad_dist, dtype=grad_dtype)
        ma.adam_step(st, dev_p, to_device_grads(grads, grad_dtype), t=t, **hp)
        ost.step(params, grads, t=t, **hp)
        if check_every_step or t == steps:
            torch.cuda.synchronize()
            for k in range(len(numels)):
                compare_params(dev_p[k].cpu().numpy(), params[k], stats, f"t={t} tensor {k}")
            got = read_state(st)
            for nm, want in ost.buffers().items():
                compare_buffer(nm, got[nm], want, hp.get("stochastic", False), stats, f"t={t}")
    st.destroy()
    return stats


# --------------------------------------------------------------------------
# full-size sets checked on a sample of blocks
# --------------------------------------------------------------------------
def block_table(numels):
    """(tensor, local start, length, flat index) of every block, in order."""
    blocks = []
    seg = 0
    for k, n in enumerate(numels):
        for s in range(0, n, 2048):
            blocks.append((k, s, min(2048, n - s), seg + s))
        seg += oracle.pad16(n)
    return blocks


def sample_blocks(blocks, n_random, seed):
    rng = np.random.default_rng(seed)
    tails = [i for i, b in enumerate(blocks) if b[2] < 2048]
    firsts = [i for i, b in enumerate(blocks) if b[1] == 0][:50]
    pick = set(tails + firsts + [0, len(blocks) - 1])
    pick.update(int(i) for i in rng.choice(len(blocks), min(n_random, len(blocks)),
                                           replace=False))
    return sorted(pick)


def _gather(tensors, sel):
    t = torch.cat([tensors[k][s:s + n] for k, s, n, _ in sel])
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _split(flat, sel):
    out = []
    o = 0
    for _, _, n, _ in sel:
        out.append(flat[o:o + n].copy())
        o += n
    return out


def run_sampled_parity(cfg, steps=None, n_random=800, log=print):
    """Full-size workload on the GPU in the benchmark's launch configuration;
    the oracle follows a sample of blocks (all tail blocks included) from the
    same inputs and the same zero state."""
    numels = cfg.numels()
    hp = dict(cfg.hp)
    steps = steps or cfg.steps
    blocks = block_table(numels)
    idx = sample_blocks(blocks, n_random, cfg.cfg_id)
    sel = [blocks[i] for i in idx]
    stats = Stats()
    params = workloads.device_params(cfg.cfg_id, numels)
    host_p = _split(_gather(params, sel), sel)
    gdt = torch.bfloat16 if cfg.grad_dtype == "bf16" else torch.float32
    grads = [torch.empty(n, dtype=gdt, device="cuda") for n in numels]
    st = ma.adam_state_create(numels, cfg.storage, cfg.grad_dtype, amsgrad=cfg.amsgrad)
    ob = oracle.OracleBlocks([(n, gidx) for _, _, n, gidx in sel], cfg.storage,
                             grad_bf16=(cfg.grad_dtype == "bf16"), amsgrad=cfg.amsgrad)
    for t in range(1, steps + 1):
        workloads.device_grads(cfg.cfg_id, numels, t, dist=cfg.grad_dist,
                               dtype=cfg.grad_dtype, out=grads)
        host_g = _split(_gather(grads, sel), sel)
        ma.adam_step(st, params, grads, t=t, **hp)
        ob.step(host_p, host_g, t=t, **hp)
        torch.cuda.synchronize()
        got_p = _split(_gather(params, sel), sel)
        for i in range(len(sel)):
            compare_params(got_p[i], host_p[i], stats, f"t={t} block {idx[i]}")
        for nm, want in ob.buffers().items():
            full = ma.adam_state_read(st, nm)
            if nm.endswith("scale"):
                got = full[torch.tensor(idx, device="cuda")].cpu().numpy()
                w = want
            else:
                got = _gather([full], [(0, g, n, g) for _, _, n, g in sel])
                w = np.concatenate([want[ob.block_slice(i)] for i in range(len(sel))])
            del full
            compare_buffer(nm, got, w, hp.get("stochastic", False), stats, f"t={t}")
        log(f"  {cfg.name} t={t}: {len(sel)} sampled blocks match ({stats})")
    st.destroy()
    del params, grads
    torch.cuda.empty_cache()
    return stats
