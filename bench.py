"""Benchmark: one compressed-moment Adam step over a full parameter set.

A step is one adam_step call through the C ABI -- one kernel launch over
every tensor of the set (dequantize / bias-corrected update / block
statistic / requantize, or the bf16-moment variant) -- on synthetic inputs
already resident in HBM.  Headline workload (`value`): the ViT-Base shaped
set (152 tensors, 86,567,656 fp32 params, fp32 grads ~N(0, 1e-3)) with bf16
moments.  With no --config the same JSON line also carries `modes`: the
8-bit sets timed the same way -- ViT-Base with 8-bit m and v, the GPT-1.3B
shaped set with Philox stochastic rounding and bf16 grads, the Llama-7B
shaped set with fp32 m, 8-bit v and the 99.9th-percentile scale; each of
these warms up for at least 0.2 s (and at least --warmup steps) before its
--steps timed steps, past the shader clock's dip at the start of a burst.
Other sets: --config (see workloads.CONFIGS).

Each record: Gparams/s, the roofline of the step kernel (algorithmic bytes
per launch / average launch time from HIP events on the launch stream,
against the 8 TB/s HBM peak; HBM traffic from rocprofv3 FETCH_SIZE /
WRITE_SIZE counters when a committed counter summary matches the current
kernel source; the stream probe's rate for the same blocks on this box, the
access pattern's ceiling) and the CPU oracle timed on the same workload
recipe, once on one thread and once on all the host cores it may use
(threads over disjoint block ranges of the oracle's sampled-block entry
point).
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "memory_efficient_adam_amd", "csrc", f)
                  for f in ("adam_kernels.hip", "adam_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")

# algorithmic bytes per parameter (read + write) and per block (scales)
#   params 4+4, grads 4 (fp32) or 2 (bf16), moments read+write, scales 4+4 per
#   block per quantized moment; AMSGrad adds the running maximum of v, stored
#   as v is (bf16: 2+2 per parameter; 8-bit: 1+1 and a scale)
_MOMENT_BYTES = {"bf16": 8, "q8": 4, "q8_v_only": 10}
_SCALE_BYTES = {"bf16": 0, "q8": 16, "q8_v_only": 8}
_VMAX_BYTES = {"bf16": (4, 0), "q8": (2, 8), "q8_v_only": (2, 8)}


def algorithmic_bytes(cfg):
    numels = cfg.numels()
    n = sum(numels)
    blocks = sum(-(-k // 2048) for k in numels)
    g = 2 if cfg.grad_dtype == "bf16" else 4
    per_n = 8 + g + _MOMENT_BYTES[cfg.storage]
    per_b = _SCALE_BYTES[cfg.storage]
    if cfg.amsgrad:
        per_n += _VMAX_BYTES[cfg.storage][0]
        per_b += _VMAX_BYTES[cfg.storage][1]
    return n * per_n + blocks * per_b


def kernel_source_hash():
    """sha256 over the code of the sources that define the step kernel
    (comments and whitespace removed, so that editing a comment does not
    retire the counter readings)."""
    import re
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def traffic_for(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none for this workload or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(workload)
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def _block_list(numels, block=2048):
    """(length, flat index) of every block of a tensor list, tensor-major,
    tensors padded to 16 elements in the flat state (layout only)."""
    out, seg = [], 0
    for n in numels:
        for s0 in range(0, n, block):
            out.append((min(block, n - s0), seg + s0))
        seg += (n + 15) // 16 * 16
    return out


def host_threads():
    """Host cores the oracle may use: the process's CPU affinity, capped by
    OMP_NUM_THREADS when set (a shared host may allot a share of its cores)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(cfg, hp, max_blocks=None, min_seconds=8.0, max_steps=12):
    """The oracle, as it is, on the same workload recipe (host-generated
    inputs of the set's value laws; generation not timed): whole steps over
    every block of the set, or over a seeded sample of max_blocks blocks.
    Timed twice on the same inputs: single-threaded, and with the blocks
    split into contiguous ranges stepped concurrently by a thread pool (the
    oracle's C entry point runs without the interpreter lock).  Steps are
    repeated until min_seconds of single-threaded oracle time."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import workloads
    blocks = _block_list(cfg.numels())
    label = f"every block of the {cfg.name} set"
    if max_blocks is not None and len(blocks) > max_blocks:
        rng = np.random.default_rng([cfg.cfg_id, 7])
        pick = np.sort(rng.choice(len(blocks), max_blocks, replace=False))
        blocks = [blocks[i] for i in pick]
        label = f"a seeded sample of {max_blocks} of the {cfg.name} set's blocks"
    lens = [n for n, _ in blocks]
    n_params = sum(lens)
    grad_bf16 = cfg.grad_dtype == "bf16"
    threads = host_threads()
    bounds = [len(blocks) * k // threads for k in range(threads + 1)]
    ranges = [(bounds[k], bounds[k + 1]) for k in range(threads) if bounds[k + 1] > bounds[k]]

    def run(n_workers, steps_cap, seconds):
        """(Gparams/s, steps): steps t = 1, 2, ... over the same inputs until
        `seconds` of oracle time or `steps_cap` steps."""
        params = workloads.host_params(cfg.cfg_id, lens)
        parts = [oracle.OracleBlocks(blocks[a:b], cfg.storage, grad_bf16=grad_bf16,
                                     amsgrad=cfg.amsgrad) for a, b in ranges]
        elapsed, steps = 0.0, 0
        with ThreadPoolExecutor(max_workers=n_workers) as pool:
            while steps < steps_cap and elapsed < seconds:
                steps += 1
                grads = workloads.host_grads(cfg.cfg_id, lens, steps, dist=cfg.grad_dist,
                                             dtype=cfg.grad_dtype)
                t0 = time.perf_counter()
                futs = [pool.submit(part.step, params[a:b], grads[a:b], t=steps, **hp)
                        for part, (a, b) in zip(parts, ranges)]
                for f in futs:
                    f.result()
                elapsed += time.perf_counter() - t0
        return n_params * steps / elapsed / 1e9, steps

    one, steps = run(1, max_steps, min_seconds)
    many, _ = run(threads, steps, float("inf"))  # the same steps on every core
    return {"value": round(many, 5), "unit": "Gparams/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} step(s) over {label} ({n_params} params), the blocks split "
                      f"into {len(ranges)} contiguous ranges stepped by {threads} threads; "
                      "host-generated inputs of the workload's recipe, generation not timed",
            "single_thread": {"value": round(one, 5), "unit": "Gparams/s", "cores": 1}}


def apply_overrides(cfg, args):
    """The workload's hyperparameters with the command line's overrides."""
    hp = dict(cfg.hp)
    if args.static_scales:
        if cfg.storage == "bf16":
            sys.exit("bench.py: --static-scales applies to 8-bit storage only")
        hp["static_scales"] = True
    if args.nearest and args.stochastic:
        sys.exit("bench.py: --nearest and --stochastic exclude each other")
    if args.nearest or args.stochastic:
        if cfg.storage == "bf16":
            sys.exit("bench.py: --nearest / --stochastic apply to 8-bit storage only")
        hp["stochastic"] = bool(args.stochastic)
    if args.percentile is not None:
        if cfg.storage == "bf16":
            sys.exit("bench.py: --percentile applies to 8-bit storage only")
        hp["percentile"] = args.percentile
    return hp


def time_workload(cfg, hp, steps, warmup, grad_buffers, traffic_key=None, min_warmup_s=0.0):
    """Times `steps` back-to-back steps of one workload (after `warmup`
    untimed ones, continued in tens until the warmup has lasted
    `min_warmup_s`) with HIP events on the launch stream; inputs resident in
    HBM before the timed region.  Frees everything it allocated."""
    import torch
    import memory_efficient_adam_amd as ma
    import workloads
    numels = cfg.numels()
    n_params = sum(numels)
    params = workloads.device_params(cfg.cfg_id, numels)
    gsets = []
    for i in range(max(1, grad_buffers)):
        gsets.append(workloads.device_grads(cfg.cfg_id, numels, i + 1, dist=cfg.grad_dist,
                                            dtype=cfg.grad_dtype))
    st = ma.adam_state_create(numels, cfg.storage, cfg.grad_dtype, amsgrad=cfg.amsgrad)
    stream = torch.cuda.current_stream()
    t = 0
    w_start = time.perf_counter()
    for _ in range(warmup):
        t += 1
        ma.adam_step(st, params, gsets[t % len(gsets)], t=t, stream=stream, **hp)
    torch.cuda.synchronize()
    while time.perf_counter() - w_start < min_warmup_s:
        for _ in range(10):
            t += 1
            ma.adam_step(st, params, gsets[t % len(gsets)], t=t, stream=stream, **hp)
        torch.cuda.synchronize()
    warmed = t
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    # two events on the launch stream around the timed steps and nothing in
    # between: an event recorded between consecutive launches costs ~3 us a
    # step (1% of a ViT-Base step), so per-step times are left to the
    # kernel tracer
    start.record(stream)
    for _ in range(steps):
        t += 1
        ma.adam_step(st, params, gsets[t % len(gsets)], t=t, stream=stream, **hp)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = start.elapsed_time(end) / steps
    st.destroy()
    del params, gsets
    torch.cuda.empty_cache()

    sec = ms / 1e3
    alg = algorithmic_bytes(cfg)
    achieved = alg / sec / 1e9
    traffic = traffic_for(traffic_key) if traffic_key else None
    return {
        "value": round(n_params / sec / 1e9, 3),
        "unit": "Gparams/s",
        "steps": steps,
        "warmup": warmed,
        "ms_per_step": round(ms, 5),
        "wall_ms_per_step": round(wall * 1e3 / steps, 5),
        "config": {
            "workload": cfg.name,
            "params": n_params,
            "tensors": len(numels),
            "blocks": sum(-(-k // 2048) for k in numels),
            "storage": cfg.storage,
            "grad_dtype": cfg.grad_dtype,
            "stochastic_rounding": bool(hp.get("stochastic")),
            "percentile": hp.get("percentile"),
            "static_scales": bool(hp.get("static_scales")),
            "amsgrad": cfg.amsgrad,
            "block_size": 2048,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": (None if traffic is None else
                               "profiles/hbm_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE "
                               "of this kernel source on this workload, copy-calibrated"),
            "algorithmic_bytes_per_launch": alg,
        },
    }


PROBE_CAPS = (2, 3, 4, 5, 6, 8)


def time_stream_probe(cfg, steps, warmup, caps=PROBE_CAPS):
    """Times the stream probe over as many full blocks as the workload has
    blocks: the step's loads and stores without its arithmetic, at each
    residency cap (workgroups per CU; 8 = uncapped), with HIP events on the
    launch stream as for the step.  Its bytes per launch are its own (the
    workload's tail blocks counted as full)."""
    import torch
    from memory_efficient_adam_amd import stream_probe as sp
    n_blocks = sum(-(-k // 2048) for k in cfg.numels())
    bufs = sp.probe_buffers(n_blocks, cfg.grad_dtype, cfg.storage, cfg.amsgrad)
    for t in bufs.values():
        if t is not None:
            t.zero_()
    nbytes = sp.adam_stream_probe_bytes(n_blocks, cfg.grad_dtype, cfg.storage, cfg.amsgrad)
    stream = torch.cuda.current_stream()
    rates = {}
    for cap in caps:
        for _ in range(warmup):
            sp.adam_stream_probe(bufs, n_blocks, cfg.grad_dtype, cfg.storage, cfg.amsgrad, cap, stream)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            sp.adam_stream_probe(bufs, n_blocks, cfg.grad_dtype, cfg.storage, cfg.amsgrad, cap, stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        gbs = nbytes / (ms / 1e3) / 1e9
        rates[str(cap)] = {"ms_per_launch": round(ms, 5), "GB/s": round(gbs, 1),
                           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del bufs
    torch.cuda.empty_cache()
    best = max(rates, key=lambda c: rates[c]["GB/s"])
    return {"workload": cfg.name, "amsgrad": cfg.amsgrad, "blocks": n_blocks,
            "bytes_per_launch": nbytes, "steps": steps, "warmup": warmup,
            "resident_per_cu": rates, "best_cap": int(best), "best": rates[best]}


def pattern_ceiling(cfg, roofline, steps=20, warmup=5):
    """The stream probe on the workload's blocks on this box (best residency
    cap), and the step's fraction of it: the same bytes in the same pattern
    without the arithmetic, which is what the access pattern itself reaches
    here.  None if the probe library is missing or the probe fails (the
    step's own record stands without it)."""
    try:
        probe = time_stream_probe(cfg, steps, warmup)
    except Exception as e:  # a measurement aid: never let it cost the bench line
        print(f"bench.py: stream probe skipped ({type(e).__name__}: {e})", file=sys.stderr, flush=True)
        return None
    best = probe["best"]
    return {"best_cap": probe["best_cap"], "frac": best["frac"], "GB/s": best["GB/s"],
            "step_over_ceiling": round(roofline["frac"] / best["frac"], 4),
            "source": "bench.py stream probe: the step's loads and stores without its arithmetic"}


# the 8-bit workloads timed beside the headline (bf16-moment) workload, with
# the host-oracle sample size for each (blocks) and the grad buffers rotated
MODES = [("vit_q8", 4096, 4), ("gpt1p3b_q8_sr", 4096, 4), ("llama7b_mf32_vq8_pct", 4096, 2)]
TARGET_FRAC = 0.75
# The 8-bit records warm up for at least this long (and at least --warmup
# steps): a burst of steps from an idle GPU runs through a dip of the shader
# clock over its first ~10-60 ms, which the steady state of a training loop
# does not see; the timed steps are then the same --steps back-to-back steps.
MODE_MIN_WARMUP_S = 0.2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    help="one workload of workloads.CONFIGS (default: the ViT-Base bf16-moment "
                         "headline plus the 8-bit modes)")
    ap.add_argument("--no-modes", action="store_true",
                    help="headline workload only (skip the 8-bit mode records)")
    ap.add_argument("--grad-buffers", type=int, default=4,
                    help="distinct pre-generated gradient sets used in rotation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--static-scales", action="store_true",
                    help="8-bit sets: keep each block's scale once set")
    ap.add_argument("--amsgrad", action="store_true",
                    help="keep the running maximum of v (AMSGrad)")
    ap.add_argument("--percentile", type=float, default=None,
                    help="8-bit sets: percentile block statistic (e.g. 99.9) instead of the set's own")
    ap.add_argument("--nearest", action="store_true",
                    help="8-bit sets: nearest-even rounding instead of the set's stochastic rounding")
    ap.add_argument("--stochastic", action="store_true",
                    help="8-bit sets: Philox stochastic rounding instead of the set's nearest rounding")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the stream-probe ceiling of each record")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time torch's device copy of 4 GiB (counter calibration run)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="time the stream probe (the step's loads and stores, no arithmetic) "
                         "on the workload's blocks at several residency caps")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark measures one GPU only (the step needs no "
              "exchange between GPUs); run with --gpus 1", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import workloads

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 30  # 4 GiB of fp32 each way
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n}), flush=True)
        return

    if args.stream_probe:
        names = [args.config] if args.config else ["vit_bf16"] + [m[0] for m in MODES]
        out = []
        for name in names:
            pcfg = workloads.CONFIGS[name]
            if args.amsgrad:
                pcfg = dataclasses.replace(pcfg, amsgrad=True)
            out.append(time_stream_probe(pcfg, args.steps, args.warmup))
        print(json.dumps({"stream_probe": out}), flush=True)
        return

    headline = args.config is None
    cfg = workloads.CONFIGS[args.config or "vit_bf16"]
    if args.amsgrad:
        cfg = dataclasses.replace(cfg, amsgrad=True)
    hp = apply_overrides(cfg, args)
    # counter readings are taken per workload for its own kernel variant (a
    # percentile, nearest-rounding or AMSGrad run of a set has its own record
    # when one was taken; static scales have none)
    key = None if args.static_scales else cfg.name + ("_amsgrad" if cfg.amsgrad else "") + (
        "_nearest" if args.nearest else "") + ("_stochastic" if args.stochastic else "") + (
        "" if args.percentile is None else f"_percentile{args.percentile}")
    rec = time_workload(cfg, hp, args.steps, args.warmup, args.grad_buffers, key)
    out = {
        "metric": "Adam step Gparams/s + achieved HBM GB/s (% of 8 TB/s), 8-bit and bf16 moments",
        "value": rec["value"],
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "wall_ms_per_step": rec["wall_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": rec["config"],
        "roofline": rec["roofline"],
    }
    modes = []
    if headline and not args.no_modes:
        for name, sample_blocks, nbuf in MODES:
            mcfg = workloads.CONFIGS[name]
            m = time_workload(mcfg, dict(mcfg.hp), args.steps, args.warmup, nbuf, name,
                              min_warmup_s=MODE_MIN_WARMUP_S)
            m["warmup_min_seconds"] = MODE_MIN_WARMUP_S
            m["target_frac"] = TARGET_FRAC
            m["meets_target"] = m["roofline"]["frac"] >= TARGET_FRAC
            modes.append((m, mcfg, sample_blocks))
        out["modes"] = [m for m, _, _ in modes]
    if not args.no_ceiling:
        out["roofline"]["pattern_ceiling"] = pattern_ceiling(cfg, out["roofline"])
        for m, mcfg, _ in modes:
            m["roofline"]["pattern_ceiling"] = pattern_ceiling(mcfg, m["roofline"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, hp)
        for m, mcfg, sample_blocks in modes:
            m["cpu_baseline"] = cpu_baseline(mcfg, dict(mcfg.hp), max_blocks=sample_blocks,
                                             min_seconds=3.0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
