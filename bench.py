#!/usr/bin/env python3
"""Throughput of the block-diffusion denoise loop on one MI355X.

One timed "step" is one whole canvas: dg_canvas_init followed by
dg_generate_canvas, i.e. denoise steps (forward over every layer, fused LM head
with entropy/argmax, commit, re-noise) until the canvas is committed or the
48-step cap is reached.  Inputs (weights, prompt KV cache) are synthetic,
seeded, and resident in HBM before the timed region starts.

Prints one JSON line: canvas tokens/s (value), denoise steps/s, the roofline
fraction of the dominant kernel (timed live with HIP events on its own stream
inside the timed region), and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "canvas tokens/s & denoise steps/s, bs=1 256-tok canvas; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (scaled by 2.0 and 1.0, the factors a 1 GiB device copy reads) for the
# kernels as they are now; profiles/moe_gateup_c2_loop30_bf16.md has the
# commands.  An entry is dropped whenever its kernel changes.
MEASURED_TRAFFIC = {
    ("moe_gateup", "c2_loop30_bf16"): (365000 * 2 + 4249) * 1024,
}


def router_in_shared(cfg) -> bool:
    """Whether the library computes the router logits inside the shared
    gate/up launch: bf16 activations and shared weights (bf16 or mxfp4
    workloads: the latter keep a bf16 shared expert), K = d_model = 2048, at
    most 512 tokens, d_shared >= 1024 (the direct-load kernel's small-M SwiGLU
    shape)."""
    T = cfg.batch * cfg.canvas_len
    return (cfg.act_dtype == "bf16" and cfg.expert_dtype in ("bf16", "mxfp4", "mxfp4_a8") and cfg.d_model == 2048
            and T <= 512 and cfg.d_shared >= 1024)


def topk_in_shared(cfg) -> bool:
    """Whether the router top-k runs as extra workgroups of the shared-down
    launch: the logits come from the shared gate/up launch, the shared down is
    the direct-load kernel's small-M fp32 shape (K = d_shared = 2048), at most
    128 experts and top 8."""
    return router_in_shared(cfg) and cfg.d_shared == 2048 and cfg.n_experts <= 128 and cfg.top_k <= 8


def algorithmic(cfg, kernel: str):
    """(bytes, flops) one timed launch of `kernel` must move/perform, per layer and step
    (per step for the LM head and the commit).  Weights are read once; activations
    are counted once in and once out."""
    T = cfg.batch * cfg.canvas_len
    d, E, k, de, ds = cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_expert, cfg.d_shared
    A = cfg.attn_dim
    ab = 2 if cfg.act_dtype == "bf16" else 4

    def routed_bytes(rows, K):  # one expert matrix [rows][K] in its storage format, scales included
        if cfg.expert_dtype == "fp8":
            return rows * K + rows * 4
        if cfg.expert_dtype in ("mxfp4", "mxfp4_a8"):
            return rows * K // 2 + rows * K // 32
        return rows * K * ab
    wb = 1 if cfg.expert_dtype == "fp8" else 2   # shared expert (bf16 in mxfp4 workloads)
    if kernel == "moe_gateup":
        return E * routed_bytes(2 * de, d) + T * d * ab + T * k * de * ab, 2.0 * T * k * 2 * de * d
    if kernel == "moe_down":
        return E * routed_bytes(d, de) + T * k * de * ab + T * k * d * 4, 2.0 * T * k * de * d
    if kernel == "lm_head":
        return cfg.vocab * d * ab + T * d * ab, 2.0 * T * cfg.vocab * d
    if kernel == "attn":
        keys = cfg.prompt_len + cfg.canvas_len
        return (cfg.batch * keys * A * 2 * ab + 2 * T * A * ab,
                4.0 * cfg.batch * cfg.canvas_len * keys * A)
    if kernel == "qkv":
        return 3 * A * d * ab + T * d * ab + 3 * T * A * ab, 2.0 * T * 3 * A * d
    # router logits: E x d weights, fp32 logits out; in the shared gate/up
    # launch when router_in_shared(cfg), else a launch of their own
    rl_bytes, rl_flops = E * d * ab + T * E * 4, 2.0 * T * E * d
    fused = router_in_shared(cfg)
    topk_bytes = T * E * 4 + 2 * T * k * 4
    if kernel == "shared":  # gate/up + SwiGLU (+ router logits), then down (fp32 out) (+ router top-k)
        w = 3 * ds * d * wb + (3 * ds * 4 if wb == 1 else 0)
        b, f = w + T * d * ab + 2 * T * ds * ab + T * d * 4, 2.0 * T * 3 * ds * d
        if topk_in_shared(cfg):
            b += topk_bytes
        return (b + rl_bytes, f + rl_flops) if fused else (b, f)
    if kernel == "router":  # top-k over the logits (+ the router GEMM when it runs alone)
        b = topk_bytes
        return (b, 0.0) if fused else (b + rl_bytes + T * d * ab, rl_flops)
    if kernel == "commit":
        return T * (4 + 4 + 4 + 1) * 2, 0.0
    raise ValueError(kernel)


# bound each kernel class is judged against: dense contractions (intensity near or
# above the bf16 ridge) against the MFMA peak, the rest against HBM bandwidth
KERNEL_BOUND = {"attn": "mfma", "qkv": "mfma", "shared": "mfma", "lm_head": "mfma",
                "moe_gateup": "hbm", "moe_down": "hbm", "router": "hbm", "commit": "hbm"}


def roofline_entry(cfg, kernel, total_ms, launches):
    bytes_, flops = algorithmic(cfg, kernel)
    avg_s = total_ms / 1e3 / max(launches, 1)
    if KERNEL_BOUND[kernel] == "mfma":
        achieved, peak, unit = flops / avg_s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = bytes_ / avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    return {"bound": KERNEL_BOUND[kernel], "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "avg_launch_us": avg_s * 1e6, "launches": launches,
            "algorithmic_bytes_per_launch": bytes_, "algorithmic_flops_per_launch": flops,
            "hbm_gbs": bytes_ / avg_s / 1e9, "tflops": flops / avg_s / 1e12}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, cfg, steps_per_canvas: float, layers: int):
    """Oracle time for a sampled step: `layers` layers + LM head + commit,
    extrapolated to a full step and a full canvas."""
    import numpy as np

    from oracle import model as om

    cores = len(os.sched_getaffinity(0))
    # every weight the sample touches is converted to float64 on the host
    # before the clock starts: the time is the oracle's arithmetic alone
    W = om.Weights(inp, cache=True)
    tp = time.perf_counter()
    W.prefetch(layers)
    kv = om.KV(inp.kv_k[:layers], inp.kv_v[:layers], inp.kv_len, bf16=cfg.act_dtype == "bf16")
    st = om.init_state(cfg, cfg.seed)
    prec = om.Prec(cfg.act_dtype)
    log(f"[bench] oracle weights prefetched in {time.perf_counter() - tp:.1f} s")
    t0 = time.perf_counter()
    x = prec.act(W.embed_rows(st.tokens[0]))
    for l in range(layers):
        kvk, kvv = kv.get(l, 0)
        x, _, _ = om.layer_forward(x, W, l, kvk, kvv, kv.length, prec, cfg)
    t1 = time.perf_counter()
    hf = prec.act(om.rmsnorm(x, cfg.rms_eps))
    z = om.lm_head_logits(hf, W)
    H, a, _ = om.confidence(z)
    om.commit_select(H, a, st.tokens[0].copy(), st.committed[0].copy(), 0, cfg.max_steps,
                     cfg.threshold)
    t2 = time.perf_counter()
    per_layer = (t1 - t0) / layers
    t_step = per_layer * cfg.n_layers + (t2 - t1)
    t_canvas = t_step * steps_per_canvas
    return {
        "value": cfg.canvas_len / t_canvas,  # the oracle runs one canvas at a time
        "unit": "canvas tokens/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{layers} of {cfg.n_layers} layers + LM head + commit of one denoise step of "
                   f"canvas 0 ({t2 - t0:.1f} s measured); extrapolated x{cfg.n_layers}/{layers} "
                   f"layers and x{steps_per_canvas:g} steps per canvas"),
        "seconds_per_step": t_step,
    }


def routing_stats(model, canvas, kv, cfg):
    """Pairs routed to each expert in one denoise step (per layer, all canvases
    pooled): how many experts exceed a 32-token pass of the batch-1 routed
    kernels, and the largest count, averaged over the layers."""
    import torch

    from diffusion_decoding_amd import runtime as rt
    counts = torch.zeros(cfg.n_layers, cfg.n_experts, dtype=torch.int32, device="cuda")
    rt.denoise_step(model, canvas, kv, expert_counts=counts)
    c = counts.cpu()
    over = (c > 32).sum(1).float()
    return {"pairs_per_step_layer": int(c[0].sum()), "experts": cfg.n_experts,
            "mean_experts_over_32_pairs": float(over.mean()), "mean_max_pairs": float(c.max(1).values.float().mean()),
            "max_pairs": int(c.max()), "mean_unused_experts": float((c == 0).sum(1).float().mean())}


def free_gpu(*objs):
    import torch
    for o in objs:
        if hasattr(o, "close"):
            o.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def time_loop(cfg, canvases: int, warmup: int, kernels=()):
    """Whole canvases (init + denoise loop) of a prompt-KV workload; inputs resident.
    kernels: classes timed with HIP events over one extra canvas each, after the timed region."""
    import torch

    from diffusion_decoding_amd import _lib
    from diffusion_decoding_amd import runtime as rt
    from workloads import make_inputs

    log(f"[bench] generating inputs for {cfg.name} on the GPU")
    inp = make_inputs(cfg, device="cuda")
    model = rt.Model(inp)
    kv = rt.KVCache(inp.kv_k, inp.kv_v, inp.kv_len)
    canvas = rt.Canvas.empty(cfg.batch, cfg.canvas_len, cfg.seed)
    for _ in range(warmup):
        rt.canvas_init(model, canvas)
        rt.generate_canvas(model, canvas, kv)
    torch.cuda.synchronize()
    steps = 0
    t0 = time.perf_counter()
    for _ in range(canvases):
        rt.canvas_init(model, canvas)
        steps += rt.generate_canvas(model, canvas, kv)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kern = {}
    for name in kernels:
        _lib.dg_profile_kernel(model.handle, _lib.DG_PROF[name])
        rt.canvas_init(model, canvas)
        rt.generate_canvas(model, canvas, kv)
        ms, cnt = _lib.dg_profile_read(model.handle)
        kern[name] = roofline_entry(cfg, name, ms, cnt)
        e = kern[name]
        log(f"[kernels] {cfg.name} {name:11s} {e['avg_launch_us']:9.1f} us/launch  {e['hbm_gbs']:7.0f} GB/s  "
            f"{100 * e['frac']:5.1f}% of {e['bound']} peak")
    if kernels:
        _lib.dg_profile_kernel(model.handle, 0)
    free_gpu(model)
    del inp, kv, canvas
    free_gpu()
    toks = cfg.batch * cfg.canvas_len * canvases
    log(f"[bench] {cfg.name}: {canvases} canvases x batch {cfg.batch}, {steps} steps in {dt:.3f} s")
    out = {"workload": cfg.name, "batch": cfg.batch, "canvas": cfg.canvas_len, "prompt_kv": cfg.prompt_len,
           "expert_dtype": cfg.expert_dtype, "canvas_tokens_per_s": toks / dt, "denoise_steps_per_s": steps / dt,
           "ms_per_denoise_step": dt / steps * 1e3, "denoise_steps_per_canvas": steps / canvases}
    if kern:
        out["kernels"] = {n: {k: e[k] for k in ("bound", "frac", "achieved", "unit", "avg_launch_us",
                                                 "algorithmic_bytes_per_launch")} for n, e in kern.items()}
    return out


def time_mixed(cfg, refine: int = 3, commit_len: int = 256, prompt_len: int = 512, passes: int = 8,
               warmup: int = 2):
    """One serving batch in different phases, at the shapes of ``cfg``: `refine`
    canvases each denoised one step against its own prompt cache, one canvas
    commit (`commit_len` tokens appended after a prompt) and one prompt read
    (`prompt_len` tokens into an empty cache).  Times one dg_mixed_step pass
    over all of them against the same work as separate calls (a batch-1
    denoise step per canvas, a causal pass per append)."""
    import torch

    from diffusion_decoding_amd import runtime as rt
    from workloads import make_inputs

    n_req = refine + 2
    P, N = cfg.prompt_len, cfg.canvas_len
    cap = P + max(commit_len, prompt_len)
    c = cfg.replace(name=cfg.name + "_mixed", batch=n_req)
    log(f"[bench] generating inputs for {c.name} ({n_req} requests) on the GPU")
    inp = make_inputs(c, device="cuda", kv_capacity=cap)
    rows = refine * N + commit_len + prompt_len
    # workspace rows = max_batch x max_tokens must hold the whole pass
    model = rt.Model(inp, max_batch=refine, max_tokens=max(commit_len, prompt_len, -(-rows // refine)), max_kv=cap)
    kvs = [rt.KVCache(inp.kv_k[:, b:b + 1].clone(), inp.kv_v[:, b:b + 1].clone(), P) for b in range(n_req)]
    kvs[-1].length = 0
    canv = [rt.Canvas.empty(1, N, cfg.seed + b) for b in range(refine)]
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 7)
    t_commit = torch.randint(0, cfg.vocab, (commit_len,), generator=g, device="cuda", dtype=torch.int32)
    t_prompt = torch.randint(0, cfg.vocab, (prompt_len,), generator=g, device="cuda", dtype=torch.int32)
    base = [kv.length for kv in kvs]

    def reset():
        for kv, L0 in zip(kvs, base):
            kv.length = L0
        for cv in canv:
            rt.canvas_init(model, cv)

    def mixed():
        segs = [rt.Refine(kvs[b], canv[b]) for b in range(refine)]
        segs += [rt.Append(kvs[refine], t_commit), rt.Append(kvs[refine + 1], t_prompt)]
        rt.mixed_step(model, segs)

    def separate():
        for b in range(refine):
            rt.denoise_step(model, canv[b], kvs[b])
        rt.commit_canvas(model, t_commit[None], kvs[refine])
        rt.commit_canvas(model, t_prompt[None], kvs[refine + 1])

    res = {}
    for name, fn in (("mixed", mixed), ("separate", separate), ("mixed_again", mixed)):
        for _ in range(warmup):
            reset()
            fn()
        torch.cuda.synchronize()
        dt = 0.0
        for _ in range(passes):
            reset()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt += time.perf_counter() - t0
        res[name] = dt / passes * 1e3
        log(f"[bench] {c.name} {name}: {res[name]:.3f} ms per pass")
    free_gpu(model)
    del inp, kvs, canv
    free_gpu()
    ms = min(res["mixed"], res["mixed_again"])
    return {"workload": c.name, "refine_canvases": refine, "canvas": N, "prompt_kv": P,
            "commit_append": commit_len, "prompt_read": prompt_len, "rows_per_pass": rows,
            "ms_per_pass_mixed": ms, "ms_per_pass_separate": res["separate"],
            "speedup": res["separate"] / ms, "rows_per_s": rows / ms * 1e3,
            "refine_canvas_tokens_per_s": refine * N / ms * 1e3}


def time_block_ar(cfg, warmup: int = 1):
    """Block-autoregressive generation: causal encode of the prompt, then
    n_canvases canvases, each committed to the KV cache by a causal pass."""
    import torch

    from diffusion_decoding_amd import runtime as rt
    from workloads import make_inputs

    log(f"[bench] generating inputs for {cfg.name} on the GPU")
    inp = make_inputs(cfg, device="cuda")
    model = rt.Model(inp)
    kv = rt.KVCache(inp.kv_k, inp.kv_v, 0)
    canvas = rt.Canvas.empty(cfg.batch, cfg.canvas_len, cfg.seed)

    def run():
        kv.length = 0
        rt.commit_canvas(model, inp.prompt_tokens, kv)
        steps = 0
        for c in range(cfg.n_canvases):
            canvas.block = c
            rt.canvas_init(model, canvas)
            steps += rt.generate_canvas(model, canvas, kv)
            rt.commit_canvas(model, canvas.tokens, kv)
        return steps

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps = run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # routing balance of the first canvas's first step, after the prompt encode
    kv.length = 0
    rt.commit_canvas(model, inp.prompt_tokens, kv)
    canvas.block = 0
    rt.canvas_init(model, canvas)
    routing = routing_stats(model, canvas, kv, cfg)
    free_gpu(model)
    del inp, kv, canvas
    free_gpu()
    toks = cfg.batch * cfg.canvas_len * cfg.n_canvases
    log(f"[bench] {cfg.name}: prompt {cfg.prompt_len} + {cfg.n_canvases} canvases, {steps} steps in {dt:.3f} s")
    return {"workload": cfg.name, "expert_dtype": cfg.expert_dtype, "prompt_tokens": cfg.prompt_len,
            "canvases": cfg.n_canvases, "canvas_tokens_per_s": toks / dt,
            "denoise_steps_per_s": steps / dt, "ms_per_denoise_step_incl_commit": dt / steps * 1e3,
            "note": "time includes the prompt encode and every causal commit pass", "routing": routing}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed canvases")
    ap.add_argument("--warmup", type=int, default=1, help="untimed canvases")
    ap.add_argument("--config", default="c2", help="c2 (batch 1) or c3 (batch 4)")
    ap.add_argument("--kernel", default="moe_gateup",
                    help="kernel class timed for the roofline (moe_gateup, moe_down, lm_head, attn)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=2)
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times and exit "
                         "(reference for the HBM byte counters)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the batch-4 (c3), batch-8 (c5), batch 16 and 32, fill-in-the-middle, block-autoregressive "
                         "fp8 (c4), MXFP4 (c6), self-conditioning and mixed-phase measurements")
    ap.add_argument("--mixed", action="store_true",
                    help="only the mixed-phase serving pass at the c2 shapes (its own JSON line; for profiling)")
    ap.add_argument("--no-kernels", action="store_true",
                    help="skip the per-kernel-class roofline table (one extra canvas per class after "
                         "the timed region)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py runs on exactly one GPU: the library has no multi-GPU path "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).")
        print(msg, file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "copies": 5}), flush=True)
        return

    from diffusion_decoding_amd import _lib
    from diffusion_decoding_amd import runtime as rt
    from workloads import get_config, make_inputs

    cfg = get_config(args.config)
    torch.cuda.set_device(0)
    if args.mixed:
        print(json.dumps({"mixed": time_mixed(get_config("c2"), passes=args.steps, warmup=args.warmup)}), flush=True)
        return
    if cfg.prompt_mode != "kv":
        # block-autoregressive workloads (c4): prompt encode + canvases with their commit passes
        res = time_block_ar(cfg, warmup=args.warmup)
        print(json.dumps({"metric": METRIC, "value": res["canvas_tokens_per_s"], "unit": "canvas tokens/s",
                          "n_gpus": 1, "steps": 1, "warmup": args.warmup, "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "bf16+" + cfg.expert_dtype,
                          "data": "synthetic", "config": {"workload": cfg.name}, "block_ar": res}), flush=True)
        return
    log(f"[bench] generating inputs for {cfg.name} on the GPU")
    inp = make_inputs(cfg, device="cuda")
    torch.cuda.synchronize()
    model = rt.Model(inp)
    kv = rt.KVCache(inp.kv_k, inp.kv_v, inp.kv_len)
    B, N = cfg.batch, cfg.canvas_len
    canvas = rt.Canvas.empty(B, N, cfg.seed)

    for w in range(args.warmup):
        rt.canvas_init(model, canvas)
        n = rt.generate_canvas(model, canvas, kv)
        log(f"[bench] warmup canvas {w}: {n} steps")
    torch.cuda.synchronize()

    _lib.dg_profile_kernel(model.handle, _lib.DG_PROF[args.kernel])
    total_steps = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        rt.canvas_init(model, canvas)
        total_steps += rt.generate_canvas(model, canvas, kv)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof_ms, launches = _lib.dg_profile_read(model.handle)
    _lib.dg_profile_kernel(model.handle, 0)
    elapsed = t1 - t0
    log(f"[bench] {args.steps} canvases, {total_steps} denoise steps in {elapsed:.3f} s")

    roofline = roofline_entry(cfg, args.kernel, prof_ms, launches)
    roofline["traffic"] = MEASURED_TRAFFIC.get((args.kernel, cfg.name))
    roofline["kernel"] = args.kernel
    roofline = {k: roofline[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                         "avg_launch_us", "launches", "algorithmic_bytes_per_launch",
                                         "algorithmic_flops_per_launch")}

    steps_per_canvas = total_steps / args.steps
    out = {
        "metric": METRIC,
        "value": B * N * args.steps / elapsed,
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype if cfg.expert_dtype != "fp8" else "bf16+fp8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "batch": B, "canvas": N,
                   "prompt_kv": cfg.prompt_len, "experts": f"{cfg.n_experts} top-{cfg.top_k} + shared",
                   "d_model": cfg.d_model, "vocab": cfg.vocab,
                   "denoise_steps_per_canvas": steps_per_canvas},
        "denoise_steps_per_s": total_steps / elapsed,
        "ms_per_denoise_step": elapsed / total_steps * 1e3,
        "roofline": roofline,
        "cpu_baseline": None,
    }

    # every kernel class, timed live with HIP events on its stream, one extra
    # (untimed) canvas per class after the timed region
    if not args.no_kernels:
        kern = {}
        for name in ("attn", "qkv", "shared", "router", "moe_gateup", "moe_down", "lm_head", "commit"):
            if name == "router" and topk_in_shared(cfg):
                log("[kernels] router      logits in the shared gate/up launch, top-k in the shared down launch")
                continue
            _lib.dg_profile_kernel(model.handle, _lib.DG_PROF[name])
            rt.canvas_init(model, canvas)
            rt.generate_canvas(model, canvas, kv)
            ms, cnt = _lib.dg_profile_read(model.handle)
            kern[name] = roofline_entry(cfg, name, ms, cnt)
            e = kern[name]
            log(f"[kernels] {name:11s} {e['avg_launch_us']:9.1f} us/launch ({cnt} launches)  "
                f"{e['hbm_gbs']:7.0f} GB/s  {e['tflops']:7.1f} TFLOP/s  {100 * e['frac']:5.1f}% of {e['bound']} peak")
        _lib.dg_profile_kernel(model.handle, 0)
        out["kernels"] = kern
        rt.canvas_init(model, canvas)
        out["routing"] = routing_stats(model, canvas, kv, cfg)
        # every class against its own bound, beside the headline kernel
        out["roofline_by_class"] = {n: {"bound": e["bound"], "frac": e["frac"], "avg_launch_us": e["avg_launch_us"]}
                                    for n, e in kern.items()}

    # fill-in-the-middle on the same model: a fixed 64-token prefix and
    # 64-token suffix (pre-committed), 128 open positions denoised around them
    if not args.no_extra and args.config == "c2":
        head = tail = N // 4
        g = torch.Generator(device="cuda").manual_seed(cfg.seed + 100)
        ptok = torch.randint(0, cfg.vocab, (B, N), generator=g, device="cuda", dtype=torch.int32)
        pmask = torch.zeros(B, N, dtype=torch.uint8, device="cuda")
        pmask[:, :head] = 1
        pmask[:, N - tail:] = 1
        rt.canvas_init(model, canvas)
        rt.canvas_prefill(model, canvas, ptok, pmask)
        rt.generate_canvas(model, canvas, kv)  # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rt.canvas_init(model, canvas)
        rt.canvas_prefill(model, canvas, ptok, pmask)
        n_inf = rt.generate_canvas(model, canvas, kv)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        opened = B * (N - head - tail)
        out["infill"] = {"workload": cfg.name, "fixed_prefix": head, "fixed_suffix": tail,
                         "open_positions": opened, "denoise_steps": n_inf,
                         "generated_tokens_per_s": opened / dt, "canvas_tokens_per_s": B * N / dt,
                         "ms_per_denoise_step": dt / n_inf * 1e3}
        log(f"[bench] infill: {opened} open positions, {n_inf} steps in {dt:.3f} s")

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sampled step")
        out["cpu_baseline"] = cpu_baseline(inp, cfg, steps_per_canvas, max(1, min(args.cpu_layers, cfg.n_layers)))
    free_gpu(model)
    del inp, kv, canvas
    free_gpu()
    if not args.no_extra and args.config == "c2":
        out["batch4"] = time_loop(get_config("c3"), canvases=1, warmup=1)
        out["batch8"] = time_loop(get_config("c5"), canvases=1, warmup=1)
        # batch sweep beyond 8 at the c2 shapes (2048-row prompts): 16 and 32
        # canvases, 4096 and 8192 tokens in one routed launch
        out["batch_sweep"] = {str(b): time_loop(get_config("c2").replace(name=f"c2_batch{b}", batch=b),
                                                canvases=1, warmup=1) for b in (16, 32)}
        # the absorbing-state (mask) noise variant: same model, [MASK] = the last id
        c2 = get_config("c2")
        out["absorbing"] = time_loop(c2.replace(name="c2_absorbing", mask_token=c2.vocab - 1),
                                     canvases=1, warmup=1)
        # the canvas-length variant: one 512-position canvas over the same prompt
        out["canvas512"] = time_loop(get_config("c2").replace(name="c2_canvas512", canvas_len=512),
                                     canvases=1, warmup=1)
        out["canvas1024"] = time_loop(get_config("c2").replace(name="c2_canvas1024", canvas_len=1024),
                                      canvases=1, warmup=1)
        out["block_ar_fp8"] = time_block_ar(get_config("c4"))
        # MXFP4 routed experts (E2M1 codes + E8M0 block scales), same shapes as the headline
        out["mxfp4"] = time_loop(get_config("c6"), canvases=1, warmup=1, kernels=("moe_gateup", "moe_down"))
        # the same MXFP4 weights with MXFP8 token rows into the routed gate/up (gfx950 scaled MFMA)
        out["mxfp4_a8"] = time_loop(get_config("c7"), canvases=1, warmup=1, kernels=("moe_gateup", "moe_down"))
        # self-conditioning: each step after the first adds the previous step's predictions to the input
        out["self_condition"] = time_loop(c2.replace(name="c2_self_condition", self_condition=True),
                                          canvases=1, warmup=1)
        # a serving batch in mixed phases: three canvases refining, a canvas commit and a prompt read
        out["mixed"] = time_mixed(get_config("c2"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
