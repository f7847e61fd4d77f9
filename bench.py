"""Benchmark of the DiT-MoE sparse MoE layer on one MI355X.

One step = one forward pass of the whole layer (gate, softmax and top-K,
permutation, routed expert MLPs, shared expert MLPs, weighted combine,
balance statistic) over one batch of seeded synthetic input, by default the
XL/2-8E2A layer at 512x512 (B=32 images x T=1024 tokens, D=1152, E=8, K=2,
n_s=2, H=4608, bf16).  Inputs and weights are resident in device memory
before the timed region starts.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="xl_8e2a_512")
    ap.add_argument("--x-perm", action="store_true",
                    help="materialise x_perm instead of gathering rows in GEMM1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes five "
                         "times (reference for the HBM byte counters)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward step, time the layer's "
                         "backward pass (after one forward pass)")
    ap.add_argument("--analytics", action="store_true",
                    help="instead of the layer, time the routing histogram "
                         "(counts by patch position and by image tag) on the "
                         "layer's routing")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager calls instead of replays of "
                         "one captured HIP graph (the default; per-call "
                         "times always come from an eager pass)")
    ap.add_argument("--recompute-u", action="store_true",
                    help="with --backward: the forward keeps no "
                         "pre-activations and the backward recomputes them")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="repetitions of each HBM-bound call timed after a "
                         "1 GiB cache flush (0: skip)")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="instead of the layer, time the CPU oracle on a "
                         "bounded sample of every configured workload")
    ap.add_argument("--mlp-fused", action="store_true",
                    help="instead of the layer, time the one-kernel expert "
                         "MLP against the two-stage grouped FFN on the "
                         "configured layer's routed and shared experts at its "
                         "own token count and at 4x")
    return ap.parse_args()


# Measured HBM traffic of the expert GEMM kernels lives in a profile summary,
# together with the SHA-256 of the kernel source it was measured on; a
# changed source means the figures no longer apply.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_expert_gemm_xl_8e2a_512.md")
FFN_SOURCE = os.path.join(ROOT, "sparse_moe_diffusion_amd", "csrc", "ffn.hip")


def code_hash(path):
    """sha256 of a C++ source with its comments and whitespace removed: the
    code the counters were taken on, unchanged by edits to its comments."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return hashlib.sha256(re.sub(r"\s+", "", text).encode()).hexdigest()


def measured_traffic(stage):
    """Bytes per launch of expert GEMM stage 1 or 2 from the counter summary,
    or None when it is missing or was taken on other code than the current
    ffn.hip's."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("-").strip()
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip().lower()] = v.strip().strip("`")
    want = fields.get("ffn.hip code sha256")
    val = fields.get(f"stage {stage} traffic bytes per launch")
    if not want or not val:
        return None
    return float(val) if code_hash(FFN_SOURCE) == want else None


def copy_calibration(nbytes):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}),
          flush=True)


def kernel_work(cfg, gather: bool):
    """Algorithmic work of each call of one step: (kind, amount).
    FLOPs count 2 per multiply-add; bytes are the unavoidable HBM traffic."""
    eb = 2 if cfg.dtype == "bf16" else 4
    N, D, H, E, K, A, n_s = cfg.N, cfg.D, cfg.H, cfg.E, cfg.K, cfg.A, cfg.n_s
    Kmax = cfg.Kmax
    w = {
        "gate": ("bytes", N * D * eb + E * D * 4 + N * E * 4 + N * Kmax * 8),
        "permute": ("bytes", N * Kmax * 4 * 2 + A * 4 +
                    (0 if gather else N * D * eb + A * D * eb)),
        "routed_up": ("flops", 2 * A * D * H),
        "routed_down": ("flops", 2 * A * D * H),
        "shared_up": ("flops", 2 * N * D * H * n_s),
        "shared_down": ("flops", 2 * N * D * H * n_s),
        # stage 2 of the shared experts with the combine in its epilogue
        "shared_down_combine": ("flops", 2 * N * D * H * n_s),
        "combine": ("bytes", A * D * eb + (N * D * eb if n_s else 0) +
                    N * D * eb + N * Kmax * 8),
        "balance": ("bytes", N * E * 4 + N * Kmax * 4),
        # the gate with the balance statistic reduced inside it: the gate's
        # bytes plus the per-image counts and probability sums
        "gate_balance": ("bytes", N * D * eb + E * D * 4 + N * E * 4 +
                         N * Kmax * 8 + cfg.B * E * 8),
    }
    # the gate, the balance statistic and the permutation's index tensors in
    # one call (routed rows gathered in the GEMM)
    w["gate_route"] = ("bytes", w["gate_balance"][1] + N * Kmax * 4 * 2 + A * 4)
    return w


def backward_bench(args):
    """Time the backward pass of the layer: gradients of <dy, y> + L_balance
    for a seeded synthetic dy, after one forward pass (routing fixed).  By
    default the forward is a training forward that keeps the expert MLPs'
    pre-activations (no recomputation in the backward); the forward's own
    time is reported beside it."""
    import torch
    import synth
    from sparse_moe_diffusion_amd import _lib, layer

    _lib.load()
    cfg = synth.CONFIGS[args.config]
    inp = synth.make_inputs(cfg)
    x = layer._to_device(inp.x, torch.bfloat16, "cuda")
    wts = layer.LayerWeights.from_inputs(inp, "cuda")
    save_u = not args.recompute_u
    buf = layer.LayerBuffers(cfg, "cuda", gather=True, save_u=save_u)
    layer.forward(cfg, x, wts, buf)
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 77)
    dy = torch.randn(cfg.N, cfg.D, device="cuda", generator=g).to(torch.bfloat16)
    grads = layer.BackwardBuffers(cfg)
    steps = layer.BACKWARD_STEPS

    def one(evs=None):
        for i, (_, fn) in enumerate(steps):
            if evs is not None:
                evs[i].record()
            fn(cfg, x, wts, buf, grads, dy, 1.0)
        if evs is not None:
            evs[len(steps)].record()

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)]
           for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        one(evs[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    per = {n: sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(K)) / K
           for i, (n, _) in enumerate(steps)}
    # the forward that feeds it (same buffers), timed alone
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        layer.forward(cfg, x, wts, buf)
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t0) * 1e3 / K
    # executed GEMM work of one grouped-MLP backward call: dgrad of both
    # matrices and wgrad of both (plus u when recomputed), 2*M*D*H FLOPs each
    prods = 4.0 if save_u else 5.0
    f_routed = 2.0 * prods * cfg.A * cfg.D * cfg.H
    f_shared = 2.0 * prods * cfg.N * cfg.D * cfg.H * cfg.n_s
    kern = {}
    for n, t in per.items():
        e = {"ms": round(t, 4)}
        fl = {"routed_ffn_backward": f_routed, "shared_ffn_backward": f_shared}.get(n)
        if fl:
            tf = fl / (t * 1e-3) / 1e12
            e.update(tflops=round(tf, 1), frac_mfma_peak=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
        kern[n] = e
    ffn_ms = per["routed_ffn_backward"] + per["shared_ffn_backward"]
    ach = (f_routed + f_shared) / (ffn_ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "MoE-layer backward tokens/sec (gradients of <dy,y> + "
                  "L_balance), XL/2-8E2A @512",
        "value": round(cfg.N / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic (seeded dy)",
        "config": {"workload": f"{cfg.name}: backward of the layer, B={cfg.B} x "
                               f"T={cfg.T}, D={cfg.D}, E={cfg.E}, K={cfg.K}, "
                               f"n_s={cfg.n_s}, H={cfg.H}",
                   "pre_activations": "kept by the forward" if save_u
                                      else "recomputed"},
        "forward_ms": round(fwd_ms, 4),
        "train_step_ms": round(fwd_ms + ms, 4),
        "roofline": {"kernel": f"grouped expert MLP backward ({int(prods)} GEMMs per call)",
                     "bound": "mfma", "achieved": round(ach, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels": kern}), flush=True)


def analytics_bench(args):
    """Time moe_routing_histogram on one batch's top-K routing of the
    configured layer, with one class tag per image out of 1000."""
    import torch
    import synth
    from sparse_moe_diffusion_amd import _lib, layer, ops

    _lib.load()
    cfg = synth.CONFIGS[args.config]
    inp = synth.make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    x = layer._to_device(inp.x, dt, "cuda")
    wts = layer.LayerWeights.from_inputs(inp, "cuda")
    buf = layer.LayerBuffers(cfg, "cuda", gather=True)
    layer.gate(cfg, x, wts, buf)
    n_tags = 1000
    tags = (torch.arange(cfg.B, device="cuda", dtype=torch.int32) * 37) % n_tags
    pos = torch.zeros(cfg.T, cfg.E, dtype=torch.int64, device="cuda")
    tag = torch.zeros(n_tags, cfg.E, dtype=torch.int64, device="cuda")

    def call():
        ops.moe_routing_histogram(buf.topk_idx, cfg.B, cfg.T, cfg.E, pos, tags,
                                  tag)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = (cfg.N * cfg.Kmax * 4 + cfg.B * 4 + 2 * cfg.T * cfg.E * 8
              + 2 * n_tags * cfg.E * 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "routing histogram by patch position and image "
                      "tag (one batch)", "value": round(ms * 1e3, 2),
                      "unit": "us per call", "higher_is_better": False,
                      "steps": args.steps, "warmup": args.warmup,
                      "config": {"workload": cfg.name, "images": cfg.B,
                                 "tokens_per_image": cfg.T, "experts": cfg.E,
                                 "slots": cfg.Kmax, "tags": n_tags},
                      "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 5),
                      "bound": "launch latency"}), flush=True)


def mlp_fused_bench(args):
    """moe_grouped_mlp_fused against moe_grouped_ffn (both stages) on the
    routed experts (E groups of the balanced A/E rows, rows gathered from x)
    and the shared experts (one group of N rows, hidden n_s*H) of a narrow
    layer, at its token count and at 4x.  One JSON line, times in us."""
    import torch
    import synth
    from sparse_moe_diffusion_amd import _lib, ops

    _lib.load()
    cfg = synth.CONFIGS[args.config]
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    rows = []
    for scale in (1, 4):
        N = cfg.N * scale
        for kind, G, per, H, gather in (
                ("routed", cfg.E, cfg.K * N // cfg.E, cfg.H, True),
                ("shared", 1, N, cfg.n_s * cfg.H, False)):
            total, D = G * per, cfg.D
            x = torch.randn(N, D, device=dev, generator=gen).to(torch.bfloat16)
            w1 = (torch.randn(G, H, D, device=dev, generator=gen) * 0.05).to(torch.bfloat16)
            w2 = (torch.randn(G, D, H, device=dev, generator=gen) * 0.05).to(torch.bfloat16)
            off = torch.arange(G + 1, device=dev, dtype=torch.int64) * per
            ri = (torch.randint(0, N, (total,), device=dev, generator=gen,
                                dtype=torch.int32) if gather else None)
            h = torch.empty(total, H, dtype=torch.bfloat16, device=dev)
            y2 = torch.empty(total, D, dtype=torch.bfloat16, device=dev)
            y1 = torch.empty(total, D, dtype=torch.bfloat16, device=dev)
            two = timed(lambda: ops.moe_grouped_ffn(x, ri, total, off, w1, None,
                                                    w2, None, h, y2))
            one = timed(lambda: ops.moe_grouped_mlp_fused(x, ri, total, off, w1,
                                                          None, w2, None, y1))
            same = bool(torch.equal(y1, y2))
            flops = 4.0 * total * D * H
            rows.append({"experts": kind, "tokens": N, "groups": G,
                         "rows": total, "D": D, "H": H,
                         "two_stage_us": round(two, 1),
                         "fused_us": round(one, 1),
                         "fused_tflops": round(flops / (one * 1e-6) / 1e12, 1),
                         "same_bits": same})
            del x, w1, w2, h, y1, y2
    print(json.dumps({"metric": "one-kernel expert MLP vs two-stage grouped FFN",
                      "unit": "us per call", "higher_is_better": False,
                      "steps": args.steps, "warmup": args.warmup,
                      "config": {"workload": cfg.name}, "cases": rows}),
          flush=True)


def host_info():
    """The host the CPU baseline runs on: logical CPUs, the ones this
    process may use, CPU model, sockets, cores and threads per core."""
    info = {"nproc": os.cpu_count()}
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    try:
        text = open("/proc/cpuinfo").read()
    except OSError:
        return info
    blocks = [b for b in text.split("\n\n") if b.strip()]
    fields = [dict((k.strip(), v.strip()) for k, v in
                   (l.split(":", 1) for l in b.splitlines() if ":" in l))
              for b in blocks]
    if fields:
        f0 = fields[0]
        info["model"] = f0.get("model name", "")
        sockets = {f.get("physical id") for f in fields if "physical id" in f}
        info["sockets"] = len(sockets) or 1
        cores = int(f0.get("cpu cores", 0) or 0)
        sib = int(f0.get("siblings", 0) or 0)
        if cores:
            info["cores_per_socket"] = cores
            info["threads_per_core"] = sib // cores if sib else 1
    return info


def blas_threads():
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def cpu_baseline(cfg, inp, target_s):
    """The CPU oracle on whole images of the same workload until about
    ``target_s`` seconds of CPU work (at least one image, or the first
    ``T`` tokens' worth of a shorter slice for very wide layers): tokens/s
    and GFLOP/s of the layer's algorithmic work."""
    import oracle
    import synth
    done_tokens, elapsed, images = 0, 0.0, 0
    while elapsed < target_s and images < cfg.B:
        b = images
        sub_cfg = cfg.with_(B=1)
        sub = synth.LayerInputs(sub_cfg, inp.x[b * cfg.T:(b + 1) * cfg.T],
                                inp.w_gate, inp.bias, inp.w1, inp.w2, inp.w1s,
                                inp.w2s)
        t0 = time.perf_counter()
        oracle.forward(sub)
        elapsed += time.perf_counter() - t0
        done_tokens += cfg.T
        images += 1
    tps = done_tokens / elapsed
    return {"value": tps, "unit": "tokens/s",
            "cores": blas_threads(), "kind": "oracle",
            "gflops": round(tps * cfg.flops_per_token() / 1e9, 2),
            "host": host_info(),
            "sample": f"{images} image(s) x {cfg.T} tokens of {cfg.name} "
                      f"(whole layer in float64 numpy, {elapsed:.1f} s)"}


def cpu_baseline_all(args):
    """The oracle on a bounded sample of every configured workload (whole
    images, about --cpu-seconds each), beside the host description: one JSON
    line.  A reported baseline, not a target."""
    import synth
    rows = []
    for name, cfg in synth.CONFIGS.items():
        inp = synth.make_inputs(cfg)
        r = cpu_baseline(cfg, inp, args.cpu_seconds)
        rows.append({"workload": name, "tokens_per_s": round(r["value"], 1),
                     "gflops": r["gflops"], "sample": r["sample"]})
        print(json.dumps({"progress": name, **rows[-1]}), flush=True)
        del inp
    print(json.dumps({"metric": "CPU oracle throughput per workload",
                      "kind": "oracle", "threads": blas_threads(),
                      "host": host_info(), "workloads": rows}), flush=True)


def cold_timings(cfg, x, wts, buf, steps, reps):
    """The HBM-bound calls of the step, each timed ``reps`` times right after
    a read of a 1 GiB buffer that evicts the 256 MB memory-side cache and
    the L2s (so their inputs come from HBM; a read leaves only clean lines,
    so no write-back of the flush competes with the timed call), and ``reps``
    times back to back (warm), plus measured-only forms: the permute that
    also copies the rows to x_perm, the separate combine kernel where the
    layer fuses it, and the gate-with-balance and index-only permute calls
    where the layer routes in one call.  Median ms, GB/s of algorithmic
    bytes and the fraction of the HBM peak, cold and warm."""
    import torch
    import numpy as np
    from sparse_moe_diffusion_amd import layer
    import copy
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    work = kernel_work(cfg, buf.gather)
    calls = [(n, f) for n, f in steps
             if n in ("gate", "gate_balance", "gate_route", "permute", "combine",
                      "balance")]
    extra = {}
    if any(n == "gate_route" for n, _ in calls):
        # the two calls the fused routing call replaces, measured only
        calls.append(("gate_balance", lambda c, x_, w, b: layer.gate_balance(c, x_, w, b)))
        calls.append(("permute", lambda c, x_, w, b: layer.permute(c, x_, b)))
    if cfg.dtype == "bf16":
        eb = 2
        xp = torch.empty(cfg.A, cfg.D, dtype=x.dtype, device="cuda")
        bx = copy.copy(buf)
        bx.x_perm = xp
        calls.append(("permute_x_perm", lambda c, x_, w, b: layer.permute(c, x_, bx)))
        extra["permute_x_perm"] = (cfg.N * cfg.D * eb + cfg.A * cfg.D * eb +
                                   cfg.N * cfg.Kmax * 8 + cfg.A * 4)
        if not any(n == "combine" for n, _ in steps) and cfg.n_s > 0:
            # the separate combine on the step's routed rows and a shared
            # output from the unfused stage 2
            layer.shared_ffn(cfg, x, wts, buf, layer.DOWN)
            yc = torch.empty_like(buf.y)
            by = copy.copy(buf)
            by.y = yc
            calls.append(("combine_separate", lambda c, x_, w, b: layer.combine(c, by)))
            extra["combine_separate"] = work["combine"][1]
    out = {}
    for name, fn in calls:
        cold, warm = [], []
        for r in range(2 * reps):
            if r < reps:
                flush.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(cfg, x, wts, buf)
            e1.record()
            torch.cuda.synchronize()
            (cold if r < reps else warm).append(e0.elapsed_time(e1))
        nbytes = extra.get(name, work.get(name, ("bytes", 0))[1])
        ms = float(np.median(cold))
        msw = float(np.median(warm))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "bytes": int(nbytes),
                     "gbs": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "ms_warm": round(msw, 4),
                     "frac_hbm_peak_warm": round(nbytes / (msw * 1e-3) / 1e9 /
                                                 HBM_PEAK_GBS, 4)}
    del flush
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer benchmark runs on one GPU only; "
                          "--gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.analytics:
        analytics_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.mlp_fused:
        mlp_fused_bench(args)
        return
    if args.cpu_baseline_all:
        cpu_baseline_all(args)
        return
    import torch
    import synth
    from sparse_moe_diffusion_amd import _lib, layer

    _lib.load()
    cfg = synth.CONFIGS[args.config]
    gather = not args.x_perm
    inp = synth.make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = "cuda"
    x = layer._to_device(inp.x, dt, dev)
    wts = layer.LayerWeights.from_inputs(inp, dev)
    buf = layer.LayerBuffers(cfg, dev, gather=gather)
    steps = list(layer.steps(cfg, buf))

    def one_step(evs=None):
        for i, (_, fn) in enumerate(steps):
            if evs is not None:
                evs[i].record()
            fn(cfg, x, wts, buf)
        if evs is not None:
            evs[len(steps)].record()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)]
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        one_step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / K
    if not args.eager:
        # the same step captured once, then K replays on the same stream
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    per_call = {}
    for i, (name, _) in enumerate(steps):
        per_call[name] = sum(evs[k][i].elapsed_time(evs[k][i + 1])
                             for k in range(K)) / K
    work = kernel_work(cfg, gather)
    kernels = {}
    for name, ms in per_call.items():
        kind, amount = work[name]
        if kind == "flops":
            ach = amount / (ms * 1e-3) / 1e12
            kernels[name] = {"ms": round(ms, 4), "tflops": round(ach, 1),
                             "frac_mfma_peak": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            ach = amount / (ms * 1e-3) / 1e9
            kernels[name] = {"ms": round(ms, 4), "gbs": round(ach, 1),
                             "frac_hbm_peak": round(ach / HBM_PEAK_GBS, 4)}

    # dominant kernel: the grouped GEMM stage with the larger total time;
    # its two launches per step (routed, shared) carry equal FLOPs.
    up = [n for n in ("routed_up", "shared_up") if n in per_call]
    down = [n for n in ("routed_down", "shared_down", "shared_down_combine")
            if n in per_call]
    t_up = sum(per_call[n] for n in up)
    t_down = sum(per_call[n] for n in down)
    dom = up if t_up >= t_down else down
    dom_name = ("gemm_bf16_kernel<gelu> (expert FFN stage 1)" if dom is up
                else "gemm_bf16_kernel<store> (expert FFN stage 2)")
    dom_flops = sum(work[n][1] for n in dom) / len(dom)
    dom_ms = sum(per_call[n] for n in dom) / len(dom)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12

    N = cfg.N
    tokens_per_s = N / (ms_per_step * 1e-3)
    layer_tflops = cfg.flops_per_token() * N / (ms_per_step * 1e-3) / 1e12
    gemm_ms = t_up + t_down
    gemm_tflops = cfg.gemm_flops() / (gemm_ms * 1e-3) / 1e12

    out = {
        "metric": "MoE-layer tokens/sec and TFLOP/s (% bf16 MFMA peak), "
                  "XL/2-8E2A @512",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": {"workload": f"{cfg.name}: DiT-MoE sparse MoE layer, "
                               f"B={cfg.B} images x T={cfg.T} tokens, D={cfg.D}, "
                               f"E={cfg.E}, K={cfg.K}, n_s={cfg.n_s}, H={cfg.H}, "
                               f"{cfg.route} routing",
                   "tokens": N, "gather_rows_in_gemm": gather,
                   "launch": "eager" if args.eager else "hip_graph"},
        "layer_tflops": round(layer_tflops, 1),
        "layer_frac_mfma_peak": round(layer_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "expert_gemm_tflops": round(gemm_tflops, 1),
        "expert_gemm_frac_mfma_peak": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"kernel": dom_name, "bound": "mfma",
                     "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "flops_per_launch": dom_flops,
                     "avg_launch_ms": round(dom_ms, 4),
                     "traffic": (measured_traffic(1 if dom is up else 2)
                                 if cfg.name == "xl_8e2a_512" and gather
                                 else None)},
        "kernels": kernels,
    }
    if args.cold_reps > 0:
        out["kernels_cache_cold"] = cold_timings(cfg, x, wts, buf, steps,
                                                 args.cold_reps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
