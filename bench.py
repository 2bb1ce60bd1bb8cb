#!/usr/bin/env python3
"""Throughput of the Z-Image S3-DiT denoiser forward on one MI355X.

A step is one full forward (patch + caption embeds, 2 noise-refiner, 2
context-refiner and 30 joint blocks, final layer) of the 1024x1024 workload:
latent [1, 16, 128, 128] (4,096 image tokens) and a 512-token caption, with
random-init bf16 weights of the full 6.15B-parameter model and N(0, 1)
synthetic inputs, all resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line: tokens/s of the whole job, ms per step, the bf16 MFMA
utilisation end to end, the roofline of the dominant kernel (timed live with
HIP events on the engine's stream) and the CPU oracle timed on a bounded
sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DiT forward tokens/sec at 1024^2 (4096+512 tok), 1 MI355X; MFMA util %"
PEAK_BF16 = 2.5e15  # dense bf16 MFMA, FLOP/s
PEAK_INT8 = 5.0e15  # dense int8 MFMA, OP/s
PEAK_HBM = 8.0e12   # bytes/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work

def stage_rows(model, n_img, lens):
    """Rows (tokens) each block of the stack processes, per sample, in order."""
    out = []
    for _ in range(model["n_noise_refiner"]):
        out.append(("noise", [n_img for _ in lens]))
    for _ in range(model["n_context_refiner"]):
        out.append(("context", list(lens)))
    for _ in range(model["n_layers"]):
        out.append(("joint", [n_img + L for L in lens]))
    return out


def work_per_forward(model, n_img, lens, cap_dim=2560, patch_dim=64, adaln=256, int8=False):
    """Algorithmic FLOPs of the MFMA classes and algorithmic HBM bytes of the
    bandwidth-bound classes, per forward, keyed by the engine's profile classes.
    int8: the block projections take int8 activations (1 B/elem written by
    the norms; the attention output and SwiGLU product are read as bf16 and
    written as int8 by the quant class)."""
    D, F = model["hidden"], model["ffn"]
    w = {k: 0.0 for k in ("gemm_qkv", "gemm_out", "gemm_w13_swiglu", "gemm_w2", "attention",
                          "pre_norm", "post_norm", "embed", "final_layer", "conditioning", "quant")}
    hb = 1.0 if int8 else 2.0  # bytes per element of a normalised block input
    stages = stage_rows(model, n_img, lens)
    prev = None
    for i, (stage, rows) in enumerate(stages):
        M = sum(rows)
        # (QK-RMSNorm + RoPE and the V transpose run in this GEMM's epilogue)
        w["gemm_qkv"] += 2.0 * M * D * 3 * D
        w["gemm_out"] += 2.0 * M * D * D
        w["gemm_w13_swiglu"] += 2.0 * M * D * 2 * F
        w["gemm_w2"] += 2.0 * M * F * D
        w["attention"] += sum(4.0 * r * r * D for r in rows)
        # pre-norm only where not fused into the previous block's last kernel
        if prev != stage:
            w["pre_norm"] += M * (4.0 + hb) * D
        # two post-norms: read y bf16, read+write x fp32, write next h (12 B/elem for bf16);
        # the last one of a stage without a fused follow-up skips the h write (10 B/elem);
        # before the final layer h is bf16 in either case
        nxt = stages[i + 1][0] if i + 1 < len(stages) else "final"
        w["post_norm"] += M * (10.0 + hb) * D + M * (10.0 + (2.0 if nxt == "final" else hb if nxt == stage else 0.0)) * D
        if int8:
            w["quant"] += M * 3.0 * (D + F)  # read bf16, write int8 (row scales are negligible)
        prev = stage
    T = sum(lens)
    w["embed"] = 2.0 * n_img * len(lens) * patch_dim * D + 2.0 * T * cap_dim * D
    w["final_layer"] = 2.0 * n_img * len(lens) * D * patch_dim
    n_mod = model["n_noise_refiner"] + model["n_layers"]
    w["conditioning"] = 2.0 * (n_mod * 4 * D + D) * adaln  # the GEMVs: bytes ~ flops (bf16 weights)
    return w


MFMA_CLASSES = ("gemm_qkv", "gemm_out", "gemm_w13_swiglu", "gemm_w2", "attention", "embed", "final_layer")
INT8_CLASSES = ("gemm_qkv", "gemm_out", "gemm_w13_swiglu", "gemm_w2")  # with linear_int8 = 1
HBM_CLASSES = ("pre_norm", "post_norm", "quant")


def summarize(stats, steps, work, int8=False):
    """Per-class time, achieved rate and fraction of the class's peak; and the
    roofline entry of the class with the most time."""
    kernels = {}
    for name, (launches, ms) in stats.items():
        if launches == 0:
            continue
        per_fwd_ms = ms / steps
        entry = {"ms_per_forward": round(per_fwd_ms, 4), "launches_per_forward": launches // steps,
                 "avg_launch_us": round(ms / launches * 1e3, 2)}
        if name in MFMA_CLASSES:
            peak = PEAK_INT8 if (int8 and name in INT8_CLASSES) else PEAK_BF16
            ach = work[name] / (per_fwd_ms * 1e-3)
            entry.update(achieved=round(ach / 1e12, 2), unit="TOP/s" if peak == PEAK_INT8 else "TFLOP/s",
                         frac=round(ach / peak, 4))
        elif name in HBM_CLASSES:
            ach = work[name] / (per_fwd_ms * 1e-3)
            entry.update(achieved=round(ach / 1e9, 1), unit="GB/s", frac=round(ach / PEAK_HBM, 4))
        kernels[name] = entry
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_forward"])
    d = kernels[dom]
    launches_dom = stats[dom][0] / steps
    per_launch = work[dom] / launches_dom if launches_dom else 0.0
    avg_s = d["avg_launch_us"] * 1e-6
    if dom in HBM_CLASSES:
        roof = {"bound": "hbm", "achieved": round(per_launch / avg_s / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s"}
    else:
        peak = PEAK_INT8 if (int8 and dom in INT8_CLASSES) else PEAK_BF16
        roof = {"bound": "mfma", "achieved": round(per_launch / avg_s / 1e12, 2), "peak": peak / 1e12,
                "unit": "TOP/s" if peak == PEAK_INT8 else "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["work_per_launch"] = per_launch
    return kernels, roof, dom


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(wl, model):
    """Time the float64 oracle on a bounded sample of the workload: one block
    of each kind on its own rows (a noise-refiner block on the image tokens, a
    context-refiner block on the caption tokens, a joint block on all of
    them) plus the embedders and the final layer, and sum the blocks by their
    counts in the stack (an estimate of one forward, labelled as such, with
    the host CPU model and BLAS)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synthetic
    from oracle import ModelConfig, manifest
    from oracle import model as om

    cfg = ModelConfig.from_dict(model)
    lat_shape, lens = wl["latent"], wl["caption_lens"]
    Hp, Wp = lat_shape[2] // 2, lat_shape[3] // 2
    n_img, L = Hp * Wp, lens[0]
    S = n_img + L
    prefixes = {"noise_refiner": "noise_refiner.0", "context_refiner": "context_refiner.0", "layers": "layers.0"}
    W = synthetic.SyntheticWeights(manifest(cfg), seed=wl["seed"])
    keep = tuple(p + "." for p in prefixes.values()) + ("t_embedder.", "all_x_embedder.", "cap_embedder.",
                                                        "all_final_layer.")
    Wb = {n: W[n] for n, _ in manifest(cfg) if n.startswith(keep)}
    lat = synthetic.latent(lat_shape, seed=wl["seed"])[0].astype(np.float64)
    feats = synthetic.captions(lens, seed=wl["seed"])[0].astype(np.float64)
    x = synthetic.residual((S, cfg.hidden), seed=wl["seed"]).astype(np.float64)
    cap_ids, img_ids = om.position_ids(L, Hp, Wp)
    cos_img, sin_img = om.rope_tables(cfg, img_ids)
    cos_cap, sin_cap = om.rope_tables(cfg, cap_ids)
    cos, sin = np.concatenate([cos_img, cos_cap]), np.concatenate([sin_img, sin_cap])
    c = om.timestep_mlp(cfg, Wb, np.array([wl["t"][0]]))[0]
    blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    threads = max([d.get("num_threads", 1) for d in blas] or [1])
    blas_name = ", ".join(sorted({f"{d.get('internal_api', '?')} {d.get('version', '')}".strip() for d in blas})) or "unknown"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    n_noise, n_ctx, n_joint = cfg.n_noise_refiner, cfg.n_context_refiner, cfg.n_layers
    p = prefixes["noise_refiner"]  # a kind absent from the stack is not timed
    t_noise = timed(lambda: om.block(cfg, Wb, p, x[:n_img], cos_img, sin_img,
                                     om.block_modulation(Wb, p, c))) if n_noise else 0.0
    p = prefixes["context_refiner"]
    t_ctx = timed(lambda: om.block(cfg, Wb, p, x[n_img:], cos_cap, sin_cap, None)) if n_ctx else 0.0
    p = prefixes["layers"]
    t_joint = timed(lambda: om.block(cfg, Wb, p, x, cos, sin, om.block_modulation(Wb, p, c))) if n_joint else 0.0
    t_ends = timed(lambda: (om.x_embed(cfg, Wb, lat), om.cap_embed(cfg, Wb, feats),
                            om.final_layer(cfg, Wb, x[:n_img], c)))
    fwd_s = n_noise * t_noise + n_ctx * t_ctx + n_joint * t_joint + t_ends
    sample_s = t_noise + t_ctx + t_joint + t_ends
    return {"value": round(S / fwd_s, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model, "blas": blas_name, "precision": "float64",
            "sample": (f"estimate from a {sample_s:.1f} s float64 sample: one block of each kind on its own rows "
                       f"(noise refiner, {n_img} image rows: {t_noise:.2f} s; context refiner, {L} caption rows: "
                       f"{t_ctx:.2f} s; joint, all {S} rows: {t_joint:.2f} s) and the embedders + final layer "
                       f"({t_ends:.2f} s); forward = {n_noise} x noise + {n_ctx} x context + {n_joint} x joint + "
                       f"embedders and final layer = {fwd_s:.1f} s; the whole forward never ran on the CPU")}


# ---------------------------------------------------------------- traffic from committed counters

def source_digest(kernel):
    """Digest of the sources that define a kernel class (its .hip file and the
    shared device header): counter figures taken on other sources do not
    apply."""
    main = "gemm.hip" if kernel.startswith("gemm") or kernel in ("embed", "final_layer") else \
        "attention.hip" if kernel == "attention" else "norm.hip"
    h = hashlib.sha256()
    for f in (main, "common.h"):
        with open(os.path.join(ROOT, "diffusion_transformer_image_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    d = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", txt)
    if not m or not d or d.group(1) != source_digest(kernel):
        return None
    return float(m.group(1))


# ---------------------------------------------------------------- guided step

def guided_step(dit, wl, lat, caps, lens, n_img, stream, steps=3, neg_len=32, guidance=3.0, dt=-0.05):
    """One classifier-free-guided sampler step at the same geometry: the
    forward of [latent; latent] with [caption; 32-token negative caption] and
    the fused guided Euler update; plus the update kernel alone."""
    import numpy as np
    import torch
    import synthetic
    from diffusion_transformer_image_amd import binding
    B = lat.shape[0]
    neg = torch.from_numpy(np.concatenate(synthetic.captions([neg_len] * B, seed=wl["seed"] + 1))).cuda()
    caps_pair = torch.cat([caps, neg])
    lens_pair = list(lens) + [neg_len] * B
    pair = torch.empty((2 * B,) + tuple(lat.shape[1:]), device="cuda")
    pout = torch.empty_like(pair)
    x = lat.clone()
    tt = [0.5] * (2 * B)

    def step():
        pair[:B].copy_(x)
        pair[B:].copy_(x)
        dit.forward(pair, caps_pair, lens_pair, tt, pout)
        binding.cfg_euler_step(x, pout[:B], pout[B:], guidance, dt)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    reps = 50
    e0.record(stream)
    for _ in range(reps):
        binding.cfg_euler_step(x, pout[:B], pout[B:], guidance, dt)
    e1.record(stream)
    torch.cuda.synchronize()
    upd_us = e0.elapsed_time(e1) / reps * 1e3
    n = x.numel()
    tokens = 2 * B * n_img + sum(lens) + B * neg_len
    return {"workload": f"guided step at the same geometry: forward of [latent; latent] with "
                        f"[caption; {neg_len}-token negative caption] + fused guided Euler update",
            "ms_per_step": round(ms, 3), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "update_us": round(upd_us, 2), "update_GBps": round(16.0 * n / (upd_us * 1e-6) / 1e9, 1),
            "update_bytes_per_element": 16}


# ---------------------------------------------------------------- int8 variant

def int8_forward(args, wl, model, lat, caps, lens, t, n_img, tokens, bf16_ms):
    """The same forward with the block projections on int8 codes (weights per
    output row, activations per token): its own engine, K timed forwards,
    then K profiled ones."""
    import torch

    import synthetic
    from diffusion_transformer_image_amd import binding
    steps = args.int8_steps
    cfg = binding.config(max_batch=lat.shape[0], max_image_tokens=n_img, max_caption_tokens=max(lens),
                         linear_int8=1, **model)
    W = synthetic.SyntheticWeights(binding.manifest(cfg), seed=wl["seed"], outlier_log2=wl.get("outlier_log2"))
    dit = binding.DiT(cfg, W.items_parallel(as_bits=True))
    out = torch.empty_like(lat)
    for _ in range(max(args.warmup, 1)):
        dit.forward(lat, caps, lens, t, out)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(steps):
        dit.forward(lat, caps, lens, t, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    assert torch.isfinite(out).all().item(), "non-finite int8 output"
    dit.profile(True)
    for _ in range(steps):
        dit.forward(lat, caps, lens, t, out)
    torch.cuda.synchronize()
    stats = dit.profile_read()
    dit.profile(False)
    dit.close()
    kernels, roof, dom = summarize(stats, steps, work_per_forward(model, n_img, lens, int8=True), int8=True)
    roof["traffic"] = committed_traffic(f"{dom}_i8" if dom in INT8_CLASSES else dom, args.workload)
    ms = wall * 1e3 / steps
    log(f"int8 forward: {ms:.2f} ms")
    return {"workload": "the same forward with the 7 projections of every block on int8 codes "
                        "(per-output-row weight scales, per-token activation scales, exact int32 sums)",
            "steps": steps, "ms_per_step": round(ms, 3), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "speedup_vs_bf16": round(bf16_ms / ms, 3), "dtype": "int8 projections, bf16 attention",
            "roofline": roof, "kernels": kernels}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dit_1024")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cfg-steps", type=int, default=3, metavar="K",
                    help="also time K classifier-free-guided steps (0: skip)")
    ap.add_argument("--int8-steps", type=int, default=10, metavar="K",
                    help="also time K forwards with int8 block projections (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also launch one plain device copy of this many MiB (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this engine runs on one GPU; --gpus {args.gpus} is not supported "
              "(data-parallel sharding over samples needs no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    from diffusion_transformer_image_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        log("library not built; building it")
        from diffusion_transformer_image_amd import build as _b
        _b.build(verbose=False)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synthetic.WORKLOADS[args.workload]
    model = wl["model"]
    lat_shape, lens = wl["latent"], list(wl["caption_lens"])
    B = lat_shape[0]
    n_img = (lat_shape[2] // 2) * (lat_shape[3] // 2)
    tokens = B * n_img + sum(lens)
    t = list(wl["t"]) if wl.get("t") else [0.5] * B

    # workspace for 2 B samples: the guided step runs [latent; latent]
    cfg = binding.config(max_batch=2 * B, max_image_tokens=n_img, max_caption_tokens=max(lens), **model)
    W = synthetic.SyntheticWeights(binding.manifest(cfg), seed=wl["seed"], outlier_log2=wl.get("outlier_log2"))
    t0 = time.perf_counter()
    log(f"drawing and uploading {len(W)} weight tensors ({args.workload})")
    dit = binding.DiT(cfg, W.items_parallel(as_bits=True))
    log(f"engine ready in {time.perf_counter() - t0:.1f} s")
    lat = torch.from_numpy(synthetic.latent(lat_shape, seed=wl["seed"])).cuda()
    caps = torch.from_numpy(np.concatenate(synthetic.captions(lens, seed=wl["seed"]))).cuda()
    out = torch.empty_like(lat)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        dit.forward(lat, caps, lens, t, out)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # timed region: K whole forwards
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        dit.forward(lat, caps, lens, t, out)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = e0.elapsed_time(e1)
    log(f"timed {args.steps} steps: wall {wall * 1e3:.1f} ms, events {gpu_ms:.1f} ms")
    assert torch.isfinite(out).all().item(), "non-finite output"

    # per-kernel timing: the same K forwards with event brackets around each kernel class
    dit.profile(True)
    for _ in range(args.steps):
        dit.forward(lat, caps, lens, t, out)
    torch.cuda.synchronize()
    stats = dit.profile_read()
    dit.profile(False)

    cfg_step = guided_step(dit, wl, lat, caps, lens, n_img, stream, steps=args.cfg_steps) if args.cfg_steps > 0 else None
    if cfg_step is not None:
        log(f"guided step: {cfg_step['ms_per_step']:.2f} ms")

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration} MiB read + written")

    work = work_per_forward(model, n_img, lens)
    kernels, roof, dom = summarize(stats, args.steps, work)
    roof["traffic"] = committed_traffic(dom, args.workload)

    ms_per_step = wall * 1e3 / args.steps
    fwd_flops = sum(work[k] for k in MFMA_CLASSES)
    result = {
        "metric": METRIC,
        "value": round(tokens * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "latent": list(lat_shape), "caption_tokens": lens,
                   "tokens_per_forward": tokens, "blocks": len(stage_rows(model, n_img, lens)),
                   "t": t},
        "mfma_util_pct": round(100.0 * fwd_flops / (ms_per_step * 1e-3) / PEAK_BF16, 2),
        "algorithmic_tflop_per_forward": round(fwd_flops / 1e12, 3),
        "roofline": roof,
        "kernels": kernels,
    }
    if cfg_step is not None:
        result["cfg_step"] = cfg_step
    dit.close()
    if args.int8_steps > 0:
        result["int8_forward"] = int8_forward(args, wl, model, lat, caps, lens, t, n_img, tokens, ms_per_step)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, model) if B == 1 else None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
