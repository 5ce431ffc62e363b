#!/usr/bin/env python3
"""Throughput of the Wan2.2 TI2V-5B VAE decode on one MI355X.

One step = one whole decode, wanvae_decode through the C ABI, of seeded synthetic latents
[1, 48, 31, 44, 80] with random-init decoder weights (decoder_base_dim 256) in bf16 (fp32
accumulation) -> video [1, 3, 121, 704, 1280]. The latents and the fp32 weights are resident
in HBM before the timed region; the decode's own weight rounding/repacking is inside it.

Prints one JSON line: decoded frames/s, the dominant kernel's roofline (the conv kernels,
all launches of the timed decodes: algorithmic FLOPs / HIP-event kernel time, against the
bf16 dense MFMA peak; the HBM bytes per launch from the stored counter measurement while the
kernel source it was taken on is unchanged), the other kernel classes, and the CPU oracle
timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --copy-bytes N    # three device-to-device copies of N bytes (counter scale)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "decoded frames/s (TI2V-5B VAE, 704x1280 bf16); conv TFLOP/s % MFMA peak"
TRAFFIC = os.path.join(ROOT, "profiles", "conv_traffic_704x1280_bf16.json")
KERNELS_SRC = os.path.join(ROOT, "video_vae_decoding_amd", "csrc", "kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, W):
    """The CPU oracle (as it stands: float64 sums, bf16 rounding points) decoding the first
    latent frame of the same decoder on an 11 x 20 crop of the latent (1/16 of the 44 x 80
    frame area: 1/16 of a video frame's work, attention aside), scaled to full frames/s."""
    import oracle
    z = cfg.latents()[:, :, :1, :11, :20]
    t0 = time.perf_counter()
    v = oracle.decode(np.ascontiguousarray(z), W, "bf16")
    dt = time.perf_counter() - t0
    frac = (11 * 20) / (cfg.h * cfg.w)
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or str(cores)
    return {"value": frac * v.shape[2] / dt, "unit": "frames/s", "cores": int(threads) if threads.isdigit() else cores,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "oracle.decode (bf16 mode, float64 sums) of latent frame 0 on an 11x20 crop of the "
                      "[1,48,31,44,80] latents: 1 video frame of 176x320 = 1/16 of a 704x1280 frame; "
                      "value = (1/16 frame) / seconds"}


def stored_traffic():
    """HBM bytes per conv launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading),
    from the stored counter measurement; None once the kernel source differs from the one
    the counters were taken on."""
    if not os.path.exists(TRAFFIC):
        return None
    with open(TRAFFIC) as f:
        t = json.load(f)
    with open(KERNELS_SRC, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["kernels_hip_sha256"]:
            return None
    return t["hbm_bytes_per_launch"]


def copy_calibration(nbytes):
    import torch
    x = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "copies": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decoder here runs on a single MI355X (got --gpus {args.gpus}); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return

    import torch

    import synthetic
    from video_vae_decoding_amd import wanvae

    dev = torch.device("cuda:0")
    cfg = synthetic.DECODE_CONFIGS["ti2v5b_landscape"]
    log("generating inputs ...")
    z, W = cfg.latents(), cfg.weights()
    zt = torch.from_numpy(z).to(dev)
    Wt = {k: torch.from_numpy(v).to(dev) for k, v in W.items()}
    dtype = torch.bfloat16
    frames = cfg.B * cfg.frames
    video = torch.empty((cfg.B, 3, cfg.frames, 16 * cfg.h, 16 * cfg.w), dtype=dtype, device=dev)
    ws = torch.empty(wanvae.decode_workspace_size(cfg.B, cfg.T, cfg.h, cfg.w, Wt, dtype), dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        wanvae.wanvae_decode(zt, Wt, dtype, video=video, workspace=ws)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    wanvae.wanvae_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wanvae.wanvae_decode(zt, Wt, dtype, video=video, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = {k: wanvae.wanvae_profile_read(getattr(wanvae, "K" + k.upper())) for k in ("conv", "norm", "attn", "other")}
    wanvae.wanvae_profile_enable(False)
    elapsed = t1 - t0
    log(f"timed {args.steps} decodes in {elapsed:.3f} s")
    assert torch.isfinite(video).all()

    conv = prof["conv"]
    conv_tflops = conv["flops"] / (conv["ms"] * 1e-3) / 1e12
    kernels = {}
    for k, p in prof.items():
        e = {"ms_per_step": round(p["ms"] / args.steps, 3), "launches_per_step": p["launches"] // max(1, args.steps)}
        if p["flops"]:
            e["TFLOP/s"] = round(p["flops"] / (p["ms"] * 1e-3) / 1e12, 2)
            e["frac_of_peak"] = round(e["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
        if p["bytes"]:
            e["GB/s"] = round(p["bytes"] / (p["ms"] * 1e-3) / 1e9, 1)
            e["frac_of_peak"] = round(e["GB/s"] / PEAK_HBM_GBS, 4)
        kernels[k] = e
    out = {
        "metric": METRIC,
        "value": round(frames * args.steps / elapsed, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ti2v5b_vae_decode_704x1280x121_bf16", "latent": [cfg.B, 48, cfg.T, cfg.h, cfg.w],
                   "video": [cfg.B, 3, cfg.frames, 16 * cfg.h, 16 * cfg.w], "weights": "random-init, seed 3",
                   "accumulate": "fp32"},
        "roofline": {"bound": "mfma",
                     "kernel": "conv (k_conv_halo for the 3x3 convs, k_conv_dma for the rest; all launches of a decode)",
                     "achieved": round(conv_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(conv_tflops / PEAK_BF16_TFLOPS, 4), "traffic": stored_traffic(),
                     "launches": conv["launches"], "avg_launch_ms": round(conv["ms"] / max(1, conv["launches"]), 4),
                     "algorithmic_tflop_per_step": round(conv["flops"] / args.steps / 1e12, 2)},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on its sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg, W)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
