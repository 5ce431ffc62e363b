#!/usr/bin/env python3
"""Throughput of the Wan2.2 TI2V-5B VAE decode on one MI355X.

One step = one whole decode, wanvae_decode through the C ABI, of seeded synthetic latents
[1, 48, 31, 44, 80] with random-init decoder weights (decoder_base_dim 256) in bf16 (fp32
accumulation) -> video [1, 3, 121, 704, 1280]. The latents and the fp32 weights are resident
in HBM before the timed region; the decode's own weight rounding/repacking is inside it.

Prints one JSON line: decoded frames/s over the timed decodes (by default the library's
two-stream chunk pipeline), the dominant kernel's roofline (the conv kernels, all launches of
K more decodes run in chunk order on one stream so that each kernel's HIP-event time is its
own: algorithmic FLOPs / event time, against the bf16 dense MFMA peak; the HBM bytes per
launch from the stored counter measurement while the kernel source it was taken on is
unchanged), the other kernel classes from the same decodes, and the CPU oracle timed on a
bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--workload NAME]
    python bench.py --copy-bytes N    # three device-to-device copies of N bytes (counter scale)

--workload picks another of the measured configurations (default ti2v5b_landscape_bf16):
ti2v5b_landscape_fp32, ti2v5b_portrait_bf16, ti2v5b_landscape_b2_bf16 (whole decodes, frames/s),
ti2v5b_landscape_bf16_tiled (the spatially tiled decode, tile 256 / stride 192 video pixels),
conv1024_l0_bf16, conv256_l3_bf16 (one causal conv, TFLOP/s; the _yf32 variants store the float32
sums unrounded), attn1024_31f_bf16 (the attention
block over 31 frames, TFLOP/s), attn384_s14400_21f_bf16 and attn1024_s14400_21f_bf16 (the block
over 21 frames of the Wan2.1 720p latent, 90x160 positions, at widths 384 and 1024).
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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas():
    """The BLAS libraries behind the oracle's products (torch.mm for the convs, numpy for the
    attention) and their thread counts."""
    import re

    import torch
    cfg = torch.__config__.show()
    tb = re.findall(r"(?:BLAS_INFO|LAPACK_INFO)=[^,\s]+", cfg)
    try:
        info = np.show_config(mode="dicts")
        nb = info.get("Build Dependencies", {}).get("blas", {}).get("name", "unknown")
    except Exception:  # noqa: BLE001
        nb = "unknown"
    return {"torch": ", ".join(tb) or "unknown", "torch_threads": torch.get_num_threads(), "numpy": nb}


def cpu_baseline(cfg, W, mode="bf16", chunks=3):
    """The CPU oracle as it stands (float64 sums, the mode's rounding points) decoding a causal
    prefix of the workload: latent frames 0..chunks-1 (chunk 0, chunk 1, and steady-state chunks
    with two frames of history) of batch element 0, on a crop of the latent with 1/32 of the frame
    area (about 20 s on 16 host cores). Measured: each chunk's seconds. Extrapolated, and
    labelled so: the full decode's time as 32 x (t0 + t1 + (T - 2) x t_steady) (conv work scales
    with the area; the attention, which scales with its square, is under 0.2% of the work) and
    its frames/s."""
    import oracle
    ch, cw = (11, 10) if cfg.h <= cfg.w else (10, 11)
    z = np.ascontiguousarray(cfg.latents()[:1, :, :chunks, :ch, :cw])
    marks = []
    t0 = time.perf_counter()
    oracle.decode(z, W, mode, on_chunk=lambda i: marks.append(time.perf_counter()))
    per = [b - a for a, b in zip([t0] + marks[:-1], marks)]
    scale = (cfg.h * cfg.w) / (ch * cw)
    t_full = scale * (per[0] + per[1] + (cfg.T - 2) * per[-1])
    frames = cfg.B * cfg.frames
    return {"value": round(frames / (cfg.B * t_full), 6), "unit": "frames/s", "cores": _cores(), "kind": "oracle",
            "extrapolated": True, "seconds": round(sum(per), 2), "chunk_seconds": [round(t, 2) for t in per],
            "full_decode_seconds_extrapolated": round(t_full, 1),
            "cpu_model": _cpu_model(), "blas": _blas(),
            "sample": f"oracle.decode ({mode} mode, float64 sums) of latent frames 0..{chunks - 1} (chunk 0, chunk 1 and "
                      f"{chunks - 2} steady chunk) on a {ch}x{cw} crop of the [{cfg.B},48,{cfg.T},{cfg.h},{cfg.w}] latents "
                      f"(batch element 0), 1/{scale:.0f} of the frame area; value = {frames} frames / the extrapolated "
                      f"time of the whole batch, {cfg.B} x {scale:.0f} x (t0 + t1 + {cfg.T - 2} x t_steady) "
                      "(extrapolated, not measured)"}


CPU_SAMPLE_SECONDS = 10.0  # the single-op oracle samples repeat until this much CPU time has passed


def _cores():
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or str(cores)
    return int(threads) if threads.isdigit() else cores


def cpu_baseline_conv(cfg):
    """The CPU oracle's causal conv (bf16 rounding, float64 sums) on the workload's tensors,
    cropped to at most 88 x 160 positions per frame, in TFLOP/s of algorithmic work."""
    import oracle
    x, cache, w, b = cfg.tensors()
    hh, ww = min(cfg.h, 88), min(cfg.w, 160)
    R = oracle.round_bf16
    xs = R(np.ascontiguousarray(x[:, :, :, :hh, :ww]))
    cs = R(np.ascontiguousarray(cache[:, :, :, :hh, :ww])) if cfg.n_cache else None
    P = oracle.Prec("bf16")
    wr, br = R(w), R(b)
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < CPU_SAMPLE_SECONDS:
        oracle.causal_conv(xs, wr, br, cs, P)
        n += 1
    dt = time.perf_counter() - t0
    flops = 2.0 * cfg.t * hh * ww * cfg.C * cfg.C * 27
    return {"value": round(n * flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _cores(), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"oracle.causal_conv (bf16 mode, float64 sums) on the workload's x and {cfg.n_cache} cached frames "
                      f"cropped to {cfg.t} frames of {hh}x{ww} ({flops / 1e9:.1f} GFLOP), run {n} times"}


def cpu_baseline_attn(cfg):
    """The CPU oracle's attention block (bf16 rounding, float64 sums) on frame 0 of the workload
    at its first R query positions (every key and value used), in TFLOP/s of the block's
    algorithmic work for those R queries."""
    import oracle
    T = cfg.tensors()
    S, C = cfg.h * cfg.w, cfg.C
    rows = np.arange(min(S, 4096))
    R = oracle.round_bf16
    frame = R(np.ascontiguousarray(T["x"][0, :, 0]))
    par = [R(T[k]) for k in ("gamma", "qkv_w", "qkv_b", "proj_w", "proj_b")]
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < CPU_SAMPLE_SECONDS:
        oracle.attention_rows(frame, *par, oracle.Prec("bf16"), rows)
        n += 1
    dt = time.perf_counter() - t0
    flops = len(rows) * (4.0 * S * C + 8.0 * C * C)
    return {"value": round(n * flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _cores(), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"oracle.attention_rows (bf16 mode, float64 sums) on frame 0 ({S} positions, C = {C}) at its first "
                      f"{len(rows)} queries, run {n} times; value = the block's work for those queries "
                      f"({flops / 1e9:.1f} GFLOP per run) / seconds (the oracle also projects k and v for every position, "
                      "not counted)"}


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


DECODES = {"ti2v5b_landscape_bf16": ("ti2v5b_landscape", "bf16"), "ti2v5b_landscape_fp32": ("ti2v5b_landscape", "fp32"),
           "ti2v5b_portrait_bf16": ("ti2v5b_portrait", "bf16"), "ti2v5b_landscape_b2_bf16": ("ti2v5b_landscape_b2", "bf16"),
           "ti2v5b_landscape_bf16_tiled": ("ti2v5b_landscape", "bf16")}
TILED = {"ti2v5b_landscape_bf16_tiled": ((256, 256), (192, 192))}  # the page's default tile and stride
SINGLE = {"conv1024_l0_bf16": ("conv", "conv1024_l0"), "conv256_l3_bf16": ("conv", "conv256_l3"),
          "conv1024_l0_bf16_yf32": ("conv", "conv1024_l0"), "conv256_l3_bf16_yf32": ("conv", "conv256_l3"),
          "attn1024_31f_bf16": ("attn", "attn1024_31f"), "attn384_s14400_21f_bf16": ("attn", "attn384_s14400_21f"),
          "attn1024_s14400_21f_bf16": ("attn", "attn1024_s14400_21f")}


def kernel_classes(prof, steps):
    out = {}
    for k, p in prof.items():
        e = {"ms_per_step": round(p["ms"] / steps, 3), "launches_per_step": p["launches"] // max(1, steps)}
        if p["flops"]:
            e["TFLOP/s"] = round(p["flops"] / (p["ms"] * 1e-3) / 1e12, 2)
        if p["bytes"]:
            e["GB/s"] = round(p["bytes"] / (p["ms"] * 1e-3) / 1e9, 1)
            e["frac_of_peak"] = round(e["GB/s"] / PEAK_HBM_GBS, 4)
        out[k] = e
    return out


def single_op(name, args):
    """One causal conv (C2a, C2b) or the attention block (C3, and at the 720p latent frame) in
    bf16, NTHWC operands resident in HBM; value = the op's algorithmic TFLOP/s over the timed
    wall time; cpu_baseline = the oracle's rate on a bounded sample of the same op."""
    import torch

    import synthetic
    from video_vae_decoding_amd import wanvae
    kind, cfg_name = SINGLE[name]
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    if kind == "conv":
        cfg = synthetic.CONV_CONFIGS[cfg_name]
        x, cache, w, b = cfg.tensors()
        xt = torch.from_numpy(x).to(dev).to(bf).permute(0, 2, 3, 4, 1).contiguous()
        ct = torch.from_numpy(cache).to(dev).to(bf).permute(0, 2, 3, 4, 1).contiguous()
        wt, bt = torch.from_numpy(w).to(dev), torch.from_numpy(b).to(dev)
        ydt = torch.float32 if name.endswith("_yf32") else bf
        y = torch.empty(1, cfg.t, cfg.h, cfg.w, cfg.C, dtype=ydt, device=dev)
        ws = torch.empty(wanvae.conv_workspace_size(1, cfg.C, cfg.C, cfg.t, cfg.h, cfg.w, cfg.n_cache, "nthwc", bf, ydt),
                         dtype=torch.uint8, device=dev)
        run = lambda: wanvae.wanvae_causal_conv3d(xt, ct, wt, bt, layout="nthwc", y=y, workspace=ws, y_dtype=ydt)
        flops = 2.0 * cfg.t * cfg.h * cfg.w * cfg.C * cfg.C * 27
        config = {"workload": name, "x": [1, cfg.C, cfg.t, cfg.h, cfg.w], "n_cache": cfg.n_cache, "kernel": "3x3x3",
                  "y_dtype": "fp32" if ydt == torch.float32 else "bf16"}
    else:
        cfg = synthetic.ATTN_CONFIGS[cfg_name]
        T = cfg.tensors()
        xt = torch.from_numpy(T["x"]).to(dev).to(bf).permute(0, 2, 3, 4, 1).contiguous()
        par = [torch.from_numpy(T[k]).to(dev) for k in ("gamma", "qkv_w", "qkv_b", "proj_w", "proj_b")]
        y = torch.empty_like(xt)
        ws = torch.empty(wanvae.attn_workspace_size(1, cfg.C, cfg.T, cfg.h, cfg.w, "nthwc", bf), dtype=torch.uint8,
                         device=dev)
        run = lambda: wanvae.wanvae_attn_block(xt, *par, layout="nthwc", y=y, workspace=ws)
        S = cfg.h * cfg.w
        flops = cfg.T * (4.0 * S * S * cfg.C + 2.0 * S * cfg.C * 4 * cfg.C)  # core + q-k-v and output projections
        config = {"workload": name, "x": [1, cfg.C, cfg.T, cfg.h, cfg.w], "S": S, "heads": 1}
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    wanvae.wanvae_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = {k: wanvae.wanvae_profile_read(getattr(wanvae, "K" + k.upper())) for k in ("conv", "norm", "attn", "other")}
    wanvae.wanvae_profile_enable(False)
    main_k = prof["conv" if kind == "conv" else "attn"]
    tf = main_k["flops"] / (main_k["ms"] * 1e-3) / 1e12
    out = {"metric": f"{'conv' if kind == 'conv' else 'attention block'} TFLOP/s (bf16)",
           "value": round(flops * args.steps / elapsed / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": config,
           "roofline": {"bound": "mfma", "kernel": "conv" if kind == "conv" else (
               "attention core (bf16: k_attn_mm scores, k_attn_fac, k_attn_mm P V; fp32: k_attn)"),
                        "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "launches": main_k["launches"], "avg_launch_ms": round(main_k["ms"] / max(1, main_k["launches"]), 4)},
           "kernels": kernel_classes(prof, args.steps)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on its sample ...")
        out["cpu_baseline"] = cpu_baseline_conv(cfg) if kind == "conv" else cpu_baseline_attn(cfg)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--workload", default="ti2v5b_landscape_bf16", choices=sorted(DECODES) + sorted(SINGLE))
    ap.add_argument("--no-pipeline", action="store_true",
                    help="decode in chunk order on one stream (default: the two-stream chunk pipeline)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decoder here runs on a single MI355X (got --gpus {args.gpus}); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.workload in SINGLE:
        single_op(args.workload, args)
        return

    import torch

    import synthetic
    from video_vae_decoding_amd import wanvae

    dev = torch.device("cuda:0")
    wanvae.wanvae_set_decode_pipeline(not args.no_pipeline)
    cfg_name, mode = DECODES[args.workload]
    cfg = synthetic.DECODE_CONFIGS[cfg_name]
    log("generating inputs ...")
    z, W = cfg.latents(), cfg.weights()
    zt = torch.from_numpy(z).to(dev)
    Wt = {k: torch.from_numpy(v).to(dev) for k, v in W.items()}
    dtype = torch.bfloat16 if mode == "bf16" else torch.float32
    peak = PEAK_BF16_TFLOPS if mode == "bf16" else PEAK_FP32_TFLOPS
    frames = cfg.B * cfg.frames
    video = torch.empty((cfg.B, 3, cfg.frames, 16 * cfg.h, 16 * cfg.w), dtype=dtype, device=dev)
    tiled = TILED.get(args.workload)
    if tiled:
        ws = torch.empty(wanvae.decode_tiled_workspace_size(cfg.B, cfg.T, cfg.h, cfg.w, Wt, dtype, *tiled),
                         dtype=torch.uint8, device=dev)
        run = lambda: wanvae.wanvae_decode_tiled(zt, Wt, dtype, *tiled, video=video, workspace=ws)
    else:
        ws = torch.empty(wanvae.decode_workspace_size(cfg.B, cfg.T, cfg.h, cfg.w, Wt, dtype), dtype=torch.uint8,
                         device=dev)
        run = lambda: wanvae.wanvae_decode(zt, Wt, dtype, video=video, workspace=ws)
    for i in range(args.warmup):
        run()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    # the timed region: K decodes as a caller runs them (the two-stream chunk pipeline unless
    # --no-pipeline)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    log(f"timed {args.steps} decodes in {elapsed:.3f} s")
    assert torch.isfinite(video).all()
    # the kernel region: K more decodes in chunk order on one stream, every kernel timed with HIP
    # events on its stream. Run alone, each kernel's event time is its own: with the pipeline
    # the two streams' kernels share the chip and their event times overlap.
    wanvae.wanvae_set_decode_pipeline(False)
    wanvae.wanvae_profile_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        run()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    prof = {k: wanvae.wanvae_profile_read(getattr(wanvae, "K" + k.upper())) for k in ("conv", "norm", "attn", "other")}
    wanvae.wanvae_profile_enable(False)
    wanvae.wanvae_set_decode_pipeline(not args.no_pipeline)
    log(f"kernel region: {args.steps} decodes in chunk order in {t3 - t2:.3f} s")

    conv = prof["conv"]
    conv_tflops = conv["flops"] / (conv["ms"] * 1e-3) / 1e12
    kernels = kernel_classes(prof, args.steps)
    for k in ("conv", "attn"):
        if "TFLOP/s" in kernels[k]:
            kernels[k]["frac_of_peak"] = round(kernels[k]["TFLOP/s"] / peak, 4)
    default = args.workload == "ti2v5b_landscape_bf16"
    out = {
        "metric": METRIC if default else METRIC.replace("704x1280 bf16", f"{16 * cfg.h}x{16 * cfg.w} {mode}"),
        "value": round(frames * args.steps / elapsed, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mode,
        "data": "synthetic",
        "config": {"workload": f"ti2v5b_vae_decode_{16 * cfg.h}x{16 * cfg.w}x{cfg.frames}_{mode}" + ("" if cfg.B == 1 else f"_b{cfg.B}")
                   + ("" if not tiled else f"_tiled{tiled[0][0]}s{tiled[1][0]}"),
                   "latent": [cfg.B, 48, cfg.T, cfg.h, cfg.w],
                   "video": [cfg.B, 3, cfg.frames, 16 * cfg.h, 16 * cfg.w], "weights": f"random-init, seed {cfg.seed}",
                   "accumulate": "fp32", "pipeline": not args.no_pipeline, "workspace_bytes": ws.numel()},
        "roofline": {"bound": "mfma",
                     "kernel": ("conv (k_conv_halo for the 3x3 convs, k_conv_dma for the rest; all launches of a decode)"
                                if mode == "bf16" else "conv (k_conv_dma, fp32 MFMA; k_conv for conv_out; all launches of a decode)"),
                     "achieved": round(conv_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(conv_tflops / peak, 4), "traffic": stored_traffic() if default else None,
                     "launches": conv["launches"], "avg_launch_ms": round(conv["ms"] / max(1, conv["launches"]), 4),
                     "algorithmic_tflop_per_step": round(conv["flops"] / args.steps / 1e12, 2)},
        "kernels": kernels,
        "chunk_order": {"frames/s": round(frames * args.steps / (t3 - t2), 3),
                        "ms_per_step": round((t3 - t2) / args.steps * 1e3, 2),
                        "note": "the kernel region: the same decodes in chunk order on one stream, "
                                "with per-kernel HIP events (roofline and kernels come from it)"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on its sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg, W, mode)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
