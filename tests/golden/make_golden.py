"""Writes the stored expected values of the full-size decode parity tests.

Calls only the CPU oracle (``oracle/``) and the seeded inputs (``synthetic/``). A decode's
first 4k - 3 frames depend only on its first k latent frames (each chunk sees earlier ones
only through the causal caches), so the oracle decodes the first K_CHUNKS latent frames of
each full-size workload and this script keeps the video at N_SAMPLES seeded positions. The
videos of a batch are independent, so a batch element can be decoded on its own.

    python tests/golden/make_golden.py [--out DIR] [--chunks K] config:mode[:batch][:f32] ...

Outputs, per job: ``<config>_<mode>[_b<batch>].npy`` (float32 sampled values) and the same
name with ``.json`` (recipe, oracle wall time, summary statistics). With ``f32`` the oracle
sums in float32 instead of float64 (name suffix ``_accf32``): the same decode in another
accumulation order, which bounds how much a bf16 decode moves with the order of its sums.
``--chunks K`` decodes K latent frames (4K - 3 video frames); the landscape files use 4, so that
two chunks run in the steady state, where every time conv has two frames of history.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

K_CHUNKS = 2          # default latent frames decoded -> 4*K_CHUNKS - 3 = 5 video frames
N_SAMPLES = 65536
SAMPLE_SEED = 20251202

JOBS = [("ti2v5b_landscape", "bf16"), ("ti2v5b_landscape", "fp32"), ("ti2v5b_portrait", "bf16"),
        ("ti2v5b_landscape_b2", "bf16:0"), ("ti2v5b_landscape_b2", "bf16:1")]


def sample_index(shape, n=N_SAMPLES, seed=SAMPLE_SEED):
    """Seeded sample positions (one int64 array per video axis) in a video of ``shape``."""
    g = np.random.default_rng(seed)
    return tuple(g.integers(0, s, n) for s in shape)


def golden_name(config, mode, batch=None, acc="f64"):
    return f"{config}_{mode}" + ("" if batch is None else f"_b{batch}") + ("" if acc == "f64" else f"_acc{acc}")


def golden_paths(config, mode, batch=None, out=HERE, acc="f64"):
    base = os.path.join(out, golden_name(config, mode, batch, acc))
    return base + ".npy", base + ".json"


def make(config, mode, batch=None, out=HERE, acc="f64", chunks=K_CHUNKS):
    import oracle
    import synthetic
    cfg = synthetic.DECODE_CONFIGS[config]
    z = cfg.latents()[:, :, :chunks]
    if batch is not None:
        z = z[batch:batch + 1]
    z = np.ascontiguousarray(z)
    W = cfg.weights()
    t0 = time.time()
    times = []

    def tick(i):
        times.append(time.time() - t0)
        print(f"{config} {mode} batch {batch}: chunk {i} done at {times[-1]:.0f} s", flush=True)

    def step(i, name):
        print(f"  chunk {i}: {name} done at {time.time() - t0:.0f} s", flush=True)

    video = oracle.decode(z, W, mode, acc=acc, on_chunk=tick, on_step=step)
    wall = time.time() - t0
    idx = sample_index(video.shape)
    vals = video[idx].astype(np.float32)
    npy, js = golden_paths(config, mode, batch, out, acc)
    np.save(npy, vals)
    meta = {
        "config": config, "mode": mode, "batch": batch, "acc": acc, "latent_frames": chunks,
        "video_shape": list(video.shape), "n_samples": N_SAMPLES, "sample_seed": SAMPLE_SEED,
        "oracle_seconds": round(wall, 1), "oracle_chunk_seconds": [round(t, 1) for t in times],
        "host_cores": len(os.sched_getaffinity(0)),
        "video_mean": float(video.mean()), "video_std": float(video.std()),
        "clamped_fraction": float(np.mean(np.abs(video) >= 1.0)),
    }
    with open(js, "w") as f:
        json.dump(meta, f, indent=1)
    print(json.dumps(meta), flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    out = HERE
    if args[:1] == ["--out"]:
        out = args[1]
        os.makedirs(out, exist_ok=True)
        args = args[2:]
    chunks = K_CHUNKS
    if args[:1] == ["--chunks"]:
        chunks = int(args[1])
        args = args[2:]
    jobs = []
    for a in args or [f"{c}:{m}" for c, m in JOBS]:
        parts = a.split(":")
        acc = "f32" if parts[-1] == "f32" else "f64"
        parts = [p for p in parts if p != "f32"]
        jobs.append((parts[0], parts[1] if len(parts) > 1 else "bf16", int(parts[2]) if len(parts) > 2 else None, acc))
    for c, m, b, acc in jobs:
        make(c, m, b, out, acc, chunks)
