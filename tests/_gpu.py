"""Helpers of the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("these tests need a GPU (run them with -m gpu on an MI355X)")
    return torch.device("cuda:0")


TORCH = {"fp32": torch.float32, "bf16": torch.bfloat16}


def to_dev(a: np.ndarray, mode: str) -> torch.Tensor:
    """A float32 array on the GPU in the compute type (bf16: nearest-even rounding)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev()).to(TORCH[mode])


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def rounded(a: np.ndarray, mode: str) -> np.ndarray:
    """The oracle's view of an input handed to the GPU in ``mode``."""
    return oracle.round_bf16(a) if mode == "bf16" else np.asarray(a, np.float32)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(e-7) for x in [2^e, 2^(e+1)))."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def acc_bound(K: int, mag) -> np.ndarray:
    """Probabilistic bound on the error of a float32 sum of K products with sum |w x| = mag:
    lambda sqrt(K) u mag with lambda = 8 (Higham and Mary, 'A new approach to probabilistic
    rounding error analysis', 2019: it fails with probability below 2 exp(-lambda^2 / 2))."""
    return 8.0 * np.sqrt(K) * 2.0 ** -24 * np.asarray(mag, np.float64)


def assert_bf16_close(got, want, err=0.0, min_exact=0.98, what=""):
    """bf16 results against the oracle's: |got - want| <= one bf16 spacing (at the larger of
    the two) + err, the bound on the float32 accumulation error before the rounding; most
    values bit-equal."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = np.abs(got - want)
    lim = bf16_ulp(np.maximum(np.abs(got), np.abs(want))) + err
    bad = d > lim
    exact = float(np.mean(d == 0))
    if bad.any():
        k = np.argmax(d - lim)
        raise AssertionError(f"{what}: {int(bad.sum())} values beyond the bound; worst got {got.flat[k]!r} "
                             f"want {want.flat[k]!r} limit {np.broadcast_to(lim, d.shape).flat[k]:.3g}; exact {exact:.4f}")
    assert exact >= min_exact, f"{what}: only {exact:.4f} bit-equal"
    return exact


def gate_bf16_scale(got, want, want_fp32, what):
    """bf16 against the oracle where the tiny decoder runs several chunks: PSNR >= 40 dB, and
    |got - want| within the oracle's own bf16-vs-fp32 distance on the same inputs (mean 1x,
    max 1.5x). Over several chunks the tiny decoder carries any early one-ulp difference into
    every later frame, and such differences settle at the scale of bf16 itself, which is that
    distance (page 3's "Precision" section measures bf16 by it too)."""
    d = np.abs(np.asarray(got, np.float64) - want)
    scale = np.abs(np.asarray(want, np.float64) - want_fp32)
    p = oracle.psnr(got, want)
    say(what, "max", d.max(), "mean", d.mean(), "psnr", p, "bf16-fp32 max", scale.max(), "mean", scale.mean())
    assert p >= 40, p
    assert d.mean() <= scale.mean(), (d.mean(), scale.mean())
    assert d.max() <= 1.5 * scale.max(), (d.max(), scale.max())
