"""Pins of the oracle's parts (CPU only).

Each part of the oracle is checked against something other than itself: brute
force on tiny inputs, a torch CPU library routine in float64, a closed form, or
an invariant stated on FastVideo's "wan22_vae_decode reference.py" page or on
MaxDiffusion PR #514's page.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.decoder import clamp

P64 = oracle.Prec("fp64")
P32 = oracle.Prec("fp32")
PBF = oracle.Prec("bf16")


def rnd(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------ bf16 rounding

def rne_bf16_bits(x):
    """Round to nearest even, float32 -> bfloat16, on the bit patterns (reference)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32)


def test_round_bf16_is_round_to_nearest_even():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 20000),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1e-45, 1.1754944e-38], np.float32),
    ]).astype(np.float32)
    # exact ties: the low 16 bits are 0x8000, half way between two bf16 values
    ties = (g.integers(0, 2**15, 4000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    got = oracle.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), rne_bf16_bits(x).view(np.uint32))
    # ties go to the even neighbour
    assert oracle.round_bf16(np.array([1.00390625], np.float32))[0] == 1.0          # 1 + 2^-8: tie, even is 1
    assert oracle.round_bf16(np.array([1.01171875], np.float32))[0] == 1.015625     # 1 + 3*2^-8: tie, even is 1 + 2^-6
    assert np.isnan(oracle.round_bf16(np.array([np.nan], np.float32)))[0]


# ------------------------------------------------------------------ causal conv

def naive_conv(x, w, b, hist):
    """Seven nested Python loops over the padded input (brute force)."""
    B, Ci, T, H, W = x.shape
    Co, _, kt, kh, kw = w.shape
    tp = 2 * (kt // 2)
    nh = 0 if hist is None else min(hist.shape[2], tp)
    seq = [np.zeros((B, Ci, H, W))] * (tp - nh)
    if nh:
        seq += [hist[:, :, hist.shape[2] - nh + k] for k in range(nh)]
    seq += [x[:, :, k] for k in range(T)]
    out = np.zeros((B, Co, T, H, W))
    for bb, o, t, y, xx in itertools.product(range(B), range(Co), range(T), range(H), range(W)):
        s = float(b[o])
        for i, dt, dy, dx in itertools.product(range(Ci), range(kt), range(kh), range(kw)):
            yy, xq = y + dy - kh // 2, xx + dx - kw // 2
            if 0 <= yy < H and 0 <= xq < W:
                s += w[o, i, dt, dy, dx] * seq[t + dt][bb, i, yy, xq]
        out[bb, o, t, y, xx] = s
    return out


@pytest.mark.parametrize("kt,kh,kw,nh", [(3, 3, 3, 0), (3, 3, 3, 1), (3, 3, 3, 2), (3, 1, 1, 2), (1, 3, 3, 0), (1, 1, 1, 0), (3, 1, 3, 1)])
def test_conv_brute_force(kt, kh, kw, nh):
    g = np.random.default_rng(kt * 100 + kh * 10 + kw + nh)
    Ci, Co, T, H, W = 3, 4, 3, 4, 5
    x = g.standard_normal((2, Ci, T, H, W))
    w = g.standard_normal((Co, Ci, kt, kh, kw))
    b = g.standard_normal(Co)
    hist = g.standard_normal((2, Ci, nh, H, W)) if nh else None
    got = oracle.causal_conv(x, w, b, hist, P64)
    np.testing.assert_allclose(got, naive_conv(x, w, b, hist), rtol=0, atol=1e-12)


@pytest.mark.parametrize("nh", [0, 1, 2])
def test_conv_matches_torch_conv3d(nh):
    g = np.random.default_rng(7 + nh)
    Ci, Co, T, H, W = 6, 5, 4, 6, 7
    x = g.standard_normal((1, Ci, T, H, W))
    w = g.standard_normal((Co, Ci, 3, 3, 3))
    b = g.standard_normal(Co)
    hist = g.standard_normal((1, Ci, nh, H, W)) if nh else None
    seq = [np.zeros((1, Ci, 2 - nh, H, W))] + ([hist] if nh else []) + [x]
    want = F.conv3d(torch.from_numpy(np.concatenate(seq, 2)), torch.from_numpy(w), torch.from_numpy(b), padding=(0, 1, 1)).numpy()
    np.testing.assert_allclose(oracle.causal_conv(x, w, b, hist, P64), want, rtol=0, atol=1e-12)


def test_conv2d_weight_matches_torch_conv2d():
    g = np.random.default_rng(3)
    x = g.standard_normal((2, 4, 3, 5, 6))
    w = g.standard_normal((7, 4, 3, 3))
    b = g.standard_normal(7)
    got = oracle.causal_conv(x, w, b, None, P64)
    frames = torch.from_numpy(x).permute(0, 2, 1, 3, 4).reshape(6, 4, 5, 6)
    want = F.conv2d(frames, torch.from_numpy(w), torch.from_numpy(b), padding=1).reshape(2, 3, 7, 5, 6).permute(0, 2, 1, 3, 4)
    np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("tap", [(2, 1, 1), (0, 0, 2), (1, 2, 0), (2, 0, 1)])
def test_conv_delta_kernel_is_shifted_copy(tap):
    """A single 1 at tap (dt, dy, dx) mapping channel i to channel i copies the input,
    shifted by (dt - 2, dy - 1, dx - 1), with zeros where the shift leaves the frame."""
    g = np.random.default_rng(1)
    C, T, H, W = 3, 3, 4, 5
    x = g.standard_normal((1, C, T, H, W)).astype(np.float32)
    hist = g.standard_normal((1, C, 2, H, W)).astype(np.float32)
    w = np.zeros((C, C, 3, 3, 3), np.float32)
    dt, dy, dx = tap
    for c in range(C):
        w[c, c, dt, dy, dx] = 1.0
    got = oracle.causal_conv(x, w, np.zeros(C, np.float32), hist, P32)
    seq = np.concatenate([hist, x], 2)
    want = np.zeros_like(x)
    for t, y, xx in itertools.product(range(T), range(H), range(W)):
        yy, xq = y + dy - 1, xx + dx - 1
        if 0 <= yy < H and 0 <= xq < W:
            want[0, :, t, y, xx] = seq[0, :, t + dt, yy, xq]
    assert np.array_equal(got, want)


def test_empty_cache_equals_two_zero_frames_and_conv2d_of_newest_tap():
    """The causal rule: no history is zero padding in time; so a one-frame chunk without
    history is a conv2d with the kernel's newest time tap (index 2)."""
    g = np.random.default_rng(5)
    x = g.standard_normal((1, 4, 1, 5, 6))
    w = g.standard_normal((3, 4, 3, 3, 3))
    b = g.standard_normal(3)
    a = oracle.causal_conv(x, w, b, None, P64)
    z = oracle.causal_conv(x, w, b, np.zeros((1, 4, 2, 5, 6)), P64)
    assert np.array_equal(a, z)
    want = F.conv2d(torch.from_numpy(x[:, :, 0]), torch.from_numpy(w[:, :, 2]), torch.from_numpy(b), padding=1).numpy()
    np.testing.assert_allclose(a[:, :, 0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("splits", [(1, 1, 1, 1, 1, 1, 1), (1, 2, 2, 2), (1, 4, 2), (3, 4), (7,)])
def test_cached_conv_chunks_equal_one_conv_over_the_sequence(splits):
    """'The loop thus computes, chunk by chunk, what one causal conv over the whole sequence
    would, with zeros before the first frame' (Causal caches)."""
    g = np.random.default_rng(11)
    x = g.standard_normal((2, 3, sum(splits), 4, 4))
    w = g.standard_normal((5, 3, 3, 3, 3))
    b = g.standard_normal(5)
    whole = oracle.causal_conv(x, w, b, None, P64)
    cache, outs, t0 = {}, [], 0
    for n in splits:
        outs.append(oracle.cached_conv(x[:, :, t0:t0 + n], w, b, "c", cache, P64))
        t0 += n
        assert cache["c"].shape[2] == min(2, t0)
        np.testing.assert_array_equal(cache["c"], x[:, :, max(0, t0 - 2):t0])
    np.testing.assert_allclose(np.concatenate(outs, 2), whole, rtol=0, atol=1e-12)


def test_conv_points_match_conv():
    g = np.random.default_rng(2)
    x = g.standard_normal((2, 5, 3, 6, 7))
    hist = g.standard_normal((2, 5, 2, 6, 7))
    w = g.standard_normal((4, 5, 3, 3, 3))
    b = g.standard_normal(4)
    full = oracle.causal_conv(x, w, b, hist, P64)
    pts = np.array([[bb, o, t, y, xx] for bb, o, t, y, xx in itertools.product(range(2), range(4), range(3), (0, 3, 5), (0, 4, 6))])
    got = oracle.conv_points(np.concatenate([hist, x], 2), w, b, pts)
    np.testing.assert_allclose(got, full[tuple(pts.T)], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ RMS norm, SiLU

def test_rms_norm_matches_f_normalize():
    g = np.random.default_rng(4)
    x = g.standard_normal((2, 16, 3, 4, 5))
    gamma = 1 + 0.1 * g.standard_normal((16, 1, 1, 1))
    want = F.normalize(torch.from_numpy(x), dim=1).numpy() * 4.0 * gamma.reshape(1, 16, 1, 1, 1)
    np.testing.assert_allclose(oracle.rms_norm(x, gamma, P64), want, rtol=1e-14, atol=0)


def test_rms_norm_closed_forms():
    g = np.random.default_rng(6)
    x = g.standard_normal((1, 24, 2, 3, 3))
    gamma = 1 + 0.1 * g.standard_normal(24)
    y = oracle.rms_norm(x, gamma, P64)
    unit = np.linalg.norm(y / (math.sqrt(24) * gamma.reshape(1, 24, 1, 1, 1)), axis=1)
    np.testing.assert_allclose(unit, 1.0, rtol=1e-14)
    assert np.array_equal(oracle.rms_norm(np.zeros((1, 8, 1, 2, 2)), np.ones(8), P64), np.zeros((1, 8, 1, 2, 2)))
    tiny = np.full((1, 4, 1, 1, 1), 1e-14)        # ||x|| = 2e-14 < 1e-12: divided by the eps
    np.testing.assert_allclose(oracle.rms_norm(tiny, np.ones(4), P64), tiny * 1e12 * 2.0, rtol=1e-14)


def test_rms_norm_bf16_rounding_points_match_torch_bf16():
    """bf16: normalise in fp32, round to bf16, then x sqrt(C) and x gamma each round (the
    torch CPU bf16 arithmetic of those three steps)."""
    g = np.random.default_rng(8)
    for C in (16, 32, 512):
        x = oracle.round_bf16(g.standard_normal((1, C, 2, 3, 4)))
        gamma = oracle.round_bf16(1 + 0.1 * g.standard_normal((C, 1, 1, 1)))
        xt = torch.from_numpy(x).to(torch.bfloat16)
        xh = F.normalize(xt.float(), dim=1).to(torch.bfloat16)
        want = (xh * C ** 0.5 * torch.from_numpy(gamma).to(torch.bfloat16)).float().numpy()
        got = oracle.rms_norm(x, gamma, PBF)
        # the oracle computes the norm in float64, torch in float32: ties may round apart
        ulp = np.abs(want) * 2.0 ** -7
        assert np.all(np.abs(got - want) <= ulp)
        assert np.mean(got == want) > 0.99


def test_silu_matches_torch():
    v = np.linspace(-60, 60, 2001)
    np.testing.assert_allclose(oracle.silu(v, P64), F.silu(torch.from_numpy(v)).numpy(), rtol=1e-15, atol=1e-300)
    assert oracle.silu(np.array([0.0]), P64)[0] == 0.0
    vb = oracle.round_bf16(np.linspace(-8, 8, 4001))
    want = F.silu(torch.from_numpy(vb).to(torch.bfloat16)).float().numpy()
    got = oracle.silu(vb, PBF)
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)


# ------------------------------------------------------------------ attention

def _attn_weights(g, C):
    return (1 + 0.1 * g.standard_normal((C, 1, 1)), g.standard_normal((3 * C, C, 1, 1)) / math.sqrt(C),
            g.standard_normal(3 * C) * 0.1, g.standard_normal((C, C, 1, 1)) / math.sqrt(C), g.standard_normal(C) * 0.1)


def test_attention_single_key_is_proj_v_plus_x():
    """With one position per frame softmax over a single key is 1 and the block returns
    proj(v) + x (MaxDiffusion PR #514's page, the bug it fixes). Random q, k and identity
    v / proj weights make every other sum a single term, so the identity is checked bit for
    bit; random weights everywhere are checked to 1e-12."""
    g = np.random.default_rng(9)
    C = 32
    x = g.standard_normal((2, C, 3, 1, 1))
    gm, wq, bq, wp, bp = _attn_weights(g, C)
    wq[2 * C:, :, 0, 0] = np.eye(C)
    wid = np.eye(C).reshape(C, C, 1, 1)
    for P in (P64, P32, PBF):
        xs = P.R(x)
        got = oracle.attention(xs, gm, wq, bq, wid, np.zeros(C), P)
        # the norm per frame [1, C, h, w], as the block takes it (numpy's reduction order
        # depends on the array's rank)
        n = np.stack([oracle.rms_norm(xs[:, :, t], gm, P) for t in range(3)], 2).astype(np.float64)
        v = P.R(n + bq[2 * C:].reshape(1, C, 1, 1, 1))
        want = P.R(v.astype(np.float64) + xs.astype(np.float64))
        assert np.array_equal(got, want)
    gm, wq, bq, wp, bp = _attn_weights(g, C)
    got = oracle.attention(x, gm, wq, bq, wp, bp, P64)
    n = oracle.rms_norm(x, gm.reshape(C, 1, 1, 1), P64)
    v = np.einsum("oc,bcthw->bothw", wq[2 * C:, :, 0, 0], n) + bq[2 * C:].reshape(1, C, 1, 1, 1)
    want = np.einsum("oc,bcthw->bothw", wp[:, :, 0, 0], v) + bp.reshape(1, C, 1, 1, 1) + x
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_attention_attends_when_frame_has_many_positions():
    """With the fix the block no longer equals proj(v) + x (the page's CPU check prints 0.0 before
    and a non-zero difference after)."""
    g = np.random.default_rng(10)
    C = 32
    x = g.standard_normal((1, C, 2, 4, 6))
    gm, wq, bq, wp, bp = _attn_weights(g, C)
    got = oracle.attention(x, gm, wq, bq, wp, bp, P64)
    n = oracle.rms_norm(x, gm.reshape(C, 1, 1, 1), P64)
    v = np.einsum("oc,bcthw->bothw", wq[2 * C:, :, 0, 0], n) + bq[2 * C:].reshape(1, C, 1, 1, 1)
    no_attn = np.einsum("oc,bcthw->bothw", wp[:, :, 0, 0], v) + bp.reshape(1, C, 1, 1, 1) + x
    assert np.max(np.abs(got - no_attn)) > 0.1


def test_attention_zero_queries_average_values():
    g = np.random.default_rng(12)
    C = 16
    x = g.standard_normal((1, C, 2, 3, 5))
    gm, wq, bq, wp, bp = _attn_weights(g, C)
    wq[:C] = 0
    bq[:C] = 0
    got = oracle.attention(x, gm, wq, bq, wp, bp, P64)
    n = oracle.rms_norm(x, gm.reshape(C, 1, 1, 1), P64)
    v = np.einsum("oc,bcthw->bothw", wq[2 * C:, :, 0, 0], n) + bq[2 * C:].reshape(1, C, 1, 1, 1)
    o = np.broadcast_to(v.mean(axis=(3, 4), keepdims=True), v.shape)
    want = np.einsum("oc,bcthw->bothw", wp[:, :, 0, 0], o) + bp.reshape(1, C, 1, 1, 1) + x
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["fp64", "fp32", "bf16"])
def test_attention_rows_equals_the_full_block_at_those_rows(mode):
    """attention_rows (queries restricted to a subset of positions) gives the full block's
    outputs at those positions: the same values, up to the summation order of the row
    subset's matrix products (a bf16 rounding may then flip by one spacing)."""
    g = np.random.default_rng(11)
    C, H, W = 32, 5, 7
    x = g.standard_normal((1, C, 1, H, W))
    gm = 1 + 0.1 * g.standard_normal((C, 1, 1))
    wq = g.standard_normal((3 * C, C, 1, 1)) / np.sqrt(C)
    bq = g.standard_normal(3 * C) / np.sqrt(C)
    wp = g.standard_normal((C, C, 1, 1)) / np.sqrt(C)
    bp = g.standard_normal(C) / np.sqrt(C)
    P = oracle.Prec(mode)
    if mode != "fp64":
        x, gm, wq, bq, wp, bp = (P.R(a) for a in (x, gm, wq, bq, wp, bp))
    full = oracle.attention(x, gm, wq, bq, wp, bp, P)[0, :, 0].reshape(C, H * W).T
    rows = np.array([0, 3, 17, 34, 20, 9])
    got = oracle.attention_rows(x[0, :, 0], gm, wq, bq, wp, bp, P, rows)
    assert got.shape == (len(rows), C)
    if mode == "fp64":
        np.testing.assert_allclose(got, full[rows], rtol=1e-12, atol=1e-12)
    else:
        d = np.abs(got - full[rows])
        spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(full[rows]), 1e-30))) - (7 if mode == "bf16" else 23))
        assert np.all(d <= spacing), d.max()
        assert np.mean(d == 0) >= 0.99


def test_attention_matches_torch_sdpa():
    """q, k, v from the (N*T, H*W, 1, C) layout through torch's scaled_dot_product_attention
    in float64, one head of dim C."""
    g = np.random.default_rng(13)
    C, T, H, W = 32, 3, 4, 5
    x = g.standard_normal((2, C, T, H, W))
    gm, wq, bq, wp, bp = _attn_weights(g, C)
    xt = torch.from_numpy(x).permute(0, 2, 1, 3, 4).reshape(2 * T, C, H, W)
    n = F.normalize(xt, dim=1) * math.sqrt(C) * torch.from_numpy(gm)
    qkv = F.conv2d(n, torch.from_numpy(wq), torch.from_numpy(bq))
    qkv = qkv.reshape(2 * T, 3 * C, H * W).transpose(1, 2)[:, None]       # [N*T, 1 head, H*W, 3C]
    q, k, v = qkv.chunk(3, dim=-1)
    o = F.scaled_dot_product_attention(q, k, v)[:, 0].transpose(1, 2).reshape(2 * T, C, H, W)
    y = F.conv2d(o, torch.from_numpy(wp), torch.from_numpy(bp)) + xt
    want = y.reshape(2, T, C, H, W).permute(0, 2, 1, 3, 4).numpy()
    np.testing.assert_allclose(oracle.attention(x, gm, wq, bq, wp, bp, P64), want, rtol=0, atol=1e-12)


def test_attention_is_permutation_equivariant_over_positions():
    g = np.random.default_rng(14)
    C, H, W = 16, 3, 4
    x = g.standard_normal((1, C, 1, H, W))
    gm, wq, bq, wp, bp = _attn_weights(g, C)
    perm = g.permutation(H * W)
    xp = x.reshape(1, C, 1, H * W)[..., perm].reshape(x.shape)
    a = oracle.attention(x, gm, wq, bq, wp, bp, P64).reshape(1, C, 1, H * W)[..., perm]
    b = oracle.attention(xp, gm, wq, bq, wp, bp, P64).reshape(1, C, 1, H * W)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ resampling, DupUp3D, unpatchify

def test_time_upsample_interleaves_channel_halves_into_frames():
    """Weights +1 (first half) and -1 (second half) on the newest time tap: frame 2t = x_t,
    frame 2t+1 = -x_t."""
    g = np.random.default_rng(15)
    C = 4
    x = g.standard_normal((1, C, 3, 2, 3)).astype(np.float32)
    w = np.zeros((2 * C, C, 3, 1, 1), np.float32)
    for c in range(C):
        w[c, c, 2] = 1
        w[C + c, c, 2] = -1
    Wt = {"tc.weight": w, "tc.bias": np.zeros(2 * C, np.float32)}
    out = oracle.time_upsample(x, Wt, "tc", {}, P32)
    assert out.shape == (1, C, 6, 2, 3)
    assert np.array_equal(out[:, :, 0::2], x) and np.array_equal(out[:, :, 1::2], -x)


def test_spatial_upsample_is_nearest_exact_then_conv2d():
    g = np.random.default_rng(16)
    x = g.standard_normal((1, 3, 2, 3, 4))
    w = g.standard_normal((5, 3, 3, 3))
    b = g.standard_normal(5)
    frames = torch.from_numpy(x).permute(0, 2, 1, 3, 4).reshape(2, 3, 3, 4)
    u = F.interpolate(frames, scale_factor=(2.0, 2.0), mode="nearest-exact")
    want = F.conv2d(u, torch.from_numpy(w), torch.from_numpy(b), padding=1).reshape(1, 2, 5, 6, 8).permute(0, 2, 1, 3, 4)
    np.testing.assert_allclose(oracle.spatial_upsample(x, w, b, P64), want.numpy(), rtol=0, atol=1e-12)
    # identity 3x3 kernel: the nearest-upsampled copy itself
    wid = np.zeros((3, 3, 3, 3))
    for c in range(3):
        wid[c, c, 1, 1] = 1
    np.testing.assert_array_equal(oracle.spatial_upsample(x, wid, np.zeros(3), P64),
                                  u.reshape(1, 2, 3, 6, 8).permute(0, 2, 1, 3, 4).numpy())


def test_dup_up_r8_is_nearest_in_t_h_w():
    g = np.random.default_rng(17)
    x = g.standard_normal((2, 8, 3, 2, 3))
    d = oracle.dup_up(x, 8, 2, first=False)
    want = np.repeat(np.repeat(np.repeat(x, 2, 2), 2, 3), 2, 4)
    assert np.array_equal(d, want)
    d0 = oracle.dup_up(x[:, :, :1], 8, 2, first=True)
    assert np.array_equal(d0, want[:, :, 1:2])         # first chunk: the last time copy only


def test_dup_up_r2_channel_pairs_become_row_pairs():
    g = np.random.default_rng(18)
    x = g.standard_normal((1, 8, 2, 2, 3))
    d = oracle.dup_up(x, 4, 1, first=False)            # in 8 -> out 4, ft 1: r = 2
    assert d.shape == (1, 4, 2, 4, 6)
    for c, i, j in itertools.product(range(4), range(2), range(2)):
        assert np.array_equal(d[:, c, :, i::2, j::2], x[:, 2 * c + i])
    assert np.array_equal(oracle.dup_up(x, 4, 1, first=True), d)


def test_unpatchify_is_pixel_shuffle_with_row_column_offsets_swapped():
    """unpatchify's channel 4k + 2j + i holds row offset i, column offset j; pixel_shuffle's
    channel 4k + 2i + j does: the two agree after swapping i and j in the channel order."""
    g = np.random.default_rng(19)
    x = g.standard_normal((2, 12, 3, 4, 5)).astype(np.float32)
    perm = [4 * k + 2 * j + i for k in range(3) for i in range(2) for j in range(2)]
    frames = torch.from_numpy(x[:, perm]).permute(0, 2, 1, 3, 4).reshape(6, 12, 4, 5)
    want = F.pixel_shuffle(frames, 2).reshape(2, 3, 3, 8, 10).permute(0, 2, 1, 3, 4).numpy()
    assert np.array_equal(oracle.unpatchify(x), want)


def test_clamp_keeps_nan_and_bounds():
    v = np.array([-3.0, -1.0, -0.5, 0.0, 0.5, 1.0, 7.0, np.nan, np.inf, -np.inf], np.float32)
    out = clamp(v)
    assert np.array_equal(out[:7], np.array([-1, -1, -0.5, 0, 0.5, 1, 1], np.float32))
    assert np.isnan(out[7]) and out[8] == 1 and out[9] == -1
    want = torch.clamp(torch.from_numpy(v), -1.0, 1.0).numpy()
    assert np.array_equal(out, want, equal_nan=True)


def test_psnr_definition():
    a = np.zeros(100)
    b = np.full(100, 0.2)                       # ((a - b)/2)^2 = 0.01 -> 20 dB
    assert abs(oracle.psnr(a, b) - 20.0) < 1e-12
    assert oracle.psnr(a, a) == float("inf")


def test_prec_rejects_other_dtypes():
    with pytest.raises(ValueError):
        oracle.Prec("fp16")
