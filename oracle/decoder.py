"""The decoder, written out from the page's definitions (test infrastructure only).

Arrays are NCTHW, [B, C, T, H, W], as on the page. Each function names the
part of FastVideo's "wan22_vae_decode reference.py" page (Wan2.2 VAE decoder
reference) it follows.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MODES = ("fp64", "fp32", "bf16")
CACHE_T = 2           # frames of history a causal conv with a 3-frame kernel keeps ("Causal caches")
PATCH = 2             # unpatchify patch size ("What is computed", step 3)
RESNETS_PER_UP_BLOCK = 3
PREFIXES = ("decoder.", "post_quant_conv.")


def round_bf16(x) -> np.ndarray:
    """Round to bfloat16, nearest even, via float32 (torch's float32 -> bfloat16 cast, a library
    primitive). Returns float32 values that are exactly representable in bfloat16; NaN stays NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return torch.from_numpy(f).to(torch.bfloat16).to(torch.float32).numpy()


class Prec:
    """Rounding and accumulation policy of one decode ("Precision" section of the page)."""

    def __init__(self, mode: str = "fp32", acc: str = "f64"):
        if mode not in MODES:
            raise ValueError(f"mode must be one of {MODES}, not {mode!r}")
        if acc not in ("f64", "f32"):
            raise ValueError(f"acc must be 'f64' or 'f32', not {acc!r}")
        self.mode, self.acc = mode, acc
        self.store = np.float64 if mode == "fp64" else np.float32
        self.acc_t = np.float64 if (acc == "f64" or mode == "fp64") else np.float32

    def R(self, x) -> np.ndarray:
        """Round a computed value to the storage precision."""
        if self.mode == "fp64":
            return np.asarray(x, dtype=np.float64)
        if self.mode == "fp32":
            return np.asarray(x, dtype=np.float32)
        return round_bf16(x)

    def scalar(self, v: float) -> float:
        """A Python-float constant as the fp32/bf16 kernels see it (float32), exact in fp64."""
        return v if self.mode == "fp64" else float(np.float32(v))


# ---------------------------------------------------------------- convolution

_POOL: dict = {}


def _scratch(role: str, shape, dtype) -> torch.Tensor:
    """A reused temporary of the conv (allocating multi-GB buffers afresh for every conv costs
    more than the arithmetic). Contents are undefined."""
    n = int(np.prod(shape))
    t = _POOL.get((role, dtype))
    if t is None or t.numel() < n:
        _POOL[(role, dtype)] = t = torch.empty(n, dtype=dtype)
    return t[:n].view(*shape)


def causal_conv(x, w, b, hist, P: Prec) -> np.ndarray:
    """WanCausalConv3d ("The parts": causal conv): stride 1, spatial zero padding kh//2, kw//2
    on both sides; in time 2*(kt//2) frames before x, the history ``hist`` first (its last
    frames), zeros for those it lacks, and none after. Cross-correlation:
    out[b,o,t,y,x] = bias[o] + sum_{i,dt,dy,dx} w[o,i,dt,dy,dx] * xt[b,i,t+dt,y+dy-kh//2,x+dx-kw//2].
    A 4-D w [Co, Ci, kh, kw] is a conv2d (kt = 1). The result is rounded to the storage type."""
    if w.ndim == 4:
        w = w[:, :, None]
    B, Ci, T, H, W = x.shape
    Co, Ci2, kt, kh, kw = w.shape
    assert Ci == Ci2, (Ci, Ci2)
    tpad = 2 * (kt // 2)
    frames = []
    if tpad > 0:
        h = hist[:, :, max(0, hist.shape[2] - tpad):] if hist is not None else x[:, :, :0]
        frames.append(np.zeros((B, Ci, tpad - h.shape[2], H, W), x.dtype))
        frames.append(h.astype(x.dtype))
    frames.append(x)
    xt = np.concatenate(frames, axis=2)
    ph, pw = kh // 2, kw // 2
    xp = np.pad(xt, ((0, 0), (0, 0), (0, 0), (ph, ph), (pw, pw)))
    Tp, Hp, Wp = xp.shape[2:]
    tdt = torch.float64 if P.acc_t == np.float64 else torch.float32
    # channels last, in the accumulation type: [B, Tp, Hp, Wp, Ci] as rows of Ci values
    xl = _scratch("x", (B, Tp, Hp, Wp, Ci), tdt)
    xl.copy_(torch.from_numpy(np.ascontiguousarray(xp)).permute(0, 2, 3, 4, 1))
    xl = xl.view(-1, Ci)
    z = _scratch("z", (xl.shape[0], Co), tdt)
    zv = z.view(B, Tp, Hp, Wp, Co)
    acc = _scratch("acc", (B, T, H, W, Co), tdt).zero_()
    # the sum over taps: every padded input row times the tap's [Ci, Co] matrix, added to the
    # output at the tap's shift (output (t, y, x) takes padded row (t + dt, y + dy, x + dx))
    for dt in range(kt):
        for dy in range(kh):
            for dx in range(kw):
                wt = torch.from_numpy(np.ascontiguousarray(w[:, :, dt, dy, dx].T, dtype=P.acc_t))
                torch.mm(xl, wt, out=z)
                acc += zv[:, dt:dt + T, dy:dy + H, dx:dx + W]
    acc += torch.from_numpy(np.asarray(b, dtype=P.acc_t))
    out = torch.from_numpy(P.R(acc.numpy()))                  # rounded while contiguous
    return out.permute(0, 4, 1, 2, 3).contiguous().numpy()


def conv_points(xt, w, b, pts, acc_t=np.float64) -> np.ndarray:
    """Single outputs of the causal conv, one dot product each (the definition above, per
    element): xt is the already time-padded sequence [B, Ci, Tp, H, W] (zeros, history,
    chunk), pts an int array [n, 5] of (b, o, t, y, x). Returns float64 sums (unrounded)."""
    if w.ndim == 4:
        w = w[:, :, None]
    Co, Ci, kt, kh, kw = w.shape
    B, _, Tp, H, W = xt.shape
    out = np.empty(len(pts), np.float64)
    for n, (bb, o, t, y, x) in enumerate(np.asarray(pts)):
        patch = np.zeros((Ci, kt, kh, kw), acc_t)
        for dy in range(kh):
            yy = y + dy - kh // 2
            if not 0 <= yy < H:
                continue
            for dx in range(kw):
                xx = x + dx - kw // 2
                if 0 <= xx < W:
                    patch[:, :, dy, dx] = xt[bb, :, t:t + kt, yy, xx]
        out[n] = float(np.sum(patch * w[o].astype(acc_t), dtype=acc_t)) + float(b[o])
    return out


def cached_conv(x, w, b, name, cache, P: Prec) -> np.ndarray:
    """causal_conv of one chunk with history cache[name]; the cache becomes the last
    min(CACHE_T, |history| + |x|) frames of (history ++ x) ("Causal caches")."""
    hist = cache.get(name)
    seq = x if hist is None else np.concatenate([hist, x], axis=2)
    cache[name] = seq[:, :, max(0, seq.shape[2] - CACHE_T):].copy()
    return causal_conv(x, w, b, hist, P)


# ---------------------------------------------------------------- elementwise parts

def rms_norm(x, gamma, P: Prec) -> np.ndarray:
    """WanRMS_norm over channels (axis 1): x / max(||x||_2, 1e-12), times sqrt(C), times gamma.
    In fp32/bf16 the normalisation is computed and rounded first, then each product rounds
    again ("Precision": the norm normalises in fp32 and rounds before the products)."""
    C = x.shape[1]
    g = np.asarray(gamma).reshape((1, C) + (1,) * (x.ndim - 2))
    xd = x.astype(np.float64)
    n = np.sqrt(np.sum(xd * xd, axis=1, keepdims=True))
    xh = P.R(xd / np.maximum(n, 1e-12))
    y = P.R(xh.astype(np.float64) * P.scalar(math.sqrt(C)))
    return P.R(y.astype(np.float64) * g.astype(np.float64))


def silu(v, P: Prec) -> np.ndarray:
    """SiLU, v * sigmoid(v) = v / (1 + exp(-v)), rounded to the storage type."""
    vd = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return P.R(vd / (1.0 + np.exp(-vd)))


def dup_up(x, out_channels, ft, first) -> np.ndarray:
    """DupUp3D ("The parts"): factor ft in time, 2 in h and w, r = out*ft*4/in copies of each
    input channel: dup[c, ft*t+a, 2y+i, 2x+j] = x[(4*ft*c + 4a + 2i + j) // r, t, y, x].
    On the first chunk only the last of the ft time copies is kept. Pure copies."""
    B, Ci, T, H, W = x.shape
    r = out_channels * ft * 4 // Ci
    out = np.empty((B, out_channels, T * ft, 2 * H, 2 * W), x.dtype)
    c = np.arange(out_channels)
    for a in range(ft):
        for i in range(2):
            for j in range(2):
                out[:, :, a::ft, i::2, j::2] = x[:, (4 * ft * c + 4 * a + 2 * i + j) // r]
    return out[:, :, ft - 1:] if first else out


def unpatchify(x) -> np.ndarray:
    """[B, 12, F, h, w] -> [B, 3, F, 2h, 2w]: video[b,k,f,2y+i,2x+j] = x[b,4k+2j+i,f,y,x]
    ("What is computed", step 3). Pure copies."""
    B, C, F, H, W = x.shape
    K = C // (PATCH * PATCH)
    v = np.empty((B, K, F, PATCH * H, PATCH * W), x.dtype)
    for k in range(K):
        for i in range(PATCH):
            for j in range(PATCH):
                v[:, k, :, i::PATCH, j::PATCH] = x[:, PATCH * PATCH * k + PATCH * j + i]
    return v


def clamp(x) -> np.ndarray:
    """Clamp to [-1, 1]; NaN passes through (as torch.clamp does)."""
    return np.where(x < -1, -1, np.where(x > 1, 1, x)).astype(x.dtype)


# ---------------------------------------------------------------- blocks

def residual_block(x, Wt, name, cache, P: Prec) -> np.ndarray:
    """WanResidualBlock: x1 = conv1(SiLU(norm1(x))), x2 = conv2(SiLU(norm2(x1))), returns
    x2 + shortcut, the shortcut being x or a 1x1x1 conv of x ("The parts")."""
    if f"{name}.conv_shortcut.weight" in Wt:
        s = causal_conv(x, Wt[f"{name}.conv_shortcut.weight"], Wt[f"{name}.conv_shortcut.bias"], None, P)
    else:
        s = x
    h = silu(rms_norm(x, Wt[f"{name}.norm1.gamma"], P), P)
    h = cached_conv(h, Wt[f"{name}.conv1.weight"], Wt[f"{name}.conv1.bias"], f"{name}.conv1", cache, P)
    h = silu(rms_norm(h, Wt[f"{name}.norm2.gamma"], P), P)
    h = cached_conv(h, Wt[f"{name}.conv2.weight"], Wt[f"{name}.conv2.bias"], f"{name}.conv2", cache, P)
    return P.R(h.astype(np.float64) + s.astype(np.float64))


def attention(x, gamma, qkv_w, qkv_b, proj_w, proj_b, P: Prec) -> np.ndarray:
    """WanAttentionBlock ("The parts"), per frame: n = RMS norm of x; q, k, v are channels
    [0,C), [C,2C), [2C,3C) of a 1x1 conv C -> 3C of n; one head of softmax(q k^T/sqrt(C)) v
    over the h*w positions of the frame (the (N*T, H*W, 1, C) layout: positions are the
    sequence, channels the head dim), then a 1x1 conv C -> C, plus x."""
    B, C, T, H, W = x.shape
    S = H * W
    out = np.empty_like(x)
    wq = np.asarray(qkv_w).reshape(3 * C, C).astype(P.acc_t)
    wp = np.asarray(proj_w).reshape(C, C).astype(P.acc_t)
    scale = 1.0 / math.sqrt(C)
    for b in range(B):
        for t in range(T):
            frame = x[b, :, t]                                   # [C, H, W]
            n = rms_norm(frame[None], gamma, P)[0]               # [C, H, W]
            seq = n.reshape(C, S).T.astype(P.acc_t)              # [S, C], row-major (y, x)
            qkv = P.R(seq @ wq.T + np.asarray(qkv_b, P.acc_t))   # [S, 3C]
            q, k, v = (qkv[:, j * C:(j + 1) * C].astype(np.float64) for j in range(3))
            s = (q @ k.T) * scale
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o = P.R(p @ v)                                       # [S, C]
            y = P.R(o.astype(P.acc_t) @ wp.T + np.asarray(proj_b, P.acc_t))
            out[b, :, t] = P.R(y.T.reshape(C, H, W).astype(np.float64) + frame.astype(np.float64))
    return out


def attention_rows(frame, gamma, qkv_w, qkv_b, proj_w, proj_b, P: Prec, rows) -> np.ndarray:
    """The attention block of one frame [C, H, W] at the query positions ``rows`` (indices
    into the row-major H*W sequence): the same steps as ``attention``, with the scores and
    outputs computed only for those queries (every key and value is still used). Returns
    [len(rows), C]; for frames too large for the full score matrix."""
    C, H, W = frame.shape
    S = H * W
    rows = np.asarray(rows)
    wq = np.asarray(qkv_w).reshape(3 * C, C).astype(P.acc_t)
    wp = np.asarray(proj_w).reshape(C, C).astype(P.acc_t)
    bq = np.asarray(qkv_b, P.acc_t)
    n = rms_norm(frame[None], gamma, P)[0]
    seq = n.reshape(C, S).T.astype(P.acc_t)                              # [S, C]
    k = P.R(seq @ wq[C:2 * C].T + bq[C:2 * C]).astype(np.float64)
    v = P.R(seq @ wq[2 * C:].T + bq[2 * C:]).astype(np.float64)
    q = P.R(seq[rows] @ wq[:C].T + bq[:C]).astype(np.float64)
    s = (q @ k.T) * (1.0 / math.sqrt(C))
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    o = P.R(p @ v)
    y = P.R(o.astype(P.acc_t) @ wp.T + np.asarray(proj_b, P.acc_t))
    return P.R(y.astype(np.float64) + frame.reshape(C, S).T[rows].astype(np.float64))


def time_upsample(x, Wt, name, cache, P: Prec) -> np.ndarray:
    """upsample3d's time conv: a causal 3x1x1 conv C -> 2C whose output channel c becomes
    frame 2t and channel C + c frame 2t + 1 ("The parts": upsample3d)."""
    B, C, T, H, W = x.shape
    y = cached_conv(x, Wt[f"{name}.weight"], Wt[f"{name}.bias"], name, cache, P)
    out = np.empty((B, C, 2 * T, H, W), y.dtype)
    out[:, :, 0::2] = y[:, :C]
    out[:, :, 1::2] = y[:, C:]
    return out


def spatial_upsample(x, w, b, P: Prec) -> np.ndarray:
    """upsample2d: per frame, nearest x2 in h and w (value at (Y, X) is x at (Y//2, X//2):
    mode nearest-exact at an exact factor 2), then a 3x3 conv2d with zero padding 1."""
    u = np.repeat(np.repeat(x, 2, axis=3), 2, axis=4)
    return causal_conv(u, w, b, None, P)


def up_block(x, Wt, i, cache, first, P: Prec) -> np.ndarray:
    """An up block: 3 residual blocks; then in up blocks 0-2 the resampler (time conv only when
    temporal and not on the first chunk, then upsample2d) plus DupUp3D of the block's input."""
    base = Wt["decoder.conv_out.weight"].shape[1]
    ups = ((4 * base, True, True), (4 * base, True, True), (2 * base, False, True), (base, False, False))
    out_channels, temporal, spatial = ups[i]
    name = f"decoder.up_blocks.{i}"
    inp = x
    for j in range(RESNETS_PER_UP_BLOCK):
        x = residual_block(x, Wt, f"{name}.resnets.{j}", cache, P)
    if not spatial:
        return x
    if temporal and not first:
        x = time_upsample(x, Wt, f"{name}.upsampler.time_conv", cache, P)
    x = spatial_upsample(x, Wt[f"{name}.upsampler.resample.1.weight"], Wt[f"{name}.upsampler.resample.1.bias"], P)
    d = dup_up(inp, out_channels, 2 if temporal else 1, first)
    return P.R(x.astype(np.float64) + d.astype(np.float64))


def decode_chunk(x, Wt, cache, first, P: Prec, on_step=None) -> np.ndarray:
    """The decoder on one latent frame [B, 48, 1, h, w] -> [B, 12, 1 or 4, 8h, 8w].
    on_step(name), if given, is called after each block (progress reporting only)."""
    step = on_step or (lambda name: None)
    x = cached_conv(x, Wt["decoder.conv_in.weight"], Wt["decoder.conv_in.bias"], "decoder.conv_in", cache, P)
    x = residual_block(x, Wt, "decoder.mid_block.resnets.0", cache, P)
    a = "decoder.mid_block.attentions.0"
    x = attention(x, Wt[f"{a}.norm.gamma"], Wt[f"{a}.to_qkv.weight"], Wt[f"{a}.to_qkv.bias"],
                  Wt[f"{a}.proj.weight"], Wt[f"{a}.proj.bias"], P)
    x = residual_block(x, Wt, "decoder.mid_block.resnets.1", cache, P)
    step("mid_block")
    for i in range(4):
        x = up_block(x, Wt, i, cache, first, P)
        step(f"up_block {i}")
    x = silu(rms_norm(x, Wt["decoder.norm_out.gamma"], P), P)
    return cached_conv(x, Wt["decoder.conv_out.weight"], Wt["decoder.conv_out.bias"], "decoder.conv_out", cache, P)


def decode(z, weights, mode: str = "fp32", acc: str = "f64", on_chunk=None, on_step=None) -> np.ndarray:
    """decode(z [B, 48, T, h, w], weights) -> video [B, 3, 4T-3, 16h, 16w] in [-1, 1].
    Only names under the decoder's prefixes are used; they and z are rounded to the mode's
    type; post_quant_conv runs over all T frames, then the chunk loop, concatenation along
    time, unpatchify and clamp ("What is computed")."""
    P = Prec(mode, acc)
    Wt = {k: P.R(v) for k, v in weights.items() if k.startswith(PREFIXES)}
    x = causal_conv(P.R(z), Wt["post_quant_conv.weight"], Wt["post_quant_conv.bias"], None, P)
    cache: dict = {}
    chunks = []
    for i in range(x.shape[2]):
        chunks.append(decode_chunk(x[:, :, i:i + 1], Wt, cache, i == 0, P,
                                   None if on_step is None else (lambda name, i=i: on_step(i, name))))
        if on_chunk is not None:
            on_chunk(i)
    return clamp(unpatchify(np.concatenate(chunks, axis=2)))


def psnr(a, b) -> float:
    """PSNR of two videos in [-1, 1]: 10 log10(1 / mean(((a - b) / 2)^2)) (the comparison
    script on MaxDiffusion PR #514's page)."""
    d = (np.asarray(a, np.float64) - np.asarray(b, np.float64)) / 2.0
    m = float(np.mean(d * d))
    return float("inf") if m == 0 else 10.0 * math.log10(1.0 / m)
