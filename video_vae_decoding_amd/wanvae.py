"""ctypes binding of libwanvae.so (include/wanvae.h).

Argument marshalling only: every step of the decoder runs in the library's HIP kernels.
torch provides device memory (outputs, workspaces) and the current HIP stream. The
library must be built (``python -m video_vae_decoding_amd.build``); loading fails loudly
when it is missing.

Status codes map to exceptions as FastVideo's "wan22_vae_decode reference.py" page raises
them: a bad dtype is a ValueError, a missing parameter a KeyError.

Before any library call every tensor is checked: inputs (z, x, cache, weights) must live on one
CUDA device, with the element types and ranks the call takes (x and cache are made contiguous,
weights must be); outputs (video, y, cache_out) and a given workspace must be contiguous tensors
of exactly the shape and element type the call writes, on that device. A tensor that fails is a
ValueError, so the kernels never see a host pointer or a buffer smaller than they address.
"""
from __future__ import annotations

import ctypes
import os
from typing import Mapping

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwanvae.so")

F32, BF16 = 0, 1
NCTHW, NTHWC = 0, 1
OK, EDTYPE, EMISSING, ESHAPE, ETOPOLOGY, EWORKSPACE, EHIP, EARG = 0, -1, -2, -3, -4, -5, -6, -7

KCONV, KNORM, KATTN, KOTHER = 0, 1, 2, 3
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
_LAYOUTS = {"ncthw": NCTHW, "nthwc": NTHWC}


class wanvae_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 5)]


class WanVAEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m video_vae_decoding_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        T = ctypes.POINTER(wanvae_tensor)
        L.wanvae_decode_workspace_size.argtypes = [i64, i64, i64, i64, T, i64, i32, ctypes.POINTER(sz)]
        L.wanvae_decode.argtypes = [vp, i32, i64, i64, i64, i64, T, i64, i32, vp, vp, sz, vp]
        L.wanvae_causal_conv3d_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64, i32, i32, i32,
                                                          ctypes.POINTER(sz)]
        L.wanvae_causal_conv3d.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, T, T, i32, i32, vp, i32, vp, vp, sz,
                                           vp]
        L.wanvae_causal_conv3d_noalloc.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, T, T, i32, i32, vp, i32, vp,
                                                   vp]
        L.wanvae_attn_block_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
        L.wanvae_attn_block.argtypes = [vp, i32, i64, i64, i64, i64, i64, T, T, T, T, T, i32, vp, vp, sz, vp]
        L.wanvae_profile_enable.argtypes = [ctypes.c_int]
        L.wanvae_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.wanvae_last_error.restype = ctypes.c_char_p
        L.wanvae_last_error.argtypes = []
        L.wanvae_version.argtypes = []
        L.wanvae_set_conv_kernel.argtypes = [ctypes.c_int]
        L.wanvae_set_decode_pipeline.argtypes = [ctypes.c_int]
        L.wanvae_set_norm_kernel.argtypes = [ctypes.c_int]
        L.wanvae_decode_tiled_workspace_size.argtypes = [i64, i64, i64, i64, T, i64, i32, i32, i32, i32, i32,
                                                         ctypes.POINTER(sz)]
        L.wanvae_decode_tiled.argtypes = [vp, i32, i64, i64, i64, i64, T, i64, i32, i32, i32, i32, i32, vp, vp, sz, vp]
        for f in ("wanvae_decode_workspace_size", "wanvae_decode", "wanvae_causal_conv3d_workspace_size",
                  "wanvae_causal_conv3d", "wanvae_causal_conv3d_noalloc", "wanvae_attn_block_workspace_size", "wanvae_attn_block", "wanvae_version",
                  "wanvae_profile_enable", "wanvae_profile_read", "wanvae_set_conv_kernel",
                  "wanvae_set_decode_pipeline", "wanvae_set_norm_kernel", "wanvae_decode_tiled_workspace_size",
                  "wanvae_decode_tiled"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def check(code: int) -> None:
    if code == OK:
        return
    msg = lib().wanvae_last_error().decode()
    if code == EDTYPE:
        raise ValueError(msg)
    if code == EMISSING:
        raise KeyError(msg)
    if code in (ESHAPE, ETOPOLOGY, EARG, EWORKSPACE):
        raise ValueError(f"[{code}] {msg}")
    raise WanVAEError(code, msg)


def dtype_code(dtype) -> int:
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be torch.float32 or torch.bfloat16, not {dtype}")
    return _DTYPES[dtype]


def _on(t: torch.Tensor, name: str, device: torch.device) -> None:
    """t must be a tensor on ``device`` (a CUDA device)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
    if device.type != "cuda":
        raise ValueError(f"{name} must be on a CUDA device, not {device}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _device_of(t: torch.Tensor, name: str) -> torch.device:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
    d = t.device
    if d.type == "cuda" and d.index is None:
        d = torch.device("cuda", torch.cuda.current_device())
    return d


def _output(t: torch.Tensor, name: str, shape, dtype) -> None:
    """A caller-given output: exactly ``shape`` and ``dtype``, contiguous."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, the call writes {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has element type {t.dtype}, the call writes {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def tensor_struct(name: str | None, t: torch.Tensor) -> wanvae_tensor:
    if t.dim() > 5:
        raise ValueError(f"{name}: more than 5 dimensions")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    shape = (ctypes.c_int64 * 5)(*list(t.shape), *([0] * (5 - t.dim())))
    return wanvae_tensor(name.encode() if name is not None else None, t.data_ptr(), dtype_code(t.dtype), t.dim(), shape)


def _weight_items(weights: Mapping[str, torch.Tensor]):
    return [(k, v) for k, v in weights.items() if k.startswith(("decoder.", "post_quant_conv."))]


def check_weights(weights: Mapping[str, torch.Tensor], device: torch.device | None = None) -> None:
    """Every parameter the decoder reads: a contiguous float32 / bfloat16 tensor of at most
    5 dimensions, on ``device`` when one is given."""
    for k, v in _weight_items(weights):
        if not isinstance(v, torch.Tensor):
            raise ValueError(f"{k} must be a torch.Tensor, not {type(v).__name__}")
        dtype_code(v.dtype)
        if v.dim() > 5:
            raise ValueError(f"{k}: more than 5 dimensions")
        if not v.is_contiguous():
            raise ValueError(f"{k}: not contiguous")
        if device is not None:
            _on(v, k, device)


def tensor_table(weights: Mapping[str, torch.Tensor]):
    items = _weight_items(weights)
    arr = (wanvae_tensor * max(1, len(items)))()
    for i, (k, v) in enumerate(items):
        arr[i] = tensor_struct(k, v)
    return arr, len(items)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_workspace(workspace: torch.Tensor | None, device) -> None:
    if workspace is None:
        return
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous torch.Tensor")
    _on(workspace, "workspace", device)


def _workspace(nbytes: int, device, workspace: torch.Tensor | None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def decode_workspace_size(B, T, h, w, weights: Mapping[str, torch.Tensor], dtype=torch.float32) -> int:
    arr, n = tensor_table(weights)
    out = ctypes.c_size_t(0)
    check(lib().wanvae_decode_workspace_size(B, T, h, w, arr, n, dtype_code(dtype), ctypes.byref(out)))
    return out.value


def wanvae_decode(z: torch.Tensor, weights: Mapping[str, torch.Tensor], dtype=torch.float32,
                  video: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode(z [B, 48, T, h, w], weights) -> video [B, 3, 4T-3, 16h, 16w] of ``dtype`` on z's device."""
    dt = dtype_code(dtype)
    B, T, h, w = _check_decode_args(z, weights, dtype, video, workspace)
    z = z.contiguous()
    arr, n = tensor_table(weights)
    need = decode_workspace_size(B, T, h, w, weights, dtype)
    if video is None:
        video = torch.empty((B, 3, 4 * T - 3, 16 * h, 16 * w), dtype=dtype, device=z.device)
    ws = _workspace(need, z.device, workspace)
    check(lib().wanvae_decode(z.data_ptr(), dtype_code(z.dtype), B, T, h, w, arr, n, dt, video.data_ptr(),
                              ws.data_ptr(), need, _stream(z.device)))
    return video


decode = wanvae_decode


def _check_decode_args(z, weights, dtype, video, workspace):
    """The decode's tensors, before any library call: z [B, 48, T, h, w] of float32 / bfloat16,
    the weights, a given video [B, 3, 4T-3, 16h, 16w] of ``dtype``, all on z's CUDA device."""
    device = _device_of(z, "z")
    if z.dim() != 5 or z.shape[1] != 48:
        raise ValueError(f"z must be [B, 48, T, h, w], got {tuple(z.shape)}")
    dtype_code(z.dtype)
    B, _, T, h, w = z.shape
    if video is not None:
        _output(video, "video", (B, 3, 4 * T - 3, 16 * h, 16 * w), dtype)
    check_weights(weights)
    _on(z, "z", device)
    check_weights(weights, device)
    if video is not None:
        _on(video, "video", device)
    _check_workspace(workspace, device)
    return B, T, h, w


def decode_tiled_workspace_size(B, T, h, w, weights: Mapping[str, torch.Tensor], dtype=torch.float32,
                                tile=(256, 256), stride=(192, 192)) -> int:
    arr, n = tensor_table(weights)
    out = ctypes.c_size_t(0)
    check(lib().wanvae_decode_tiled_workspace_size(B, T, h, w, arr, n, dtype_code(dtype), tile[0], tile[1], stride[0],
                                                   stride[1], ctypes.byref(out)))
    return out.value


def wanvae_decode_tiled(z: torch.Tensor, weights: Mapping[str, torch.Tensor], dtype=torch.float32,
                        tile=(256, 256), stride=(192, 192), video: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The spatially tiled decode: overlapping tiles of tile[0] x tile[1] video pixels every
    stride[0] x stride[1], each decoded on its own, blended where they overlap."""
    dt = dtype_code(dtype)
    B, T, h, w = _check_decode_args(z, weights, dtype, video, workspace)
    z = z.contiguous()
    arr, n = tensor_table(weights)
    need = decode_tiled_workspace_size(B, T, h, w, weights, dtype, tile, stride)
    if video is None:
        video = torch.empty((B, 3, 4 * T - 3, 16 * h, 16 * w), dtype=dtype, device=z.device)
    ws = _workspace(need, z.device, workspace)
    check(lib().wanvae_decode_tiled(z.data_ptr(), dtype_code(z.dtype), B, T, h, w, arr, n, dt, tile[0], tile[1],
                                    stride[0], stride[1], video.data_ptr(), ws.data_ptr(), need, _stream(z.device)))
    return video


decode_tiled = wanvae_decode_tiled


def conv_workspace_size(B, Cin, Cout, t, h, w, n_cache, layout, dtype, y_dtype=None) -> int:
    out = ctypes.c_size_t(0)
    y_dtype = dtype if y_dtype is None else y_dtype
    check(lib().wanvae_causal_conv3d_workspace_size(B, Cin, Cout, t, h, w, n_cache, _LAYOUTS[layout], dtype_code(dtype),
                                                    dtype_code(y_dtype), ctypes.byref(out)))
    return out.value


def wanvae_causal_conv3d(x: torch.Tensor, cache: torch.Tensor | None, weight: torch.Tensor, bias: torch.Tensor,
                         layout: str = "ncthw", y: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, y_dtype=None,
                         cache_out: torch.Tensor | None = None, return_cache: bool = False):
    """One causal conv of chunk x with ``cache`` frames of history; compute type = x.dtype.

    ``y_dtype`` (default x.dtype) is the output's element type: torch.float32 with a bfloat16
    x stores the float32 sums unrounded. ``cache_out`` (or, with ``return_cache``, a new tensor)
    receives the updated cache, the last min(2, n_cache + t) frames of cache ++ x; it may be
    ``cache`` itself when that holds 2 frames. Returns y, or (y, cache_out) with
    ``return_cache``."""
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}, not {layout!r}")
    device = _device_of(x, "x")
    dtype = x.dtype
    dtype_code(dtype)
    y_dtype = dtype if y_dtype is None else y_dtype
    dtype_code(y_dtype)
    if x.dim() != 5:
        raise ValueError(f"x must have 5 dimensions, got {tuple(x.shape)}")
    if not isinstance(weight, torch.Tensor) or weight.dim() != 5:
        raise ValueError("weight must be a [Cout, Cin, kt, kh, kw] tensor")
    Cout = weight.shape[0]
    if layout == "ncthw":
        B, Cin, t, h, w = x.shape
        tax = 2
    else:
        B, t, h, w, Cin = x.shape
        tax = 1
    n_cache = 0
    if cache is not None:
        if not isinstance(cache, torch.Tensor) or cache.dim() != 5 or cache.dtype != dtype:
            raise ValueError("cache must be a 5-D tensor of x's element type")
        n_cache = cache.shape[tax]
        want = list(x.shape)
        want[tax] = n_cache
        if list(cache.shape) != want:
            raise ValueError(f"cache has shape {tuple(cache.shape)}; with x {tuple(x.shape)} it must be {tuple(want)}")
    yshape = (B, Cout, t, h, w) if layout == "ncthw" else (B, t, h, w, Cout)
    if y is not None:
        _output(y, "y", yshape, y_dtype)
    n_out = min(2, n_cache + t)
    cshape = list(x.shape)
    cshape[tax] = n_out
    if cache_out is not None:
        _output(cache_out, "cache_out", tuple(cshape), dtype)
    for nm, tt in (("weight", weight), ("bias", bias)):
        if not isinstance(tt, torch.Tensor) or not tt.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous tensor")
        dtype_code(tt.dtype)
    _on(x, "x", device)
    for nm, tt in (("cache", cache), ("weight", weight), ("bias", bias), ("y", y), ("cache_out", cache_out)):
        if tt is not None:
            _on(tt, nm, device)
    _check_workspace(workspace, device)
    x = x.contiguous()
    if cache is not None:
        cache = cache if cache_out is not None and cache_out.data_ptr() == cache.data_ptr() else cache.contiguous()
    if y is None:
        y = torch.empty(yshape, dtype=y_dtype, device=device)
    if cache_out is None and return_cache:
        cache_out = torch.empty(tuple(cshape), dtype=dtype, device=device)
    need = conv_workspace_size(B, Cin, Cout, t, h, w, n_cache, layout, dtype, y_dtype)
    ws = _workspace(need, device, workspace)
    W, Bt = tensor_struct("weight", weight), tensor_struct("bias", bias)
    cache_ptr = None if cache is None else cache.data_ptr()
    co_ptr = None if cache_out is None else cache_out.data_ptr()
    check(lib().wanvae_causal_conv3d(x.data_ptr(), cache_ptr, B, Cin, t, h, w, n_cache, ctypes.byref(W),
                                     ctypes.byref(Bt), _LAYOUTS[layout], dtype_code(dtype), y.data_ptr(),
                                     dtype_code(y_dtype), co_ptr, ws.data_ptr(), need, _stream(device)))
    return (y, cache_out) if return_cache else y


causal_conv3d = wanvae_causal_conv3d


def wanvae_causal_conv3d_noalloc(x: torch.Tensor, cache: torch.Tensor | None, weight: torch.Tensor,
                                 bias: torch.Tensor, y: torch.Tensor, layout: str = "ncthw",
                                 cache_out: torch.Tensor | None = None) -> torch.Tensor:
    """wanvae_causal_conv3d on the library's fixed scratch (no device allocation, neither here
    nor in the library): x, cache, weight and bias must be contiguous, and y (of the element
    type it is to hold) and cache_out are given by the caller. Returns y."""
    if not isinstance(y, torch.Tensor):
        raise ValueError("y must be given: this entry point allocates nothing")
    for nm, tt in (("x", x), ("cache", cache)):
        if tt is not None and (not isinstance(tt, torch.Tensor) or not tt.is_contiguous()):
            raise ValueError(f"{nm} must be a contiguous tensor (it is not copied here)")
    device = _device_of(x, "x")
    dtype = x.dtype
    dtype_code(dtype)
    if x.dim() != 5 or not isinstance(weight, torch.Tensor) or weight.dim() != 5:
        raise ValueError("x must be 5-D and weight [Cout, Cin, kt, kh, kw]")
    tax = 2 if layout == "ncthw" else 1
    if layout == "ncthw":
        B, Cin, t, h, w = x.shape
    elif layout == "nthwc":
        B, t, h, w, Cin = x.shape
    else:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}, not {layout!r}")
    n_cache = 0
    if cache is not None:
        want = list(x.shape)
        want[tax] = cache.shape[tax]
        if cache.dim() != 5 or list(cache.shape) != want or cache.dtype != dtype:
            raise ValueError(f"cache {tuple(cache.shape)} {cache.dtype} does not match x {tuple(x.shape)} {dtype}")
        n_cache = cache.shape[tax]
    Cout = weight.shape[0]
    _output(y, "y", (B, Cout, t, h, w) if layout == "ncthw" else (B, t, h, w, Cout), y.dtype)
    dtype_code(y.dtype)
    if cache_out is not None:
        cshape = list(x.shape)
        cshape[tax] = min(2, n_cache + t)
        _output(cache_out, "cache_out", tuple(cshape), dtype)
    for nm, tt in (("weight", weight), ("bias", bias)):
        if not isinstance(tt, torch.Tensor) or not tt.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous tensor")
        dtype_code(tt.dtype)
    for nm, tt in (("x", x), ("cache", cache), ("weight", weight), ("bias", bias), ("y", y), ("cache_out", cache_out)):
        if tt is not None:
            _on(tt, nm, device)
    W, Bt = tensor_struct("weight", weight), tensor_struct("bias", bias)
    check(lib().wanvae_causal_conv3d_noalloc(x.data_ptr(), None if cache is None else cache.data_ptr(), B, Cin, t, h, w,
                                             n_cache, ctypes.byref(W), ctypes.byref(Bt), _LAYOUTS[layout],
                                             dtype_code(dtype), y.data_ptr(), dtype_code(y.dtype),
                                             None if cache_out is None else cache_out.data_ptr(), _stream(device)))
    return y


def attn_workspace_size(B, C, T, h, w, layout, dtype) -> int:
    out = ctypes.c_size_t(0)
    check(lib().wanvae_attn_block_workspace_size(B, C, T, h, w, _LAYOUTS[layout], dtype_code(dtype), ctypes.byref(out)))
    return out.value


def wanvae_attn_block(x: torch.Tensor, gamma, qkv_w, qkv_b, proj_w, proj_b, layout: str = "ncthw",
                      y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The mid-block attention block on x; compute type = x.dtype."""
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}, not {layout!r}")
    device = _device_of(x, "x")
    dtype = x.dtype
    dtype_code(dtype)
    if x.dim() != 5:
        raise ValueError(f"x must have 5 dimensions, got {tuple(x.shape)}")
    if layout == "ncthw":
        B, C, T, h, w = x.shape
    else:
        B, T, h, w, C = x.shape
    if y is not None:
        _output(y, "y", tuple(x.shape), dtype)
    params = (("gamma", gamma), ("qkv_w", qkv_w), ("qkv_b", qkv_b), ("proj_w", proj_w), ("proj_b", proj_b))
    for nm, tt in params:
        if not isinstance(tt, torch.Tensor) or not tt.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous tensor")
        dtype_code(tt.dtype)
    _on(x, "x", device)
    for nm, tt in params + (("y", y),):
        if tt is not None:
            _on(tt, nm, device)
    _check_workspace(workspace, device)
    x = x.contiguous()
    if y is None:
        y = torch.empty_like(x)
    need = attn_workspace_size(B, C, T, h, w, layout, dtype)
    ws = _workspace(need, device, workspace)
    ts = [tensor_struct(n, t) for n, t in
          (("gamma", gamma), ("qkv_w", qkv_w), ("qkv_b", qkv_b), ("proj_w", proj_w), ("proj_b", proj_b))]
    check(lib().wanvae_attn_block(x.data_ptr(), _LAYOUTS[layout], B, C, T, h, w, *[ctypes.byref(t) for t in ts],
                                  dtype_code(dtype), y.data_ptr(), ws.data_ptr(), need, _stream(device)))
    return y


attn_block = wanvae_attn_block


CONV_KERNELS = 14


def wanvae_set_conv_kernel(kernel: int) -> None:
    """Use conv kernel ``kernel`` wherever it can run a conv (-1: each conv's default)."""
    check(lib().wanvae_set_conv_kernel(kernel))


def wanvae_set_norm_kernel(mode: int) -> None:
    """bf16 SiLU after the RMS norm: from the LDS table on large launches (-1, the default),
    arithmetic only (0) or the table on every launch (1). The results are the same bits."""
    check(lib().wanvae_set_norm_kernel(mode))


def wanvae_set_decode_pipeline(on: bool) -> None:
    """Overlap each latent frame's low-level stage with the previous frame's high levels
    on two streams (True, the default) or run the decode in chunk order on the caller's
    stream (False). The video is bit-identical either way."""
    check(lib().wanvae_set_decode_pipeline(1 if on else 0))


def wanvae_profile_enable(on: bool = True) -> None:
    """Start (clearing earlier records) or stop timing every kernel the library enqueues."""
    check(lib().wanvae_profile_enable(1 if on else 0))


def wanvae_profile_read(kind: int) -> dict:
    """Summed event time (ms), launches, FLOPs and bytes of one kernel kind (KCONV, ...)."""
    ms, n, fl, by = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    check(lib().wanvae_profile_read(kind, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl), ctypes.byref(by)))
    return {"ms": ms.value, "launches": n.value, "flops": fl.value, "bytes": by.value}
