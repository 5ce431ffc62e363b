"""ctypes binding of libwanvae.so (include/wanvae.h).

Argument marshalling only: every step of the decoder runs in the library's HIP kernels.
torch provides device memory (outputs, workspaces) and the current HIP stream. The
library must be built (``python -m video_vae_decoding_amd.build``); loading fails loudly
when it is missing.

Status codes map to exceptions as FastVideo's "wan22_vae_decode reference.py" page raises
them: a bad dtype is a ValueError, a missing parameter a KeyError.
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
        L.wanvae_causal_conv3d_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
        L.wanvae_causal_conv3d.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, T, T, i32, i32, vp, vp, sz, vp]
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
        L.wanvae_decode_tiled_workspace_size.argtypes = [i64, i64, i64, i64, T, i64, i32, i32, i32, i32, i32,
                                                         ctypes.POINTER(sz)]
        L.wanvae_decode_tiled.argtypes = [vp, i32, i64, i64, i64, i64, T, i64, i32, i32, i32, i32, i32, vp, vp, sz, vp]
        for f in ("wanvae_decode_workspace_size", "wanvae_decode", "wanvae_causal_conv3d_workspace_size",
                  "wanvae_causal_conv3d", "wanvae_attn_block_workspace_size", "wanvae_attn_block", "wanvae_version",
                  "wanvae_profile_enable", "wanvae_profile_read", "wanvae_set_conv_kernel",
                  "wanvae_set_decode_pipeline", "wanvae_decode_tiled_workspace_size", "wanvae_decode_tiled"):
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


def tensor_struct(name: str | None, t: torch.Tensor) -> wanvae_tensor:
    if t.dim() > 5:
        raise ValueError(f"{name}: more than 5 dimensions")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    shape = (ctypes.c_int64 * 5)(*list(t.shape), *([0] * (5 - t.dim())))
    return wanvae_tensor(name.encode() if name is not None else None, t.data_ptr(), dtype_code(t.dtype), t.dim(), shape)


def tensor_table(weights: Mapping[str, torch.Tensor]):
    items = [(k, v) for k, v in weights.items() if k.startswith(("decoder.", "post_quant_conv."))]
    arr = (wanvae_tensor * max(1, len(items)))()
    for i, (k, v) in enumerate(items):
        arr[i] = tensor_struct(k, v)
    return arr, len(items)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


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
    if z.dim() != 5:
        raise ValueError(f"z must be [B, 48, T, h, w], got {tuple(z.shape)}")
    B, C, T, h, w = z.shape
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
    if z.dim() != 5:
        raise ValueError(f"z must be [B, 48, T, h, w], got {tuple(z.shape)}")
    B, C, T, h, w = z.shape
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


def conv_workspace_size(B, Cin, Cout, t, h, w, n_cache, layout, dtype) -> int:
    out = ctypes.c_size_t(0)
    check(lib().wanvae_causal_conv3d_workspace_size(B, Cin, Cout, t, h, w, n_cache, _LAYOUTS[layout], dtype_code(dtype),
                                                    ctypes.byref(out)))
    return out.value


def wanvae_causal_conv3d(x: torch.Tensor, cache: torch.Tensor | None, weight: torch.Tensor, bias: torch.Tensor,
                         layout: str = "ncthw", y: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One causal conv of chunk x with ``cache`` frames of history; compute type = x.dtype."""
    dtype = x.dtype
    if layout == "ncthw":
        B, Cin, t, h, w = x.shape
        n_cache = 0 if cache is None else cache.shape[2]
        yshape = (B, weight.shape[0], t, h, w)
    else:
        B, t, h, w, Cin = x.shape
        n_cache = 0 if cache is None else cache.shape[1]
        yshape = (B, t, h, w, weight.shape[0])
    if y is None:
        y = torch.empty(yshape, dtype=dtype, device=x.device)
    need = conv_workspace_size(B, Cin, weight.shape[0], t, h, w, n_cache, layout, dtype)
    ws = _workspace(need, x.device, workspace)
    W, Bt = tensor_struct("weight", weight), tensor_struct("bias", bias)
    cache_ptr = None if cache is None else cache.data_ptr()
    check(lib().wanvae_causal_conv3d(x.data_ptr(), cache_ptr, B, Cin, t, h, w, n_cache, ctypes.byref(W),
                                     ctypes.byref(Bt), _LAYOUTS[layout], dtype_code(dtype), y.data_ptr(),
                                     ws.data_ptr(), need, _stream(x.device)))
    return y


causal_conv3d = wanvae_causal_conv3d


def attn_workspace_size(B, C, T, h, w, layout, dtype) -> int:
    out = ctypes.c_size_t(0)
    check(lib().wanvae_attn_block_workspace_size(B, C, T, h, w, _LAYOUTS[layout], dtype_code(dtype), ctypes.byref(out)))
    return out.value


def wanvae_attn_block(x: torch.Tensor, gamma, qkv_w, qkv_b, proj_w, proj_b, layout: str = "ncthw",
                      y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The mid-block attention block on x; compute type = x.dtype."""
    dtype = x.dtype
    if layout == "ncthw":
        B, C, T, h, w = x.shape
    else:
        B, T, h, w, C = x.shape
    if y is None:
        y = torch.empty_like(x)
    need = attn_workspace_size(B, C, T, h, w, layout, dtype)
    ws = _workspace(need, x.device, workspace)
    ts = [tensor_struct(n, t) for n, t in
          (("gamma", gamma), ("qkv_w", qkv_w), ("qkv_b", qkv_b), ("proj_w", proj_w), ("proj_b", proj_b))]
    check(lib().wanvae_attn_block(x.data_ptr(), _LAYOUTS[layout], B, C, T, h, w, *[ctypes.byref(t) for t in ts],
                                  dtype_code(dtype), y.data_ptr(), ws.data_ptr(), need, _stream(x.device)))
    return y


attn_block = wanvae_attn_block


CONV_KERNELS = 14


def wanvae_set_conv_kernel(kernel: int) -> None:
    """Use conv kernel ``kernel`` wherever it can run a conv (-1: each conv's default)."""
    check(lib().wanvae_set_conv_kernel(kernel))


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
