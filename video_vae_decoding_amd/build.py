"""Builds libwanvae.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python -m video_vae_decoding_amd.build      # or: python video_vae_decoding_amd/build.py

Every HIP source is compiled with packed fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwanvae.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("WANVAE_ARCH", "gfx950")
SOURCES = ["kernels.hip", "tiles.hip", "wanvae.cpp", "noalloc.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compiles the sources and links libwanvae.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="wanvae_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(len(cmds)) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = LIB + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
