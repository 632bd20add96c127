"""Build libconv2d.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m cnn_convolution_conv2d_amd.build

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` at the
repository root, in parallel, then linked into
``cnn_convolution_conv2d_amd/libconv2d.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libconv2d.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("CONV2D_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libconv2d.so)")


# Packed fp32 VALU ops are disabled for every device pass; -O3 would otherwise
# form them from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
            "-Wno-unused-function", "-I", os.path.join(ROOT, "include")] + DEVICE_FLAGS


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj] + compile_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libconv2d.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def sources() -> list[str]:
    """Every file the library is built from: the HIP sources, their headers and
    the public header."""
    pats = ("*.hip", "*.hpp", "*.h")
    found = [p for pat in pats for p in glob.glob(os.path.join(CSRC, pat))]
    found += glob.glob(os.path.join(ROOT, "include", "*.h"))
    found.append(os.path.abspath(__file__))
    return sorted(found)


def stale() -> bool:
    """True when libconv2d.so is missing or older than any file it is built from."""
    if not os.path.exists(OUT):
        return True
    built = os.path.getmtime(OUT)
    return any(os.path.getmtime(p) > built for p in sources())


def ensure_built(verbose: bool = False) -> str:
    """Build libconv2d.so if it is missing or stale; returns its path."""
    if stale():
        build(verbose=verbose)
    return OUT


if __name__ == "__main__":
    build()
