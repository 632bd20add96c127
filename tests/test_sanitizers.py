"""Host-side AddressSanitizer + UBSan runs (no GPU).

1. The fp64 oracle, built with gcc under both sanitizers, driven by
   tests/sanitize/oracle_driver.c over small and degenerate shapes.
2. libconv2d.so's host code -- argument validation, output sizes, the tile
   plans behind every kernel's support check and the path choice -- rebuilt
   with both sanitizers on the host side only.  The device code is not
   rebuilt: each object's GPU binary is taken from the regular build under
   _build/ and embedded into the sanitized host compile.  Driven by
   tests/sanitize/dispatch_driver.cpp over valid, invalid and extreme
   arguments; it calls host-only entry points, so nothing touches a GPU.

Any report aborts the driver (halt on error), which fails the test.
"""
import glob
import os
import shutil
import subprocess

import pytest

from helpers import ROOT, ensure_built

OUT = os.path.join(ROOT, "_build", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{err[-3000:]}"
    return r.stdout


def test_oracle_under_asan_ubsan():
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run([gcc, "-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "conv2d_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"])
    out = _run([exe], env=SAN_ENV, timeout=600)
    assert "oracle sanitize ok" in out


def test_dispatcher_host_code_under_asan_ubsan():
    ensure_built()
    import importlib.util
    spec = importlib.util.spec_from_file_location("conv2d_build", os.path.join(ROOT, "cnn_convolution_conv2d_amd",
                                                                                "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    hipcc = b.hipcc()
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
    objcopy, clangxx = os.path.join(llvm, "llvm-objcopy"), os.path.join(llvm, "clang++")
    if not (os.path.exists(objcopy) and os.path.exists(clangxx)):
        pytest.skip("ROCm llvm tools not found")
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
           "-fno-sanitize-recover=all"]
    objs = []
    for src in sorted(glob.glob(os.path.join(b.CSRC, "*.hip"))):
        name = os.path.basename(src)
        fatbin = os.path.join(OUT, name + ".hipfb")
        obj = os.path.join(OUT, name + ".o")
        _run([objcopy, "--dump-section=.hip_fatbin=" + fatbin, os.path.join(b.BUILD_DIR, name + ".o")])
        _run([hipcc, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, "-c", src,
              "-o", obj, "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")] + san)
        objs.append(obj)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    drv = os.path.join(OUT, "dispatch_driver.o")
    _run([clangxx, "-c", os.path.join(ROOT, "tests", "sanitize", "dispatch_driver.cpp"), "-o", drv, "-O1", "-g",
          "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
          os.path.join(rocm, "include"), "-fsanitize=address,undefined"])
    exe = os.path.join(OUT, "dispatch_driver")
    _run([clangxx, "-o", exe, drv] + objs + ["-fsanitize=address,undefined", "-L", os.path.join(rocm, "lib"),
                                             "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")])
    out = _run([exe], env=SAN_ENV, timeout=600)
    assert "dispatch sanitize ok" in out
