"""fp64 CPU oracle for the 2D convolution forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and never imports it; the GPU library never imports this.

The arithmetic lives in ``conv2d_oracle.c`` (plain C, fp64, the loop nest of
the definition); this module builds it with gcc, loads it with ctypes and adds
the explicit im2col x GEMM lowering used by the oracle's self-tests
(page "How a GPU executes NN convolution", lincklin.cn, section 7: the
convolution is W_matrix [Cout x Cin*Kh*Kw] times X_matrix [Cin*Kh*Kw x N*Ho*Wo];
"lpnh.cn/news/2674933" section 4.3: a grouped convolution is G such products
on contiguous channel blocks).

Arrays are NCHW activations, [Cout][Cin/G][Kh][Kw] weights, fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv2d_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_libs = {}


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle (default ``oracle/liboracle.so``) with gcc -O2 -fopenmp."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load_library(path: str | None = None):
    """ctypes handle of the oracle library (the default one, built on demand,
    or another build of the same source given by ``path``)."""
    key = path or _LIB
    if key in _libs:
        return _libs[key]
    if path is None and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(key)
    L, P = ctypes.c_long, ctypes.c_void_p
    lib.oracle_out_dim.restype = L
    lib.oracle_out_dim.argtypes = [L] * 5
    lib.oracle_conv2d_f64.restype = ctypes.c_int
    lib.oracle_conv2d_f64.argtypes = [P, P, P, ctypes.c_int, P, P] + [L] * 11
    lib.oracle_conv2d_points_f64.restype = ctypes.c_int
    lib.oracle_conv2d_points_f64.argtypes = [P, P, P, ctypes.c_int, P, L, P, P] + [L] * 11
    lib.oracle_im2col_f64.restype = ctypes.c_int
    lib.oracle_im2col_f64.argtypes = [P, P] + [L] * 9
    lib.oracle_transpose_out_dim.restype = L
    lib.oracle_transpose_out_dim.argtypes = [L] * 6
    lib.oracle_conv_transpose2d_f64.restype = ctypes.c_int
    lib.oracle_conv_transpose2d_f64.argtypes = [P, P, P, ctypes.c_int, P, P] + [L] * 12
    lib.oracle_conv_transpose2d_points_f64.restype = ctypes.c_int
    lib.oracle_conv_transpose2d_points_f64.argtypes = [P, P, P, ctypes.c_int, P, L, P, P] + [L] * 12
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _libs[key] = lib
    return lib


def _load(lib=None):
    return lib if lib is not None else load_library()


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def out_dim(size: int, k: int, stride: int = 1, pad: int = 0, dilation: int = 1, lib=None) -> int:
    """floor((size + 2*pad - dilation*(k-1) - 1)/stride) + 1 (lpnh.cn section 6.2)."""
    return int(_load(lib).oracle_out_dim(size, k, stride, pad, dilation))


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load(lib).oracle_num_threads())


def effective_kernel(k: int, dilation: int) -> int:
    """Span of a dilated filter: k + (k-1)(dilation-1) (lpnh.cn sections 2.3, 4.2)."""
    return k + (k - 1) * (dilation - 1)


def conv2d(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, relu=False,
           with_scale=True, lib=None):
    """Direct-loop convolution in fp64.  Returns (y, S) with S = sum|x*w| over
    the valid taps (or (y, None) when ``with_scale`` is False)."""
    x, w = _f64(x), _f64(w)
    N, Cin, H, W = x.shape
    Cout, cin_g, Kh, Kw = w.shape
    if cin_g * groups != Cin:
        raise ValueError("weight shape does not match Cin/groups")
    b = None if bias is None else _f64(bias)
    Ho = out_dim(H, Kh, stride, pad, dilation, lib=lib)
    Wo = out_dim(W, Kw, stride, pad, dilation, lib=lib)
    if Ho < 1 or Wo < 1:
        raise ValueError("empty output")
    y = np.empty((N, Cout, Ho, Wo), np.float64)
    s = np.empty_like(y) if with_scale else None
    rc = _load(lib).oracle_conv2d_f64(_ptr(x), _ptr(w), _ptr(b), int(bool(relu)), _ptr(y), _ptr(s),
                                   N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups)
    if rc:
        raise ValueError(f"oracle_conv2d_f64 rejected the shape (rc={rc})")
    return y, s


def conv2d_points(x, w, idx, bias=None, stride=1, pad=0, dilation=1, groups=1, relu=False,
                  lib=None):
    """Selected outputs by flat NCHW index.  Returns (y[idx], S[idx])."""
    x, w = _f64(x), _f64(w)
    N, Cin, H, W = x.shape
    Cout, _, Kh, Kw = w.shape
    b = None if bias is None else _f64(bias)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    y = np.empty(idx.shape[0], np.float64)
    s = np.empty_like(y)
    rc = _load(lib).oracle_conv2d_points_f64(_ptr(x), _ptr(w), _ptr(b), int(bool(relu)), _ptr(idx),
                                          idx.shape[0], _ptr(y), _ptr(s), N, Cin, H, W, Cout,
                                          Kh, Kw, stride, pad, dilation, groups)
    if rc:
        raise ValueError(f"oracle_conv2d_points_f64 rejected the call (rc={rc})")
    return y, s


def im2col(x, Kh, Kw, stride=1, pad=0, dilation=1, lib=None):
    """Explicit im2col: [C*Kh*Kw][N*Ho*Wo], rows (c,kh,kw), columns (n,ho,wo)."""
    x = _f64(x)
    N, C, H, W = x.shape
    Ho = out_dim(H, Kh, stride, pad, dilation, lib=lib)
    Wo = out_dim(W, Kw, stride, pad, dilation, lib=lib)
    xcol = np.empty((C * Kh * Kw, N * Ho * Wo), np.float64)
    rc = _load(lib).oracle_im2col_f64(_ptr(x), _ptr(xcol), N, C, H, W, Kh, Kw, stride, pad, dilation)
    if rc:
        raise ValueError(f"oracle_im2col_f64 rejected the shape (rc={rc})")
    return xcol


def conv2d_by_gemm(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, relu=False,
                   lib=None):
    """Explicit lowering: per group, W_g [Cout/G x (Cin/G)*Kh*Kw] @ im2col(X_g),
    then reshape the [Cout x N*Ho*Wo] product back to NCHW."""
    x, w = _f64(x), _f64(w)
    N, Cin, H, W = x.shape
    Cout, cin_g, Kh, Kw = w.shape
    cout_g = Cout // groups
    Ho = out_dim(H, Kh, stride, pad, dilation, lib=lib)
    Wo = out_dim(W, Kw, stride, pad, dilation, lib=lib)
    parts = []
    for g in range(groups):
        xcol = im2col(x[:, g * cin_g:(g + 1) * cin_g], Kh, Kw, stride, pad, dilation, lib=lib)
        wmat = w[g * cout_g:(g + 1) * cout_g].reshape(cout_g, cin_g * Kh * Kw)
        parts.append(wmat @ xcol)
    y = np.concatenate(parts, axis=0).reshape(Cout, N, Ho, Wo).transpose(1, 0, 2, 3)
    if bias is not None:
        y = y + _f64(bias)[None, :, None, None]
    if relu:
        y = np.maximum(y, 0.0)
    return np.ascontiguousarray(y)


def round_to_bf16(v):
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.

    Used where a test compares an exactly-representable fp32 result (the
    exact-integer mode) with a bf16 output: both sides take the fp32 -> bf16
    decision with round-to-nearest-even.  Values here are exact in fp32, so
    the fp64 -> fp32 step is exact.
    """
    a = np.ascontiguousarray(v, dtype=np.float64).astype(np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    keep = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & 1) == 1))
    r = ((keep + up.astype(np.uint64)) << 16).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    out[np.isnan(a)] = np.nan
    return out


def bf16_round(v):
    """Round fp64 values to the nearest bf16 (8 significant bits, fp32's
    exponent range), ties to even, in one step from the fp64 value; returned
    as fp64.  Magnitudes past the largest bf16 become infinities; below
    2**-126 the spacing stays 2**-133 (subnormals)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    _, e = np.frexp(v[fin])  # |v| = m * 2**e with 0.5 <= m < 1
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    out[fin] = np.round(v[fin] / ulp) * ulp  # np.round: half to even; the scaling is exact
    big = np.abs(out) > np.ldexp(255.0 / 128.0, 127)  # largest finite bf16: (2 - 2**-7) * 2**127
    out[big] = np.copysign(np.inf, out[big])
    return out


def separable(x, w_dw, w_pw, bias_dw=None, bias_pw=None, stride=1, pad=1, dw_relu=True,
              pw_relu=False, lib=None):
    """The depthwise-separable block (page "How a GPU executes NN convolution",
    lincklin.cn, section 25; "lnrq.cn" section 3.1): the 3x3 depthwise
    convolution (groups = C) with its bias and ReLU, its result rounded to
    bf16 (the value a depthwise layer stores), then the 1x1 convolution with
    its own bias and ReLU.  Returns (y, S), S = sum over the C input channels
    of |t * w_pw| for each output (t the rounded intermediate)."""
    C = np.asarray(x).shape[1]
    t, _ = conv2d(x, w_dw, bias_dw, stride, pad, 1, C, relu=dw_relu, with_scale=False, lib=lib)
    return conv2d(bf16_round(t), w_pw, bias_pw, 1, 0, 1, 1, relu=pw_relu, lib=lib)


def conv2d_bn(x, w, scale, shift, bias=None, stride=1, pad=0, dilation=1, groups=1, relu=False, lib=None):
    """Convolution with batch normalisation (inference form) folded into the
    epilogue (page "How a GPU executes NN convolution", lincklin.cn, section
    31): the sum, plus the bias, times scale[co] plus shift[co], then ReLU.
    Returns (y, S) with S = |scale| * (sum|x*w| + |bias|) + |shift|, the
    magnitude the result is rounded against."""
    y, s = conv2d(x, w, bias, stride, pad, dilation, groups, relu=False, lib=lib)
    sc = _f64(scale)[None, :, None, None]
    sh = _f64(shift)[None, :, None, None]
    y = y * sc + sh
    if relu:
        y = np.maximum(y, 0.0)
    b = 0.0 if bias is None else np.abs(_f64(bias))[None, :, None, None]
    return y, np.abs(sc) * (s + b) + np.abs(sh)


def transpose_out_dim(size: int, k: int, stride: int = 1, pad: int = 0, dilation: int = 1,
                      out_pad: int = 0, lib=None) -> int:
    """Output extent of the transposed convolution:
    (size-1)*stride - 2*pad + dilation*(k-1) + out_pad + 1, with
    0 <= out_pad < max(stride, dilation); -1 for arguments out of range."""
    return int(_load(lib).oracle_transpose_out_dim(size, k, stride, pad, dilation, out_pad))


def conv_transpose2d(x, w, bias=None, stride=1, pad=0, out_pad=0, dilation=1, groups=1, relu=False,
                     lib=None):
    """Transposed convolution ("lpnh.cn/news/2674933" sections 2.3, 4.2) in
    fp64 by scattering W^T X: every input pixel times the whole filter, added
    into the output window it spans.  x is NCHW, w is [Cin][Cout/G][Kh][Kw].
    Returns (y, S), S = sum |x*w| of the products each output received."""
    x, w = _f64(x), _f64(w)
    N, Cin, H, W = x.shape
    cin_w, cout_g, Kh, Kw = w.shape
    if cin_w != Cin:
        raise ValueError("weight's first dimension must be Cin")
    Cout = cout_g * groups
    b = None if bias is None else _f64(bias)
    Ho = transpose_out_dim(H, Kh, stride, pad, dilation, out_pad, lib=lib)
    Wo = transpose_out_dim(W, Kw, stride, pad, dilation, out_pad, lib=lib)
    if Ho < 1 or Wo < 1:
        raise ValueError("empty output")
    y = np.empty((N, Cout, Ho, Wo), np.float64)
    s = np.empty_like(y)
    rc = _load(lib).oracle_conv_transpose2d_f64(_ptr(x), _ptr(w), _ptr(b), int(bool(relu)), _ptr(y), _ptr(s),
                                             N, Cin, H, W, Cout, Kh, Kw, stride, pad, out_pad, dilation, groups)
    if rc:
        raise ValueError(f"oracle_conv_transpose2d_f64 rejected the shape (rc={rc})")
    return y, s


def conv_transpose2d_points(x, w, idx, bias=None, stride=1, pad=0, out_pad=0, dilation=1, groups=1,
                            relu=False, lib=None):
    """Selected outputs of the transposed convolution by flat NCHW index, each
    gathered from the input pixels whose window covers it.  Returns
    (y[idx], S[idx])."""
    x, w = _f64(x), _f64(w)
    N, Cin, H, W = x.shape
    _, cout_g, Kh, Kw = w.shape
    b = None if bias is None else _f64(bias)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    y = np.empty(idx.shape[0], np.float64)
    s = np.empty_like(y)
    rc = _load(lib).oracle_conv_transpose2d_points_f64(
        _ptr(x), _ptr(w), _ptr(b), int(bool(relu)), _ptr(idx), idx.shape[0], _ptr(y), _ptr(s),
        N, Cin, H, W, cout_g * groups, Kh, Kw, stride, pad, out_pad, dilation, groups)
    if rc:
        raise ValueError(f"oracle_conv_transpose2d_points_f64 rejected the call (rc={rc})")
    return y, s
