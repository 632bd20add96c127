"""Python binding of libconv2d.so, the gfx950 conv2d forward library.

Argument marshalling only: every function here forwards to the C entry point
of the same name in ``include/conv2d.h``; all computation runs in the HIP
kernels of ``libconv2d.so``.  Tensor arguments may be torch tensors (their
``data_ptr()`` is passed) or raw integer device addresses.  ``stream`` defaults
to torch's current stream on the current device.  A non-zero return code
raises ``Conv2dError``.  There is no fallback: if the library is not built the
import fails.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# CONV2D_LIBRARY may name another build of the same sources (tuning sweeps).
LIB_PATH = os.environ.get("CONV2D_LIBRARY") or os.path.join(_HERE, "libconv2d.so")

F32, BF16 = 0, 1
EPI_NONE, EPI_BIAS, EPI_RELU = 0, 1, 2
PATH_AUTO, PATH_DIRECT, PATH_DEPTHWISE, PATH_GEMM1X1, PATH_IGEMM = 0, 1, 2, 3, 4
PATH_IGEMM_GATHER, PATH_IGEMM_HALO = 5, 6
PATH_NAMES = {PATH_DIRECT: "direct", PATH_DEPTHWISE: "depthwise", PATH_GEMM1X1: "gemm1x1",
              PATH_IGEMM: "igemm", PATH_IGEMM_GATHER: "igemm_gather", PATH_IGEMM_HALO: "igemm_halo"}

OK = 0
ERR_ARG, ERR_GROUPS, ERR_EMPTY_OUTPUT, ERR_UNSUPPORTED, ERR_HIP = -1, -2, -3, -4, -5
ERR_NULL, ERR_DTYPE, ERR_EPILOGUE, ERR_ALIGN = -6, -7, -8, -9

# Every symbol include/conv2d.h declares.
EXPORTS = ("conv2d_fwd", "conv2d_fwd_noalloc", "conv2d_fwd_nhwc_packed", "conv2d_fwd_bn", "conv2d_fwd_nhwc_packed_bn",
           "conv2d_fwd_separable_nhwc",
           "conv2d_winograd_weight_bytes", "conv2d_winograd_transform_weights", "conv2d_fwd_winograd_nhwc",
           "conv2d_transpose_fwd", "conv2d_transpose_fwd_nhwc_packed", "conv2d_transpose_pack_weights",
           "conv2d_transpose_out_dim", "conv2d_transpose_check_args", "conv2d_transpose_select_path",
           "conv2d_packed_weight_bytes",
           "conv2d_pack_weights", "conv2d_nchw_to_nhwc", "conv2d_nhwc_to_nchw",
           "conv2d_out_dim", "conv2d_check_args", "conv2d_select_path",
           "conv2d_set_path_override", "conv2d_set_grid_limit", "conv2d_release_scratch", "conv2d_strerror",
           "conv2d_last_error")


class Conv2dError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where} failed: {strerror(code)} ({code}): {last_error()}")


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime under the same soname; importing it first
    # makes libconv2d.so bind to that one, so the process holds one runtime and
    # torch's device pointers and streams are valid in our launches.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m cnn_convolution_conv2d_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    conv_args = [P, P, P, P] + [I] * 11 + [I, I, P]
    for name in ("conv2d_fwd", "conv2d_fwd_noalloc", "conv2d_fwd_nhwc_packed"):
        f = getattr(lib, name)
        f.argtypes, f.restype = conv_args, I
    for name in ("conv2d_fwd_bn", "conv2d_fwd_nhwc_packed_bn"):
        f = getattr(lib, name)
        f.argtypes, f.restype = [P] * 6 + [I] * 13 + [P], I
    lib.conv2d_fwd_separable_nhwc.argtypes = [P] * 6 + [I] * 10 + [P]
    lib.conv2d_fwd_separable_nhwc.restype = I
    lib.conv2d_winograd_weight_bytes.argtypes = [I] * 3
    lib.conv2d_winograd_weight_bytes.restype = ctypes.c_size_t
    lib.conv2d_winograd_transform_weights.argtypes = [P, P] + [I] * 3 + [P]
    lib.conv2d_winograd_transform_weights.restype = I
    lib.conv2d_fwd_winograd_nhwc.argtypes = [P] * 4 + [I] * 8 + [P]
    lib.conv2d_fwd_winograd_nhwc.restype = I
    for name in ("conv2d_transpose_fwd", "conv2d_transpose_fwd_nhwc_packed"):
        f = getattr(lib, name)
        f.argtypes, f.restype = [P] * 4 + [I] * 14 + [P], I
    lib.conv2d_transpose_pack_weights.argtypes = [P, P] + [I] * 6 + [P]
    lib.conv2d_transpose_pack_weights.restype = I
    lib.conv2d_transpose_out_dim.argtypes, lib.conv2d_transpose_out_dim.restype = [I] * 6, I
    lib.conv2d_transpose_check_args.argtypes = [P] * 4 + [I] * 14
    lib.conv2d_transpose_check_args.restype = I
    lib.conv2d_transpose_select_path.argtypes, lib.conv2d_transpose_select_path.restype = [I] * 13, I
    lib.conv2d_packed_weight_bytes.argtypes = [I] * 6
    lib.conv2d_packed_weight_bytes.restype = ctypes.c_size_t
    lib.conv2d_pack_weights.argtypes = [P, P] + [I] * 6 + [P]
    lib.conv2d_pack_weights.restype = I
    for name in ("conv2d_nchw_to_nhwc", "conv2d_nhwc_to_nchw"):
        f = getattr(lib, name)
        f.argtypes, f.restype = [P, P] + [I] * 5 + [P], I
    lib.conv2d_out_dim.argtypes, lib.conv2d_out_dim.restype = [I] * 5, I
    lib.conv2d_check_args.argtypes, lib.conv2d_check_args.restype = [P, P, P, P] + [I] * 13, I
    lib.conv2d_select_path.argtypes, lib.conv2d_select_path.restype = [I] * 12, I
    lib.conv2d_set_path_override.argtypes, lib.conv2d_set_path_override.restype = [I], I
    lib.conv2d_set_grid_limit.argtypes, lib.conv2d_set_grid_limit.restype = [I], I
    lib.conv2d_release_scratch.argtypes, lib.conv2d_release_scratch.restype = [], None
    lib.conv2d_strerror.argtypes, lib.conv2d_strerror.restype = [I], ctypes.c_char_p
    lib.conv2d_last_error.argtypes, lib.conv2d_last_error.restype = [], ctypes.c_char_p
    return lib


lib = _load()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise Conv2dError(rc, where)
    return rc


def strerror(code: int) -> str:
    return lib.conv2d_strerror(code).decode()


def last_error() -> str:
    return lib.conv2d_last_error().decode()


def conv2d_fwd(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
               dtype, epilogue, stream=None) -> None:
    """NCHW x, [Cout][Cin/G][Kh][Kw] w, fp32 bias or None, NCHW y."""
    _check(lib.conv2d_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, Cin, H, W, Cout, Kh, Kw,
                          stride, pad, dilation, groups, dtype, epilogue, _stream(stream)),
           "conv2d_fwd")


def conv2d_fwd_noalloc(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                       dtype, epilogue, stream=None) -> None:
    """conv2d_fwd staging through the library's static 64 MiB device array
    (no allocation; calls on one GPU must not overlap)."""
    _check(lib.conv2d_fwd_noalloc(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, Cin, H, W, Cout, Kh, Kw,
                                  stride, pad, dilation, groups, dtype, epilogue, _stream(stream)),
           "conv2d_fwd_noalloc")


def conv2d_fwd_nhwc_packed(x, w_packed, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                           dilation, groups, dtype, epilogue, stream=None) -> None:
    """NHWC x, packed w (from conv2d_pack_weights), fp32 bias or None, NHWC y."""
    _check(lib.conv2d_fwd_nhwc_packed(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(y), N, Cin, H, W,
                                      Cout, Kh, Kw, stride, pad, dilation, groups, dtype, epilogue,
                                      _stream(stream)),
           "conv2d_fwd_nhwc_packed")


def conv2d_fwd_bn(x, w, bias, scale, shift, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                  dtype, epilogue, stream=None) -> None:
    """conv2d_fwd with the folded batch normalisation (fp32 scale, shift [Cout])."""
    _check(lib.conv2d_fwd_bn(_ptr(x), _ptr(w), _ptr(bias), _ptr(scale), _ptr(shift), _ptr(y), N, Cin, H, W,
                             Cout, Kh, Kw, stride, pad, dilation, groups, dtype, epilogue, _stream(stream)),
           "conv2d_fwd_bn")


def conv2d_fwd_nhwc_packed_bn(x, w_packed, bias, scale, shift, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                              dilation, groups, dtype, epilogue, stream=None) -> None:
    """conv2d_fwd_nhwc_packed with the folded batch normalisation."""
    _check(lib.conv2d_fwd_nhwc_packed_bn(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(scale), _ptr(shift),
                                         _ptr(y), N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                                         dtype, epilogue, _stream(stream)),
           "conv2d_fwd_nhwc_packed_bn")


def conv2d_fwd_separable_nhwc(x, w_dw, bias_dw, w_pw, bias_pw, y, N, C, H, W, Cout, stride, pad,
                              dtype, dw_epilogue, pw_epilogue, stream=None) -> None:
    """Fused 3x3 depthwise (+ its epilogue) then 1x1 (+ its epilogue): NHWC x,
    packed [3][3][C] w_dw, [Cout][C] w_pw, fp32 biases or None, NHWC y."""
    _check(lib.conv2d_fwd_separable_nhwc(_ptr(x), _ptr(w_dw), _ptr(bias_dw), _ptr(w_pw), _ptr(bias_pw),
                                         _ptr(y), N, C, H, W, Cout, stride, pad, dtype, dw_epilogue,
                                         pw_epilogue, _stream(stream)),
           "conv2d_fwd_separable_nhwc")


def conv2d_winograd_weight_bytes(Cout, Cin, dtype) -> int:
    return int(lib.conv2d_winograd_weight_bytes(Cout, Cin, dtype))


def conv2d_winograd_transform_weights(w, w_wino, Cout, Cin, dtype, stream=None) -> None:
    """[Cout][Cin][3][3] bf16 -> G g G^T as [16][Cin/8][Cout][8] bf16."""
    _check(lib.conv2d_winograd_transform_weights(_ptr(w), _ptr(w_wino), Cout, Cin, dtype, _stream(stream)),
           "conv2d_winograd_transform_weights")


def conv2d_fwd_winograd_nhwc(x, w_wino, bias, y, N, Cin, H, W, Cout, pad, dtype, epilogue, stream=None) -> None:
    """3x3 stride-1 convolution by Winograd F(2x2,3x3): NHWC x, transformed w, NHWC y."""
    _check(lib.conv2d_fwd_winograd_nhwc(_ptr(x), _ptr(w_wino), _ptr(bias), _ptr(y), N, Cin, H, W, Cout, pad, dtype,
                                        epilogue, _stream(stream)), "conv2d_fwd_winograd_nhwc")


def conv2d_transpose_fwd(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding, dilation,
                         groups, dtype, epilogue, stream=None) -> None:
    """Transposed convolution: NCHW x, [Cin][Cout/G][Kh][Kw] w, fp32 bias or None, NCHW y."""
    _check(lib.conv2d_transpose_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, Cin, H, W, Cout, Kh, Kw, stride,
                                    pad, output_padding, dilation, groups, dtype, epilogue, _stream(stream)),
           "conv2d_transpose_fwd")


def conv2d_transpose_fwd_nhwc_packed(x, w_packed, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad,
                                     output_padding, dilation, groups, dtype, epilogue, stream=None) -> None:
    """Transposed convolution: NHWC x, packed w (conv2d_transpose_pack_weights), NHWC y."""
    _check(lib.conv2d_transpose_fwd_nhwc_packed(_ptr(x), _ptr(w_packed), _ptr(bias), _ptr(y), N, Cin, H, W,
                                                Cout, Kh, Kw, stride, pad, output_padding, dilation, groups,
                                                dtype, epilogue, _stream(stream)),
           "conv2d_transpose_fwd_nhwc_packed")


def conv2d_transpose_pack_weights(w, w_packed, Cin, Cout, Kh, Kw, groups, dtype, stream=None) -> None:
    _check(lib.conv2d_transpose_pack_weights(_ptr(w), _ptr(w_packed), Cin, Cout, Kh, Kw, groups, dtype,
                                             _stream(stream)), "conv2d_transpose_pack_weights")


def conv2d_transpose_out_dim(size, k, stride=1, pad=0, dilation=1, output_padding=0) -> int:
    return int(lib.conv2d_transpose_out_dim(size, k, stride, pad, dilation, output_padding))


def conv2d_transpose_check_args(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding,
                                dilation, groups, dtype, epilogue) -> int:
    return int(lib.conv2d_transpose_check_args(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, Cin, H, W, Cout, Kh,
                                               Kw, stride, pad, output_padding, dilation, groups, dtype,
                                               epilogue))


def conv2d_transpose_select_path(N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding, dilation, groups,
                                 dtype) -> int:
    return _check(int(lib.conv2d_transpose_select_path(N, Cin, H, W, Cout, Kh, Kw, stride, pad, output_padding,
                                                       dilation, groups, dtype)), "conv2d_transpose_select_path")


def conv2d_packed_weight_bytes(Cout, Cin, Kh, Kw, groups, dtype) -> int:
    return int(lib.conv2d_packed_weight_bytes(Cout, Cin, Kh, Kw, groups, dtype))


def conv2d_pack_weights(w, w_packed, Cout, Cin, Kh, Kw, groups, dtype, stream=None) -> None:
    _check(lib.conv2d_pack_weights(_ptr(w), _ptr(w_packed), Cout, Cin, Kh, Kw, groups, dtype,
                                   _stream(stream)), "conv2d_pack_weights")


def conv2d_nchw_to_nhwc(src, dst, N, C, H, W, dtype, stream=None) -> None:
    _check(lib.conv2d_nchw_to_nhwc(_ptr(src), _ptr(dst), N, C, H, W, dtype, _stream(stream)),
           "conv2d_nchw_to_nhwc")


def conv2d_nhwc_to_nchw(src, dst, N, C, H, W, dtype, stream=None) -> None:
    _check(lib.conv2d_nhwc_to_nchw(_ptr(src), _ptr(dst), N, C, H, W, dtype, _stream(stream)),
           "conv2d_nhwc_to_nchw")


def conv2d_out_dim(size, k, stride=1, pad=0, dilation=1) -> int:
    return int(lib.conv2d_out_dim(size, k, stride, pad, dilation))


def conv2d_check_args(x, w, bias, y, N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups,
                      dtype, epilogue) -> int:
    """Host-only validation; returns the code a forward call would return."""
    return int(lib.conv2d_check_args(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), N, Cin, H, W, Cout,
                                     Kh, Kw, stride, pad, dilation, groups, dtype, epilogue))


def conv2d_select_path(N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation, groups, dtype) -> int:
    return _check(int(lib.conv2d_select_path(N, Cin, H, W, Cout, Kh, Kw, stride, pad, dilation,
                                             groups, dtype)), "conv2d_select_path")


def conv2d_set_path_override(path: int) -> int:
    return _check(int(lib.conv2d_set_path_override(path)), "conv2d_set_path_override")


def conv2d_set_grid_limit(max_workgroups: int) -> int:
    return _check(int(lib.conv2d_set_grid_limit(max_workgroups)), "conv2d_set_grid_limit")


def conv2d_release_scratch() -> None:
    lib.conv2d_release_scratch()
