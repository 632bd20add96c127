"""Host-side tests of the C ABI (no GPU): the library loads, exports every
symbol the header declares, and validates arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import conv_inputs as ci
import oracle
from helpers import ROOT, ensure_built

ensure_built()
import cnn_convolution_conv2d_amd as c2  # noqa: E402

HEADER = os.path.join(ROOT, "include", "conv2d.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv2d_\w+)\s*\(", text)))


def test_header_declares_what_binding_lists():
    assert header_functions() == sorted(c2.EXPORTS)


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(c2.LIB_PATH)
    for name in header_functions():
        assert hasattr(raw, name), name


def test_out_dim_agrees_with_oracle():
    for n in (1, 2, 3, 5, 7, 56, 64, 112, 224):
        for k in (1, 2, 3, 5, 7):
            for s in (1, 2, 3):
                for p in (0, 1, 2, 3):
                    for d in (1, 2, 3):
                        want = oracle.out_dim(n, k, s, p, d)
                        assert c2.conv2d_out_dim(n, k, s, p, d) == max(want, 0), (n, k, s, p, d)
    assert c2.conv2d_out_dim(224, 3, 0, 1, 1) == c2.ERR_ARG
    assert c2.conv2d_out_dim(224, 3, 1, -1, 1) == c2.ERR_ARG
    assert c2.conv2d_out_dim(224, 3, 1, 1, 0) == c2.ERR_ARG


GOOD = dict(N=2, Cin=8, H=9, W=9, Cout=16, Kh=3, Kw=3, stride=1, pad=1, dilation=1, groups=2,
            dtype=c2.BF16, epilogue=c2.EPI_BIAS | c2.EPI_RELU)
P = 0x1000  # a non-NULL address; nothing is dereferenced by validation


def _check(**over):
    a = dict(GOOD)
    a.update(over)
    ptrs = dict(x=P, w=P, bias=P, y=P)
    for k in ("x", "w", "bias", "y"):
        if k in a:
            ptrs[k] = a.pop(k)
    return c2.conv2d_check_args(ptrs["x"], ptrs["w"], ptrs["bias"], ptrs["y"], **a)


@pytest.mark.parametrize("over,code", [
    ({}, c2.OK),
    ({"N": 0}, c2.ERR_ARG), ({"Cin": -1}, c2.ERR_ARG), ({"H": 0}, c2.ERR_ARG),
    ({"Kh": 0}, c2.ERR_ARG), ({"stride": 0}, c2.ERR_ARG), ({"dilation": 0}, c2.ERR_ARG),
    ({"pad": -1}, c2.ERR_ARG), ({"groups": 0}, c2.ERR_ARG),
    ({"groups": 3}, c2.ERR_GROUPS), ({"Cout": 15}, c2.ERR_GROUPS),
    ({"H": 2, "pad": 0}, c2.ERR_EMPTY_OUTPUT), ({"W": 4, "pad": 0, "dilation": 2}, c2.ERR_EMPTY_OUTPUT),
    ({"dtype": 7}, c2.ERR_DTYPE), ({"epilogue": 4}, c2.ERR_EPILOGUE), ({"epilogue": -1}, c2.ERR_EPILOGUE),
    ({"x": None}, c2.ERR_NULL), ({"w": None}, c2.ERR_NULL), ({"y": None}, c2.ERR_NULL),
    ({"bias": None}, c2.ERR_NULL),
    ({"bias": None, "epilogue": c2.EPI_RELU}, c2.OK),
    ({"N": 1 << 20, "Cin": 64, "H": 64, "W": 64, "groups": 1}, c2.ERR_UNSUPPORTED),
])
def test_check_args_codes(over, code):
    assert _check(**over) == code


def test_forward_entries_reject_bad_args_before_any_gpu_work():
    # invalid calls return their code without enqueueing anything, GPU or not
    for fn in (c2.lib.conv2d_fwd, c2.lib.conv2d_fwd_nhwc_packed):
        rc = fn(P, P, P, P, 0, 8, 9, 9, 16, 3, 3, 1, 1, 1, 1, c2.BF16, 0, None)
        assert rc == c2.ERR_ARG
        rc = fn(P, P, None, P, 1, 8, 9, 9, 16, 3, 3, 1, 1, 1, 1, c2.BF16, c2.EPI_BIAS, None)
        assert rc == c2.ERR_NULL
        assert "bias" in c2.last_error()
    for fn in (c2.lib.conv2d_fwd_bn, c2.lib.conv2d_fwd_nhwc_packed_bn):
        # scale and shift are required; other checks as for the plain entries
        rc = fn(P, P, P, None, P, P, 1, 8, 9, 9, 16, 3, 3, 1, 1, 1, 1, c2.BF16, 0, None)
        assert rc == c2.ERR_NULL and "scale" in c2.last_error()
        rc = fn(P, P, P, P, None, P, 1, 8, 9, 9, 16, 3, 3, 1, 1, 1, 1, c2.BF16, 0, None)
        assert rc == c2.ERR_NULL
        assert fn(P, P, P, P, P, P, 0, 8, 9, 9, 16, 3, 3, 1, 1, 1, 1, c2.BF16, 0, None) == c2.ERR_ARG
        assert fn(P, P, P, P, P, P, 1, 8, 9, 9, 16, 3, 3, 1, 1, 1, 3, c2.BF16, 0, None) == c2.ERR_GROUPS
    assert c2.lib.conv2d_pack_weights(P, P, 16, 8, 3, 3, 3, c2.BF16, None) == c2.ERR_GROUPS
    assert c2.lib.conv2d_nchw_to_nhwc(P, None, 1, 8, 9, 9, c2.BF16, None) == c2.ERR_NULL
    assert c2.lib.conv2d_nhwc_to_nchw(P, P, 1, 8, 9, 9, 5, None) == c2.ERR_DTYPE


def _sep_call(x=P, wd=P, bd=P, wq=P, bq=P, y=P, **over):
    a = dict(N=1, C=144, H=9, W=9, Cout=24, stride=1, pad=1, dtype=c2.BF16,
             dw=c2.EPI_BIAS | c2.EPI_RELU, pw=c2.EPI_NONE)
    a.update(over)
    return c2.lib.conv2d_fwd_separable_nhwc(x, wd, bd, wq, bq, y, a["N"], a["C"], a["H"], a["W"],
                                            a["Cout"], a["stride"], a["pad"], a["dtype"], a["dw"],
                                            a["pw"], None)


@pytest.mark.parametrize("over,code", [
    ({"N": 0}, c2.ERR_ARG), ({"C": 0}, c2.ERR_ARG), ({"Cout": -2}, c2.ERR_ARG),
    ({"stride": 0}, c2.ERR_ARG), ({"pad": -1}, c2.ERR_ARG),
    ({"dtype": 7}, c2.ERR_DTYPE), ({"dw": 4}, c2.ERR_EPILOGUE), ({"pw": -1}, c2.ERR_EPILOGUE),
    ({"x": None}, c2.ERR_NULL), ({"wd": None}, c2.ERR_NULL), ({"wq": None}, c2.ERR_NULL),
    ({"y": None}, c2.ERR_NULL), ({"bd": None}, c2.ERR_NULL),
    ({"bq": None, "pw": c2.EPI_BIAS}, c2.ERR_NULL),
    ({"H": 1, "pad": 0}, c2.ERR_EMPTY_OUTPUT), ({"W": 2, "pad": 0, "stride": 2}, c2.ERR_EMPTY_OUTPUT),
    ({"dtype": c2.F32}, c2.ERR_UNSUPPORTED), ({"C": 12}, c2.ERR_UNSUPPORTED),
    ({"C": 264}, c2.ERR_UNSUPPORTED), ({"Cout": 22}, c2.ERR_UNSUPPORTED),
    ({"Cout": 132}, c2.ERR_UNSUPPORTED), ({"stride": 3}, c2.ERR_UNSUPPORTED),
    ({"x": P + 8}, c2.ERR_ALIGN), ({"wq": P + 4}, c2.ERR_ALIGN),
])
def test_separable_entry_rejects_bad_args_before_any_gpu_work(over, code):
    """Every one of these returns its code from the host checks, so nothing
    is enqueued (none of the addresses is ever dereferenced)."""
    assert _sep_call(**over) == code
    assert c2.last_error()


def test_strerror_names_every_code():
    seen = set()
    for code in range(0, -10, -1):
        s = c2.strerror(code)
        assert s and s != "unknown error code"
        seen.add(s)
    assert len(seen) == 10
    assert c2.strerror(-100) == "unknown error code"


def test_packed_weight_bytes():
    assert c2.conv2d_packed_weight_bytes(256, 128, 3, 3, 1, c2.BF16) == 256 * 128 * 9 * 2
    assert c2.conv2d_packed_weight_bytes(256, 256, 3, 3, 4, c2.BF16) == 256 * 64 * 9 * 2
    assert c2.conv2d_packed_weight_bytes(32, 3, 3, 3, 1, c2.F32) == 32 * 27 * 4
    assert c2.conv2d_packed_weight_bytes(16, 8, 3, 3, 3, c2.BF16) == 0


@pytest.mark.parametrize("cid,li,path", [
    (1, 0, c2.PATH_DIRECT), (2, 0, c2.PATH_IGEMM_HALO), (3, 0, c2.PATH_DEPTHWISE),
    (3, 1, c2.PATH_GEMM1X1), (4, 0, c2.PATH_IGEMM_HALO), (5, 0, c2.PATH_GEMM1X1),
    (5, 1, c2.PATH_IGEMM_HALO), (5, 2, c2.PATH_GEMM1X1), (5, 3, c2.PATH_IGEMM_GATHER),
])
def test_path_selection_for_workloads(cid, li, path):
    ly = ci.layer(cid, li)
    dt = c2.F32 if ly.dtype == ci.F32 else c2.BF16
    assert c2.conv2d_select_path(ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh, ly.Kw, ly.stride, ly.pad,
                                 ly.dilation, ly.groups, dt) == path


def test_path_selection_fallbacks_and_override():
    # channels not a multiple of 8 -> direct loop; depthwise with odd C -> direct
    assert c2.conv2d_select_path(1, 3, 9, 9, 16, 3, 3, 1, 1, 1, 1, c2.BF16) == c2.PATH_DIRECT
    assert c2.conv2d_select_path(1, 6, 9, 9, 6, 3, 3, 1, 1, 1, 6, c2.BF16) == c2.PATH_DIRECT
    # 1x1 with stride 2 is not a plain GEMM -> implicit GEMM (gather: stride 2)
    assert c2.conv2d_select_path(1, 64, 9, 9, 64, 1, 1, 2, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    # few output channels per group, or a filter span beyond the halo buffer -> gather
    assert c2.conv2d_select_path(1, 64, 9, 9, 32, 3, 3, 1, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    assert c2.conv2d_select_path(1, 64, 19, 19, 64, 3, 3, 1, 3, 3, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    assert c2.conv2d_select_path(1, 64, 19, 19, 64, 5, 5, 1, 2, 1, 1, c2.BF16) == c2.PATH_IGEMM_HALO
    prev = c2.conv2d_set_path_override(c2.PATH_DIRECT)
    try:
        assert prev == c2.PATH_AUTO
        assert c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 1, 1, 1, 1, c2.BF16) == c2.PATH_DIRECT
        c2.conv2d_set_path_override(c2.PATH_GEMM1X1)
        with pytest.raises(c2.Conv2dError):
            c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 1, 1, 1, 1, c2.BF16)
    finally:
        c2.conv2d_set_path_override(c2.PATH_AUTO)
    c2.conv2d_set_path_override(c2.PATH_IGEMM)
    try:
        assert c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 1, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_HALO
        # the implicit-GEMM override picks the gather for every stride above 1
        assert c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 2, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
        assert c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 3, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
        c2.conv2d_set_path_override(c2.PATH_IGEMM_HALO)
        # forced halo path: 3x3 stride 2 runs on the phase-split staged window;
        # stride 3, or stride 2 with dilation, has no halo kernel
        assert c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 2, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_HALO
        with pytest.raises(c2.Conv2dError):
            c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 3, 1, 1, 1, c2.BF16)
        with pytest.raises(c2.Conv2dError):
            c2.conv2d_select_path(1, 64, 9, 9, 64, 3, 3, 2, 1, 2, 1, c2.BF16)
        with pytest.raises(c2.Conv2dError):  # 32 output channels: below the kernel's minimum
            c2.conv2d_select_path(1, 64, 9, 9, 32, 3, 3, 2, 1, 1, 1, c2.BF16)
    finally:
        c2.conv2d_set_path_override(c2.PATH_AUTO)
    assert c2.lib.conv2d_set_path_override(9) == c2.ERR_ARG


def test_tensors_past_the_buffer_offset_limit_take_the_direct_path():
    """The MFMA and depthwise kernels stand for a zero tap or a dropped store
    with the out-of-range buffer offset 0x7ffffff0; an activation of 2 GiB or
    more (valid: below 2**31 elements) would put real data at that offset, so
    such shapes must go to the direct kernel."""
    big = 4100  # 64 channels x 4100 x 4100 bf16 = 2.15 GB, 1.08e9 elements
    assert 64 * big * big * 2 >= 0x7fff0000 and 64 * big * big < 2**31 - 1
    # padded 3x3 (halo and gather), stride-2 3x3 (gather), 1x1 (GEMM), depthwise
    for args in ((1, 64, big, big, 64, 3, 3, 1, 1, 1, 1), (1, 64, big, big, 64, 3, 3, 2, 1, 1, 1),
                 (1, 64, big, big, 64, 1, 1, 1, 0, 1, 1), (1, 64, big, big, 64, 3, 3, 1, 1, 1, 64)):
        assert c2.conv2d_select_path(*args, c2.BF16) == c2.PATH_DIRECT, args
    # the output alone past the limit (a 1x1 widening 8 -> 128 channels)
    assert c2.conv2d_select_path(1, 8, 3000, 3000, 128, 1, 1, 1, 0, 1, 1, c2.BF16) == c2.PATH_DIRECT
    # just below the limit the MFMA paths still serve it
    assert c2.conv2d_select_path(1, 64, 4000, 4000, 64, 3, 3, 2, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    assert c2.conv2d_transpose_select_path(1, 64, big, big, 64, 3, 3, 1, 1, 0, 1, 1, c2.BF16) == c2.PATH_DIRECT


def test_grid_limit_is_validated_and_returns_previous():
    assert c2.lib.conv2d_set_grid_limit(-1) == c2.ERR_ARG
    assert c2.conv2d_set_grid_limit(7) == 0
    assert c2.conv2d_set_grid_limit(0) == 7


# ------------------------------------------------------------------ transposed convolution

def test_transpose_out_dim_agrees_with_oracle():
    for H in (1, 2, 5, 28, 56):
        for K in (1, 2, 3, 4, 5):
            for S in (1, 2, 3):
                for P in (0, 1, 2, 3):
                    for D in (1, 2):
                        for OP in range(max(S, D)):
                            want = oracle.transpose_out_dim(H, K, S, P, D, OP)
                            got = c2.conv2d_transpose_out_dim(H, K, S, P, D, OP)
                            assert got == max(want, 0), (H, K, S, P, D, OP)
    assert c2.conv2d_transpose_out_dim(5, 3, 2, 1, 1, 2) == c2.ERR_ARG   # OP >= max(S, D)
    assert c2.conv2d_transpose_out_dim(5, 3, 0, 1, 1, 0) == c2.ERR_ARG
    assert c2.conv2d_transpose_out_dim(5, 3, 2, -1, 1, 0) == c2.ERR_ARG


TGOOD = dict(x=P, w=P, bias=P, y=P, N=2, Cin=16, H=7, W=9, Cout=24, Kh=4, Kw=4, stride=2, pad=1,
             output_padding=0, dilation=1, groups=2, dtype=c2.BF16, epilogue=3)


@pytest.mark.parametrize("over,code", [
    ({}, c2.OK),
    ({"dtype": 5}, c2.ERR_DTYPE),
    ({"epilogue": 4}, c2.ERR_EPILOGUE),
    ({"N": 0}, c2.ERR_ARG),
    ({"Kh": 0}, c2.ERR_ARG),
    ({"stride": 0}, c2.ERR_ARG),
    ({"pad": -1}, c2.ERR_ARG),
    ({"output_padding": 2}, c2.ERR_ARG),
    ({"output_padding": -1}, c2.ERR_ARG),
    ({"output_padding": 1, "stride": 1, "dilation": 2}, c2.OK),
    ({"groups": 5}, c2.ERR_GROUPS),
    ({"x": None}, c2.ERR_NULL),
    ({"bias": None}, c2.ERR_NULL),
    ({"bias": None, "epilogue": 2}, c2.OK),
    ({"H": 1, "W": 1, "Kh": 1, "Kw": 1, "pad": 1}, c2.ERR_EMPTY_OUTPUT),
    ({"N": 4096, "Cin": 1024, "H": 64, "W": 64}, c2.ERR_UNSUPPORTED),
])
def test_transpose_check_args_codes(over, code):
    a = dict(TGOOD, **over)
    assert c2.conv2d_transpose_check_args(**a) == code


def test_transpose_entries_reject_bad_args_before_any_gpu_work():
    for fn in (c2.lib.conv2d_transpose_fwd, c2.lib.conv2d_transpose_fwd_nhwc_packed):
        assert fn(P, P, P, P, 1, 8, 9, 9, 16, 3, 3, 2, 1, 2, 1, 1, c2.BF16, 0, None) == c2.ERR_ARG
        assert fn(None, P, P, P, 1, 8, 9, 9, 16, 3, 3, 2, 1, 0, 1, 1, c2.BF16, 0, None) == c2.ERR_NULL
        assert fn(P, P, P, P, 1, 8, 9, 9, 16, 3, 3, 2, 1, 0, 1, 3, c2.BF16, 0, None) == c2.ERR_GROUPS
    lib = c2.lib
    assert lib.conv2d_transpose_pack_weights(P, P, 16, 8, 3, 3, 3, c2.BF16, None) == c2.ERR_GROUPS
    assert lib.conv2d_transpose_pack_weights(None, P, 16, 8, 3, 3, 1, c2.BF16, None) == c2.ERR_NULL
    assert lib.conv2d_transpose_pack_weights(P, P, 16, 8, 3, 3, 1, 9, None) == c2.ERR_DTYPE


def test_transpose_path_selection():
    sel = c2.conv2d_transpose_select_path
    for li, want in ((0, c2.PATH_IGEMM_HALO), (1, c2.PATH_GEMM1X1)):
        ly = ci.layer(6, li)
        assert sel(ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh, ly.Kw, ly.stride, ly.pad, ly.out_pad, ly.dilation,
                   ly.groups, c2.BF16) == want
    # kernel == stride but padding, output padding or too many rows: the phase GEMM
    assert sel(1, 16, 8, 8, 32, 2, 2, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    assert sel(1, 16, 8, 8, 32, 2, 2, 2, 0, 1, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    assert sel(1, 16, 8, 8, 32, 4, 4, 4, 0, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
    assert sel(1, 16, 8, 8, 48, 2, 2, 2, 0, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER   # Cout % 32
    assert sel(1, 12, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_DIRECT   # Cin % 8 != 0
    assert sel(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER   # Cin % 32 != 0
    assert sel(1, 32, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_HALO
    assert sel(1, 32, 8, 8, 16, 4, 4, 2, 1, 0, 2, 1, c2.BF16) == c2.PATH_IGEMM_GATHER   # dilation 2
    assert sel(1, 32, 8, 8, 16, 3, 3, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER   # 3x3
    assert sel(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.F32) == c2.PATH_DIRECT
    prev = c2.conv2d_set_path_override(c2.PATH_DEPTHWISE)
    try:
        with pytest.raises(c2.Conv2dError):
            sel(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16)
        c2.conv2d_set_path_override(c2.PATH_DIRECT)
        assert sel(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_DIRECT
        c2.conv2d_set_path_override(c2.PATH_IGEMM)
        assert sel(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_GATHER
        c2.conv2d_set_path_override(c2.PATH_IGEMM_HALO)
        assert sel(1, 32, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16) == c2.PATH_IGEMM_HALO
        with pytest.raises(c2.Conv2dError):
            sel(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16)
    finally:
        c2.conv2d_set_path_override(prev)


# ------------------------------------------------------------------ Winograd

def test_winograd_entries_reject_bad_args_before_any_gpu_work():
    assert c2.conv2d_winograd_weight_bytes(256, 128, c2.BF16) == 16 * 256 * 128 * 2
    assert c2.conv2d_winograd_weight_bytes(256, 12, c2.BF16) == 0
    assert c2.conv2d_winograd_weight_bytes(256, 128, c2.F32) == 0
    f = c2.lib.conv2d_fwd_winograd_nhwc
    assert f(None, P, P, P, 1, 16, 8, 8, 16, 1, c2.BF16, 0, None) == c2.ERR_NULL
    assert f(P, P, None, P, 1, 16, 8, 8, 16, 1, c2.BF16, 1, None) == c2.ERR_NULL
    assert f(P, P, P, P, 1, 16, 8, 8, 16, -1, c2.BF16, 0, None) == c2.ERR_ARG
    assert f(P, P, P, P, 0, 16, 8, 8, 16, 1, c2.BF16, 0, None) == c2.ERR_ARG
    assert f(P, P, P, P, 1, 16, 2, 2, 16, 0, c2.BF16, 0, None) == c2.ERR_EMPTY_OUTPUT
    assert f(P, P, P, P, 1, 16, 8, 8, 16, 1, c2.F32, 0, None) == c2.ERR_UNSUPPORTED
    assert f(P, P, P, P, 1, 12, 8, 8, 16, 1, c2.BF16, 0, None) == c2.ERR_UNSUPPORTED
    assert f(P, P, P, P, 1, 16, 8, 8, 18, 1, c2.BF16, 0, None) == c2.ERR_UNSUPPORTED
    assert f(P, P, P, P, 1, 16, 8, 8, 16, 1, 7, 0, None) == c2.ERR_DTYPE
    assert f(P, P, P, P, 1, 16, 8, 8, 16, 1, c2.BF16, 8, None) == c2.ERR_EPILOGUE
    assert f(P + 2, P, P, P, 1, 16, 8, 8, 16, 1, c2.BF16, 0, None) == c2.ERR_ALIGN
    t = c2.lib.conv2d_winograd_transform_weights
    assert t(None, P, 16, 16, c2.BF16, None) == c2.ERR_NULL
    assert t(P, P, 16, 12, c2.BF16, None) == c2.ERR_UNSUPPORTED
    assert t(P, P, 16, 16, c2.F32, None) == c2.ERR_UNSUPPORTED
    assert t(P, P, 0, 16, c2.BF16, None) == c2.ERR_ARG
