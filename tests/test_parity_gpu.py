"""GPU parity: every kernel path against the fp64 oracle through the C ABI.

Tolerances (written here, applied element by element):
  fp32  max |y - yref| / (S + |b|) <= 1e-5
  bf16  |y - yref| <= 1e-2 * S + 1e-3
  exact-integer mode: x in {-2..2}, w in {-1,0,1}, integer bias; every
  partial sum is an integer below 2^24, exact in fp32 in any order, so the
  bf16 output must equal round-to-nearest-even(yref) bit for bit.
S = sum |x*w| over the valid taps of each output (from the oracle).
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import check_bf16, check_f32, compare_full, ensure_built, gpu_available, run_nchw, run_nhwc

pytestmark = pytest.mark.gpu

if gpu_available():
    ensure_built()
    import torch
    import cnn_convolution_conv2d_amd as c2


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")
    yield
    c2.conv2d_set_path_override(c2.PATH_AUTO)


def _relu(ly):
    return bool(ly.epilogue & ci.EPI_RELU)


def _ref(x, w, b, ly):
    return oracle.conv2d(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, relu=_relu(ly))


def _compare(y, yref, s, b, dtype, what):
    if dtype == ci.F32:
        bb = 0.0 if b is None else np.abs(b.astype(np.float64))[None, :, None, None]
        return check_f32(y, yref, s, bb, what)
    return check_bf16(y, yref, s, what)


# Reduced activation sizes that still span several tiles and end in a
# ragged tile; channel counts, kernels, strides, groups stay those of the layer.
SMALL = {(1, 0): dict(N=1), (2, 0): dict(N=2, H=23, W=23), (3, 0): dict(N=2, H=19, W=21),
         (3, 1): dict(N=2, H=19, W=21), (4, 0): dict(N=2, H=19, W=17), (5, 0): dict(N=2, H=21, W=21),
         (5, 1): dict(N=2, H=21, W=21), (5, 2): dict(N=2, H=21, W=21), (5, 3): dict(N=2, H=21, W=23)}
LAYERS = list(SMALL)


@pytest.mark.parametrize("cid,li", LAYERS, ids=[f"cfg{c}-{ci.layer(c, l).name}" for c, l in LAYERS])
def test_layer_small_random(cid, li):
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, **SMALL[(cid, li)])
    say(f"[parity] cfg{cid} {ly.name} random x{x.shape}")
    y = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    yref, s = _ref(x, w, b, ly)
    _compare(y, yref, s, b, ly.dtype, f"cfg{cid} {ly.name}")


@pytest.mark.parametrize("cid,li", LAYERS, ids=[f"cfg{c}-{ci.layer(c, l).name}" for c, l in LAYERS])
def test_layer_small_exact_integer(cid, li):
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, mode="int", **SMALL[(cid, li)])
    say(f"[parity] cfg{cid} {ly.name} exact-integer x{x.shape}")
    y = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    yref, _ = _ref(x, w, b, ly)
    want = yref if ly.dtype == ci.F32 else oracle.round_to_bf16(yref)
    np.testing.assert_array_equal(y, want)


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("cid,li", LAYERS, ids=[f"cfg{c}-{ci.layer(c, l).name}" for c, l in LAYERS])
def test_layer_full_size(cid, li, mode):
    """Full workload size, the same NHWC entry and launch the benchmark times;
    every output element compared with the oracle (run a few images at a
    time)."""
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, mode=mode)
    say(f"[parity] cfg{cid} {ly.name} full {mode} x{x.shape}")
    yd = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue,
                  return_dev=True)
    assert not torch.isnan(yd.float()).any().item()
    worst = compare_full(yd, x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, _relu(ly), ly.dtype, mode,
                         f"cfg{cid} {ly.name} full {mode}")
    say(f"[parity] cfg{cid} {ly.name} full {mode}: worst err/tol {worst:.3g}")


@pytest.mark.parametrize("mode", ["random", "int"])
def test_stride2_staged_window_full_size(mode):
    """The 3x3 stride-2 layer (64 x 128 x 56 x 56 -> 128 x 28 x 28) on the
    phase-split staged-window kernel, which runs when the halo path is
    forced; every output element compared with the oracle."""
    cid, li = 5, 3
    ly = ci.layer(cid, li)
    assert ly.stride == 2 and ly.Kh == 3
    x, w, b = ci.layer_tensors(cid, li, mode=mode)
    c2.conv2d_set_path_override(c2.PATH_IGEMM_HALO)
    try:
        assert c2.conv2d_select_path(ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh, ly.Kw, ly.stride, ly.pad,
                                     ly.dilation, ly.groups, c2.BF16) == c2.PATH_IGEMM_HALO
        say(f"[parity] cfg{cid} {ly.name} staged window full {mode} x{x.shape}")
        yd = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue,
                      return_dev=True)
    finally:
        c2.conv2d_set_path_override(c2.PATH_AUTO)
    worst = compare_full(yd, x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, _relu(ly), ly.dtype, mode,
                         f"cfg{cid} {ly.name} staged window full {mode}")
    say(f"[parity] cfg{cid} {ly.name} staged window full {mode}: worst err/tol {worst:.3g}")


def test_chained_separable_pair():
    """Pointwise takes the GPU's own depthwise output (each kernel checked on
    exactly the input it saw)."""
    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    x, wdw, bdw = ci.layer_tensors(3, 0, N=2, H=23, W=23)
    _, wpw, bpw = ci.layer_tensors(3, 1)
    say("[parity] cfg3 chained depthwise -> pointwise")
    t = run_nhwc(x, wdw, bdw, dw.stride, dw.pad, dw.dilation, dw.groups, dw.dtype, dw.epilogue)
    tref, ts = _ref(x, wdw, bdw, dw)
    check_bf16(t, tref, ts, "depthwise")
    y = run_nhwc(t.astype(np.float32), wpw, bpw, pw.stride, pw.pad, pw.dilation, pw.groups, pw.dtype,
                 pw.epilogue)
    yref, s = _ref(t, wpw, bpw, pw)
    check_bf16(y, yref, s, "pointwise on GPU depthwise output")


def test_chained_bottleneck():
    lys = [ci.layer(5, i) for i in range(3)]
    x, _, _ = ci.layer_tensors(5, 0, N=2, H=15, W=17)
    for i, ly in enumerate(lys):
        _, w, b = ci.layer_tensors(5, i)
        say(f"[parity] cfg5 chained {ly.name}")
        y = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
        yref, s = _ref(x, w, b, ly)
        check_bf16(y, yref, s, ly.name)
        x = y.astype(np.float32)


# ------------------------------------------------------------------ path sweep

def _sweep():
    cases = []
    # (N, Cin, H, W, Cout, Kh, Kw, S, P, D, G)
    for S in (1, 2, 3):
        for P in (0, 1, 2):
            for D in (1, 2):
                cases.append((2, 16, 11, 9, 32, 3, 3, S, P, D, 1))
    cases += [
        (1, 8, 5, 7, 8, 1, 1, 1, 0, 1, 1), (3, 24, 6, 5, 40, 1, 1, 1, 0, 1, 1),
        (1, 32, 9, 9, 16, 5, 5, 1, 2, 1, 1), (2, 64, 7, 8, 64, 3, 2, 2, 1, 1, 2),
        (1, 16, 4, 4, 16, 3, 3, 1, 0, 1, 1), (1, 16, 1, 1, 16, 3, 3, 1, 1, 1, 1),
        (2, 48, 13, 3, 12, 3, 3, 1, 1, 3, 1), (1, 8, 3, 3, 4, 7, 7, 1, 3, 1, 1),
        (1, 96, 10, 10, 96, 1, 1, 2, 0, 1, 1), (2, 32, 8, 8, 32, 3, 3, 1, 1, 1, 4),
        (1, 256, 5, 6, 8, 3, 3, 1, 1, 1, 1), (1, 8, 6, 6, 260, 3, 3, 1, 1, 1, 1),
        # shapes for the halo-tile kernel (stride 1, Cout/G > 32): ragged 16x16
        # and 8x32 pixel blocks, dilation, 5x5, groups, Cin/G not a multiple of
        # the 32-channel chunk, Cout/G not a multiple of the channel tile
        (2, 64, 19, 21, 64, 3, 3, 1, 1, 1, 1), (1, 32, 17, 40, 48, 3, 3, 1, 1, 1, 1),
        (2, 128, 9, 35, 256, 3, 3, 1, 1, 1, 1), (1, 40, 12, 12, 36, 3, 3, 1, 2, 2, 1),
        (1, 64, 11, 13, 128, 5, 5, 1, 2, 1, 1), (2, 96, 10, 10, 192, 3, 3, 1, 1, 1, 2),
        (1, 16, 20, 18, 300, 3, 1, 1, 0, 1, 1), (1, 24, 7, 33, 72, 1, 3, 1, 1, 2, 1),
        (1, 8, 2, 3, 40, 3, 3, 1, 1, 1, 1), (1, 136, 6, 5, 64, 3, 3, 1, 0, 1, 1),
        # 1x1 shapes for the streaming pointwise kernel (Cin up to 256 in
        # 16-channel slices, Cout split into 128-channel work items, Cout not a
        # multiple of 8, more 32-pixel tiles than waves) and for the tiled GEMM
        # (Cin or Cout above 256)
        (2, 256, 9, 11, 64, 1, 1, 1, 0, 1, 1), (1, 64, 13, 17, 256, 1, 1, 1, 0, 1, 1),
        (1, 144, 7, 9, 24, 1, 1, 1, 0, 1, 1), (1, 32, 5, 5, 20, 1, 1, 1, 0, 1, 1),
        (16, 16, 64, 70, 16, 1, 1, 1, 0, 1, 1), (1, 264, 3, 5, 16, 1, 1, 1, 0, 1, 1),
        (1, 16, 4, 6, 272, 1, 1, 1, 0, 1, 1), (2, 40, 9, 7, 136, 1, 1, 1, 0, 1, 1),
        # 192 and 256 input channels: activations through half tiles in LDS
        (1, 192, 7, 13, 96, 1, 1, 1, 0, 1, 1), (2, 256, 5, 7, 40, 1, 1, 1, 0, 1, 1),
        (1, 192, 3, 11, 256, 1, 1, 1, 0, 1, 1),
    ]
    return cases


DW_CASES = [(2, 16, 11, 9, 3, 3, 1, 1, 1), (1, 32, 7, 8, 3, 3, 2, 1, 1), (2, 8, 9, 9, 5, 5, 1, 2, 1),
            (1, 24, 10, 7, 3, 3, 1, 2, 2), (1, 16, 1, 1, 3, 3, 1, 1, 1), (1, 8, 6, 5, 3, 3, 1, 0, 1),
            (2, 144, 9, 13, 3, 3, 1, 1, 1), (1, 40, 8, 8, 1, 1, 1, 0, 1)]


PATHS = {"direct": "PATH_DIRECT", "igemm_gather": "PATH_IGEMM_GATHER", "igemm_halo": "PATH_IGEMM_HALO",
         "gemm1x1": "PATH_GEMM1X1"}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("mode", ["random", "int"])
def test_path_sweep(path, mode):
    """Every case the forced path can run (the library's own support check),
    each with and without the bias+ReLU epilogue."""
    pid = getattr(c2, PATHS[path])
    ran = 0
    for k, (N, Cin, H, W, Cout, Kh, Kw, S, P, D, G) in enumerate(_sweep()):
        if oracle.out_dim(H, Kh, S, P, D) < 1 or oracle.out_dim(W, Kw, S, P, D) < 1:
            continue
        c2.conv2d_set_path_override(pid)
        try:
            c2.conv2d_select_path(N, Cin, H, W, Cout, Kh, Kw, S, P, D, G, c2.BF16)
        except c2.Conv2dError:
            continue
        for epi in (0, 3):
            x, w, b = ci.random_tensors(100 + k, N, Cin, H, W, Cout, Kh, Kw, G, mode=mode, bias=epi & 1)
            say(f"[sweep] {path} {mode} case {k} {(N, Cin, H, W, Cout, Kh, Kw, S, P, D, G)} epi {epi}")
            y = run_nhwc(x, w, b, S, P, D, G, ci.BF16, epi)
            yref, s = oracle.conv2d(x, w, b, S, P, D, G, relu=bool(epi & 2))
            if mode == "int":
                np.testing.assert_array_equal(y, oracle.round_to_bf16(yref))
            else:
                check_bf16(y, yref, s, f"{path} case {k}")
            ran += 1
    assert ran >= 4


@pytest.mark.parametrize("path", ["depthwise", "direct"])
@pytest.mark.parametrize("mode", ["random", "int"])
def test_depthwise_sweep(path, mode):
    c2.conv2d_set_path_override(c2.PATH_DEPTHWISE if path == "depthwise" else c2.PATH_DIRECT)
    for k, (N, C, H, W, Kh, Kw, S, P, D) in enumerate(DW_CASES):
        for epi in (0, 1, 3):
            x, w, b = ci.random_tensors(300 + k, N, C, H, W, C, Kh, Kw, C, mode=mode, bias=epi & 1)
            say(f"[sweep] {path} {mode} dw case {k} epi {epi}")
            y = run_nhwc(x, w, b, S, P, D, C, ci.BF16, epi)
            yref, s = oracle.conv2d(x, w, b, S, P, D, C, relu=bool(epi & 2))
            if mode == "int":
                np.testing.assert_array_equal(y, oracle.round_to_bf16(yref))
            else:
                check_bf16(y, yref, s, f"dw case {k}")


@pytest.mark.parametrize("mode", ["random", "int"])
def test_direct_fp32_sweep(mode):
    for k, (N, Cin, H, W, Cout, Kh, Kw, S, P, D, G) in enumerate(_sweep()[:24]):
        if oracle.out_dim(H, Kh, S, P, D) < 1 or oracle.out_dim(W, Kw, S, P, D) < 1:
            continue
        x, w, b = ci.random_tensors(500 + k, N, Cin, H, W, Cout, Kh, Kw, G, dtype=ci.F32, mode=mode)
        say(f"[sweep] fp32 {mode} case {k}")
        y = run_nhwc(x, w, b, S, P, D, G, ci.F32, 3)
        yref, s = oracle.conv2d(x, w, b, S, P, D, G, relu=True)
        if mode == "int":
            np.testing.assert_array_equal(y, yref)
        else:
            check_f32(y, yref, s, np.abs(b)[None, :, None, None].astype(np.float64), f"fp32 case {k}")


# 3x3 over at most four input channels per group (the unrolled small-K
# direct kernel): (N, Cin, H, W, Cout, S, P, D, G), ragged pixel counts,
# output channels not a multiple of the 8-channel block.
SMALL_K_CASES = [(1, 3, 17, 23, 32, 2, 1, 1, 1), (2, 1, 9, 8, 8, 1, 1, 1, 1), (1, 2, 12, 7, 20, 1, 0, 2, 1),
                 (1, 4, 15, 15, 16, 3, 2, 1, 1), (2, 4, 10, 11, 24, 1, 1, 1, 2), (1, 8, 9, 9, 16, 2, 1, 2, 4),
                 (1, 3, 1, 1, 12, 1, 1, 1, 1), (3, 3, 33, 31, 8, 2, 1, 1, 1)]


@pytest.mark.parametrize("dtype", [ci.F32, ci.BF16])
@pytest.mark.parametrize("mode", ["random", "int"])
def test_direct_small_k_sweep(dtype, mode):
    """The small-K direct kernel through both entries (NHWC packed, NCHW)."""
    c2.conv2d_set_path_override(c2.PATH_DIRECT)
    for k, (N, Cin, H, W, Cout, S, P, D, G) in enumerate(SMALL_K_CASES):
        for epi in (0, 1, 3):
            x, w, b = ci.random_tensors(700 + k, N, Cin, H, W, Cout, 3, 3, G, dtype=dtype, mode=mode,
                                        bias=epi & 1)
            yref, s = oracle.conv2d(x, w, b, S, P, D, G, relu=bool(epi & 2))
            for entry, run in (("nhwc", run_nhwc), ("nchw", run_nchw)):
                say(f"[sweep] small-K direct {entry} {dtype} {mode} case {k} epi {epi}")
                y = run(x, w, b, S, P, D, G, dtype, epi)
                if mode == "int":
                    want = yref if dtype == ci.F32 else oracle.round_to_bf16(yref)
                    np.testing.assert_array_equal(y, want)
                else:
                    _compare(y, yref, s, b, dtype, f"small-K {entry} case {k}")


# ------------------------------------------------------------------ NCHW entry

@pytest.mark.parametrize("cid,li", [(1, 0), (2, 0), (3, 0), (3, 1), (4, 0), (5, 3)])
def test_nchw_entry(cid, li):
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, **SMALL[(cid, li)])
    say(f"[parity] NCHW entry cfg{cid} {ly.name}")
    y = run_nchw(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    yref, s = _ref(x, w, b, ly)
    _compare(y, yref, s, b, ly.dtype, f"NCHW cfg{cid} {ly.name}")


def test_nchw_entry_full_first_layer():
    """The fp32 first layer at its full stated size, NCHW in and out."""
    ly = ci.layer(1, 0)
    x, w, b = ci.layer_tensors(1, 0)
    say("[parity] NCHW entry cfg1 full")
    y = run_nchw(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    yref, s = _ref(x, w, b, ly)
    assert y.shape == (1, 32, 112, 112)
    check_f32(y, yref, s, np.abs(b)[None, :, None, None].astype(np.float64), "cfg1 full NCHW")


def test_nchw_entry_two_streams():
    """The NCHW entry on two streams at once, each with its own input: every
    stream stages through its own scratch block, so the two never overwrite
    each other's repacked data; both results against the oracle."""
    from helpers import lib_dtype, to_dev
    N, Cin, H, W, Cout = 4, 64, 40, 40, 128
    xs, outs = [], []
    _, w, b = ci.random_tensors(7100, N, Cin, H, W, Cout, 3, 3, 1, bias=1)
    for k in range(2):
        x, _, _ = ci.random_tensors(7101 + k, N, Cin, H, W, Cout, 3, 3, 1, bias=1)
        xs.append(x)
    wd, bd = to_dev(w, ci.BF16), torch.from_numpy(np.asarray(b, np.float32)).cuda()
    xd = [to_dev(x, ci.BF16) for x in xs]
    yd = [torch.full((N, Cout, H, W), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say("[parity] NCHW entry on two streams")
    for rep in range(6):
        for k in range(2):
            c2.conv2d_fwd(xd[k], wd, bd, yd[k], N, Cin, H, W, Cout, 3, 3, 1, 1, 1, 1, lib_dtype(ci.BF16),
                          ci.EPI_BIAS | ci.EPI_RELU, stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        yref, sc = oracle.conv2d(xs[k], w, b, 1, 1, 1, 1, relu=True)
        check_bf16(yd[k].float().cpu().numpy().astype(np.float64), yref, sc, f"stream {k}")


def test_conv2d_log_names_the_path():
    """With CONV2D_LOG set, a forward call prints its shape and the kernel
    path it took (a child process: the switch is read once per process)."""
    import os
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    code = (f"import sys; sys.path.insert(0, {os.path.dirname(here)!r}); sys.path.insert(0, {here!r})\n"
            "import conv_inputs as ci\n"
            "from helpers import run_nhwc\n"
            "x, w, b = ci.random_tensors(1, 1, 64, 9, 9, 128, 3, 3, 1, bias=1)\n"
            "run_nhwc(x, w, b, 1, 1, 1, 1, ci.BF16, 3)\n")
    say("[parity] CONV2D_LOG child process")
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, CONV2D_LOG="1"), capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert ("conv2d: conv2d_fwd_nhwc_packed N=1 Cin=64 H=9 W=9 Cout=128 K=3x3 S=1 P=1 D=1 G=1 dtype=bf16 epi=3 "
            "-> igemm_halo") in r.stderr, r.stderr[-2000:]


# ------------------------------------------------------------------ repacks

@pytest.mark.parametrize("dtype", [ci.F32, ci.BF16])
# (channels and H*W multiples of 8 take the 8x8-block bf16 kernel, with full
# and partial 64x64 tiles; the others the LDS-tile kernel)
@pytest.mark.parametrize("shape", [(2, 3, 5, 7), (1, 144, 56, 56), (3, 65, 1, 130), (1, 1, 1, 1),
                                   (2, 40, 9, 24), (3, 256, 28, 28), (1, 8, 1, 8)])
def test_layout_repack_roundtrip(dtype, shape):
    from helpers import lib_dtype, to_dev
    rng = np.random.default_rng(1)
    a = ci.to_storage(rng.standard_normal(shape), dtype)
    N, C, H, W = shape
    say(f"[repack] {dtype} {shape}")
    src = to_dev(a, dtype)
    mid = torch.empty_like(src)
    back = torch.empty_like(src)
    c2.conv2d_nchw_to_nhwc(src, mid, N, C, H, W, lib_dtype(dtype))
    c2.conv2d_nhwc_to_nchw(mid, back, N, C, H, W, lib_dtype(dtype))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(mid.float().cpu().numpy().reshape(N, H, W, C), ci.nchw_to_nhwc(a))
    np.testing.assert_array_equal(back.float().cpu().numpy(), a)


def test_weight_pack_layouts():
    from helpers import pack_weights, to_dev
    rng = np.random.default_rng(2)
    w = ci.to_storage(rng.standard_normal((12, 4, 3, 2)), ci.BF16)
    wp = pack_weights(to_dev(w, ci.BF16), 12, 8, 3, 2, 2, ci.BF16).float().cpu().numpy()
    np.testing.assert_array_equal(wp.reshape(12, 3, 2, 4), w.transpose(0, 2, 3, 1))
    wd = ci.to_storage(rng.standard_normal((16, 1, 3, 3)), ci.BF16)
    wdp = pack_weights(to_dev(wd, ci.BF16), 16, 16, 3, 3, 16, ci.BF16).float().cpu().numpy()
    np.testing.assert_array_equal(wdp.reshape(3, 3, 16), wd[:, 0].transpose(1, 2, 0))


# ------------------------------------------------------------------ errors on GPU

def test_forced_path_that_cannot_run_is_an_error():
    x, w, b = ci.random_tensors(1, 1, 16, 8, 8, 16, 3, 3)
    c2.conv2d_set_path_override(c2.PATH_GEMM1X1)
    with pytest.raises(c2.Conv2dError) as e:
        run_nhwc(x, w, b, 1, 1, 1, 1, ci.BF16, 1)
    assert e.value.code == c2.ERR_UNSUPPORTED


def test_misaligned_pointer_is_rejected():
    from helpers import to_dev
    x, w, b = ci.random_tensors(1, 1, 16, 8, 8, 16, 3, 3)
    xd = to_dev(np.concatenate([np.zeros(1, np.float32), ci.nchw_to_nhwc(x).reshape(-1)]), ci.BF16)
    wd = to_dev(w.transpose(0, 2, 3, 1), ci.BF16)
    yd = torch.empty(1 * 8 * 8 * 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(c2.Conv2dError) as e:
        c2.conv2d_fwd_nhwc_packed(xd.data_ptr() + 2, wd, None, yd, 1, 16, 8, 8, 16, 3, 3, 1, 1, 1, 1,
                                  c2.BF16, 0)
    assert e.value.code == c2.ERR_ALIGN


def test_single_hip_runtime_in_process():
    """libconv2d.so and torch must share one HIP runtime (torch bundles its own
    under the same soname); two runtimes would not share devices or pointers."""
    libs = set()
    for ln in open("/proc/self/maps"):
        if "libamdhip64" in ln:
            libs.add(ln.split()[-1])
    assert len(libs) == 1, libs
    assert any("libconv2d.so" in ln for ln in open("/proc/self/maps"))
