"""GPU parity of the transposed convolution ("lpnh.cn/news/2674933" sections
2.3 and 4.2) against the fp64 oracle's scatter of W^T X, through the C ABI.

Tolerances, element by element, with S = sum |x w| of the products each
output receives (from the oracle):
  fp32  |y - yref| <= 1e-5 (S + |b|)
  bf16  |y - yref| <= 1e-2 S + 1e-3
  exact-integer mode (x in {-2..2}, w in {-1,0,1}, integer bias): every
  partial sum is an integer below 2^24, so the bf16 output equals
  round-to-nearest-even(yref) bit for bit.
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import check_bf16, check_f32, ensure_built, gpu_available, run_tnchw, run_tnhwc

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


def _tensors(seed, N, Cin, H, W, Cout, K, G, dtype, mode, bias=True):
    rng = np.random.default_rng(seed)
    xs, ws = (N, Cin, H, W), (Cin, Cout // G, K, K)
    if mode == "int":
        x = rng.integers(-2, 3, size=xs).astype(np.float32)
        w = rng.integers(-1, 2, size=ws).astype(np.float32)
        b = rng.integers(-4, 5, size=Cout).astype(np.float32)
    else:
        x = ci.to_storage(np.abs(rng.standard_normal(size=xs)), dtype)
        w = ci.to_storage(rng.standard_normal(size=ws) * np.sqrt(2.0 / (Cin // G * K * K / 4)), dtype)
        b = (rng.standard_normal(Cout) * 0.01).astype(np.float32)
    return x, w, (b if bias else None)


def _check(y, x, w, b, S, P, OP, D, G, dtype, epi, mode, what):
    yref, s = oracle.conv_transpose2d(x, w, b, S, P, OP, D, G, relu=bool(epi & ci.EPI_RELU))
    assert y.shape == yref.shape, what
    if mode == "int":
        want = yref if dtype == ci.F32 else oracle.round_to_bf16(yref)
        np.testing.assert_array_equal(y, want, err_msg=what)
    elif dtype == ci.F32:
        bb = 0.0 if b is None else np.abs(b.astype(np.float64))[None, :, None, None]
        check_f32(y, yref, s, bb, what)
    else:
        check_bf16(y, yref, s, what)


# (N, Cin, H, W, Cout, K, stride, pad, out_pad, dil, groups)
SWEEP = [
    (2, 32, 9, 11, 48, 4, 2, 1, 0, 1, 1),    # 2x upsampling, several tiles, ragged last tile
    (2, 64, 7, 6, 64, 2, 2, 0, 0, 1, 1),     # kernel = stride: one tap per phase
    (1, 16, 8, 7, 24, 3, 2, 1, 1, 1, 1),     # odd kernel: phases with 2 and 1 taps, output padding
    (1, 32, 5, 6, 40, 3, 3, 1, 2, 1, 2),     # stride 3, output padding 2, grouped
    (2, 24, 6, 6, 36, 3, 1, 1, 0, 1, 1),     # stride 1 (one phase: a flipped-kernel convolution)
    (1, 16, 6, 5, 16, 3, 2, 2, 1, 2, 2),     # dilation 2 with stride 2: only even taps per phase
    (1, 8, 5, 4, 12, 1, 2, 0, 1, 1, 1),      # 1x1 kernel at stride 2: odd outputs get the bias only
    (1, 16, 4, 4, 8, 5, 2, 3, 0, 1, 1),      # padding above the stride
    (1, 40, 6, 5, 132, 4, 2, 1, 1, 1, 1),    # Cout above one 128-channel tile, output padding
    (1, 8, 1, 1, 8, 3, 2, 0, 0, 1, 1),       # a single input pixel
]


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("path", ["phase_gemm", "direct"])
def test_transposed_sweep(path, mode):
    c2.conv2d_set_path_override(c2.PATH_IGEMM_GATHER if path == "phase_gemm" else c2.PATH_DIRECT)
    for k, (N, Cin, H, W, Cout, K, S, P, OP, D, G) in enumerate(SWEEP):
        for epi in (0, 3):
            x, w, b = _tensors(700 + k, N, Cin, H, W, Cout, K, G, ci.BF16, mode, bias=bool(epi & 1))
            say(f"[tconv] {path} {mode} case {k} {(N, Cin, H, W, Cout, K, S, P, OP, D, G)} epi {epi}")
            y = run_tnhwc(x, w, b, S, P, OP, D, G, ci.BF16, epi)
            _check(y, x, w, b, S, P, OP, D, G, ci.BF16, epi, mode, f"{path} case {k} epi {epi}")


# kernel == stride, no padding: (N, Cin, H, W, Cout, K=S)
SHUFFLE = [
    (2, 32, 9, 11, 64, 2),     # 256 GEMM rows, ragged last pixel tile
    (1, 16, 5, 7, 32, 2),      # 128 rows
    (1, 8, 4, 4, 32, 2),       # one 16-byte vector of input channels
    (2, 192, 4, 3, 32, 2),     # 12 channel slices
    (1, 64, 3, 5, 32, 4),      # stride 4: 16 taps, 512 rows > 256 -> not eligible (checked)
]


@pytest.mark.parametrize("mode", ["random", "int"])
def test_transposed_pixel_shuffle(mode):
    """The pointwise GEMM with pixel-shuffled output (forced), against the
    oracle; a shape it cannot take is refused when forced."""
    c2.conv2d_set_path_override(c2.PATH_GEMM1X1)
    ran = 0
    for k, (N, Cin, H, W, Cout, K) in enumerate(SHUFFLE):
        if Cout * K * K > 256:
            with pytest.raises(c2.Conv2dError):
                c2.conv2d_transpose_select_path(N, Cin, H, W, Cout, K, K, K, 0, 0, 1, 1, c2.BF16)
            continue
        for epi in (0, 3):
            x, w, b = _tensors(950 + k, N, Cin, H, W, Cout, K, 1, ci.BF16, mode, bias=bool(epi & 1))
            say(f"[tconv] pixel shuffle {mode} case {k} {(N, Cin, H, W, Cout, K)} epi {epi}")
            y = run_tnhwc(x, w, b, K, 0, 0, 1, 1, ci.BF16, epi)
            _check(y, x, w, b, K, 0, 0, 1, 1, ci.BF16, epi, mode, f"shuffle case {k} epi {epi}")
            ran += 1
    assert ran == 8


# stride 2, 4x4 kernel: (N, Cin, H, W, Cout, pad, out_pad)
HALO = [
    (2, 32, 9, 11, 48, 1, 0),     # several tiles' worth of rows, ragged columns, a partial channel group
    (1, 64, 17, 40, 32, 1, 1),    # two column tiles, output padding
    (1, 32, 5, 6, 36, 0, 0),      # padding 0: output 2H + 2
    (1, 32, 6, 5, 40, 2, 1),      # padding 2
    (2, 96, 4, 3, 8, 3, 0),       # padding 3, three channel chunks
    (1, 32, 1, 1, 4, 1, 0),       # a single input pixel
    (2, 160, 11, 37, 192, 1, 1),  # three channel blocks, the last half past Cin; three channel groups; two column tiles
    (1, 192, 9, 30, 72, 2, 1),    # three whole channel blocks; a partial second channel group
]


@pytest.mark.parametrize("mode", ["random", "int"])
def test_transposed_halo_window(mode):
    """All phases from one staged input window (forced), against the oracle;
    a shape it cannot take is refused when forced."""
    c2.conv2d_set_path_override(c2.PATH_IGEMM_HALO)
    for k, (N, Cin, H, W, Cout, P, OP) in enumerate(HALO):
        for epi in (0, 3):
            x, w, b = _tensors(980 + k, N, Cin, H, W, Cout, 4, 1, ci.BF16, mode, bias=bool(epi & 1))
            say(f"[tconv] halo window {mode} case {k} {(N, Cin, H, W, Cout, P, OP)} epi {epi}")
            y = run_tnhwc(x, w, b, 2, P, OP, 1, 1, ci.BF16, epi)
            _check(y, x, w, b, 2, P, OP, 1, 1, ci.BF16, epi, mode, f"halo case {k} epi {epi}")
    with pytest.raises(c2.Conv2dError):   # Cin not a multiple of 32
        c2.conv2d_transpose_select_path(1, 24, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16)


@pytest.mark.parametrize("mode", ["random", "int"])
def test_transposed_fp32_direct(mode):
    for k, (N, Cin, H, W, Cout, K, S, P, OP, D, G) in enumerate(SWEEP[:8]):
        x, w, b = _tensors(800 + k, N, min(Cin, 12), H, W, min(Cout, 12), K, 1, ci.F32, mode)
        say(f"[tconv] fp32 {mode} case {k}")
        y = run_tnhwc(x, w, b, S, P, OP, D, 1, ci.F32, 3)
        _check(y, x, w, b, S, P, OP, D, 1, ci.F32, 3, mode, f"fp32 case {k}")


@pytest.mark.parametrize("dtype", [ci.F32, ci.BF16])
def test_transposed_nchw_entry(dtype):
    """The pages' layouts: fp32 runs the direct kernel in place, bf16 goes
    through the repack and the phase GEMM."""
    x, w, b = _tensors(901, 2, 32, 7, 9, 48, 4, 2, ci.BF16, "random")
    x = ci.to_storage(x.astype(np.float64), dtype)
    w = ci.to_storage(w.astype(np.float64), dtype)
    say(f"[tconv] NCHW entry {dtype}")
    y = run_tnchw(x, w, b, 2, 1, 1, 1, 2, dtype, 3)
    _check(y, x, w, b, 2, 1, 1, 1, 2, dtype, 3, "random", f"nchw {dtype}")


LAYERS = [(6, 0), (6, 1)]


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("cid,li", LAYERS, ids=[ci.layer(c, l).name for c, l in LAYERS])
def test_workload_layer_reduced(cid, li, mode):
    """The decoder layers' channels, kernels and strides on a reduced batch
    and image (several tiles per phase, a ragged last tile)."""
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, N=2, H=ly.H // 2 + 1, W=ly.W // 2 - 1, mode=mode)
    say(f"[tconv] {ly.name} reduced {mode} x{x.shape}")
    want = c2.PATH_GEMM1X1 if ly.Kh == ly.stride and ly.pad == 0 else c2.PATH_IGEMM_HALO
    assert c2.conv2d_transpose_select_path(2, ly.Cin, x.shape[2], x.shape[3], ly.Cout, ly.Kh, ly.Kw, ly.stride,
                                           ly.pad, ly.out_pad, ly.dilation, ly.groups, c2.BF16) == want
    y = run_tnhwc(x, w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    _check(y, x, w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue, mode,
           f"{ly.name} reduced {mode}")


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("li", [0, 1])
def test_workload_layer_on_phase_gemm(li, mode):
    """Each decoder layer forced onto the phase-split gather GEMM (their
    automatic paths are the halo window and the pixel-shuffle GEMM)."""
    ly = ci.layer(6, li)
    x, w, b = ci.layer_tensors(6, li, N=2, H=15, W=13, mode=mode)
    c2.conv2d_set_path_override(c2.PATH_IGEMM_GATHER)
    say(f"[tconv] {ly.name} on the phase GEMM {mode}")
    y = run_tnhwc(x, w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    _check(y, x, w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue, mode,
           f"{ly.name} phase GEMM {mode}")


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("cid,li", LAYERS, ids=[ci.layer(c, l).name for c, l in LAYERS])
def test_workload_layer_full_size(cid, li, mode):
    """Full size, the entry and launch the benchmark times; every output
    element against the oracle's scatter form, a few images at a time."""
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, mode=mode)
    say(f"[tconv] {ly.name} full {mode} x{x.shape}")
    yd = run_tnhwc(x, w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue,
                   return_dev=True)
    assert not torch.isnan(yd.float()).any().item()
    N = yd.shape[0]
    step = 4
    for n0 in range(0, N, step):
        y = ci.nhwc_to_nchw(yd[n0:n0 + step].float().cpu().numpy()).astype(np.float64)
        yref, s = oracle.conv_transpose2d(x[n0:n0 + step], w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation,
                                          ly.groups, relu=bool(ly.epilogue & ci.EPI_RELU))
        if mode == "int":
            np.testing.assert_array_equal(y, oracle.round_to_bf16(yref), err_msg=f"images {n0}..")
        else:
            check_bf16(y, yref, s, f"{ly.name} full, images {n0}..")


def test_transposed_forced_path_that_cannot_run_is_an_error():
    c2.conv2d_set_path_override(c2.PATH_IGEMM_HALO)
    with pytest.raises(c2.Conv2dError):
        c2.conv2d_transpose_select_path(1, 16, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16)
    c2.conv2d_set_path_override(c2.PATH_IGEMM_GATHER)
    with pytest.raises(c2.Conv2dError):   # channels not a multiple of 8
        c2.conv2d_transpose_select_path(1, 12, 8, 8, 16, 4, 4, 2, 1, 0, 1, 1, c2.BF16)
