"""GPU parity of the folded batch-normalisation epilogue (bias, then the
per-channel scale and shift, then ReLU; lincklin.cn lesson 9, section 31)
against the fp64 oracle, on every kernel path and both entries.

Tolerances, element by element, with S' = |scale| (sum |x w| + |b|) + |shift|
from the oracle:
  fp32  |y - yref| <= 1e-5 * S'
  bf16  |y - yref| <= 1e-2 * S' + 1e-3
  exact-integer mode (x in {-2..2}, w in {-1,0,1}, integer bias, scale in
  {-2,-1,1,2}, integer shift): every step is exact in fp32, so the bf16
  output equals round-to-nearest-even(yref) bit for bit.
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import check_bf16, ensure_built, gpu_available, run_nchw, run_nhwc

pytestmark = pytest.mark.gpu

if gpu_available():
    ensure_built()
    import cnn_convolution_conv2d_amd as c2


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")
    yield
    c2.conv2d_set_path_override(c2.PATH_AUTO)


B, R = ci.EPI_BIAS, ci.EPI_RELU

# (name, path, dtype, N, Cin, H, W, Cout, K, stride, pad, dil, groups, epilogue)
CASES = [
    ("direct_f32", "PATH_DIRECT", ci.F32, 1, 3, 13, 11, 8, 3, 2, 1, 1, 1, B | R),
    ("direct_bf16_odd_c", "PATH_DIRECT", ci.BF16, 2, 6, 9, 9, 12, 3, 1, 1, 1, 1, B),
    ("depthwise_3x3", "PATH_DEPTHWISE", ci.BF16, 2, 24, 11, 13, 24, 3, 1, 1, 1, 24, B | R),
    ("depthwise_5x5_s2", "PATH_DEPTHWISE", ci.BF16, 1, 16, 12, 10, 16, 5, 2, 2, 1, 16, R),
    ("pointwise", "PATH_GEMM1X1", ci.BF16, 2, 48, 9, 11, 40, 1, 1, 0, 1, 1, B | R),
    ("pointwise_wide", "PATH_GEMM1X1", ci.BF16, 1, 64, 7, 9, 144, 1, 1, 0, 1, 1, B),
    ("gemm1x1_tiled", "PATH_GEMM1X1", ci.BF16, 1, 320, 9, 7, 96, 1, 1, 0, 1, 1, B | R),
    ("gather_s2", "PATH_IGEMM_GATHER", ci.BF16, 2, 32, 13, 11, 48, 3, 2, 1, 1, 1, B | R),
    ("gather_grouped", "PATH_IGEMM_GATHER", ci.BF16, 1, 64, 9, 9, 64, 3, 1, 1, 1, 2, 0),
    ("halo_3x3", "PATH_IGEMM_HALO", ci.BF16, 2, 32, 19, 21, 72, 3, 1, 1, 1, 1, B | R),
    ("halo_3x3_d2_g2", "PATH_IGEMM_HALO", ci.BF16, 1, 64, 17, 15, 80, 3, 1, 2, 2, 2, R),
    ("halo_5x5", "PATH_IGEMM_HALO", ci.BF16, 1, 16, 15, 17, 48, 5, 1, 2, 1, 1, B | R),
]


def _tensors(seed, dtype, N, Cin, H, W, Cout, K, groups, epi, mode):
    x, w, b = ci.random_tensors(seed, N, Cin, H, W, Cout, K, K, groups=groups, dtype=dtype, mode=mode,
                                bias=bool(epi & B))
    rng = np.random.default_rng(seed + 1)
    if mode == "int":
        scale = rng.choice([-2.0, -1.0, 1.0, 2.0], size=Cout).astype(np.float32)
        shift = rng.integers(-4, 5, size=Cout).astype(np.float32)
    else:
        scale = rng.uniform(0.5, 1.5, Cout).astype(np.float32) * rng.choice([-1.0, 1.0], size=Cout).astype(np.float32)
        shift = (rng.standard_normal(Cout) * 0.1).astype(np.float32)
    return x, w, b, scale, shift


def _check(y, x, w, b, scale, shift, stride, pad, dil, groups, dtype, epi, mode, what):
    yref, s = oracle.conv2d_bn(x, w, scale, shift, b, stride, pad, dil, groups, relu=bool(epi & R))
    if mode == "int":
        want = yref if dtype == ci.F32 else oracle.round_to_bf16(yref)
        np.testing.assert_array_equal(y, want, err_msg=what)
    elif dtype == ci.F32:
        err = np.abs(y - yref)
        assert np.all(err <= 1e-5 * s + 1e-30), f"{what}: worst err/S {float((err / s).max()):.3g}"
    else:
        check_bf16(y, yref, s, what)


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bn_epilogue_nhwc(case, mode):
    name, path, dtype, N, Cin, H, W, Cout, K, stride, pad, dil, groups, epi = case
    say(f"[bn] {name} {mode} (NHWC entry, {path})")
    x, w, b, scale, shift = _tensors(500 + CASES.index(case), dtype, N, Cin, H, W, Cout, K, groups, epi, mode)
    c2.conv2d_set_path_override(getattr(c2, path))
    y = run_nhwc(x, w, b, stride, pad, dil, groups, dtype, epi, scale=scale, shift=shift)
    _check(y, x, w, b, scale, shift, stride, pad, dil, groups, dtype, epi, mode, f"bn {name} {mode}")


@pytest.mark.parametrize("mode", ["random", "int"])
def test_bn_epilogue_nchw_entry(mode):
    """The NCHW entry: fp32 in place (direct) and bf16 through the repack."""
    for dtype, epi in ((ci.F32, B | R), (ci.BF16, B | R)):
        x, w, b, scale, shift = _tensors(7, dtype, 2, 32, 11, 13, 48, 3, 1, epi, mode)
        say(f"[bn] NCHW entry {dtype} {mode}")
        y = run_nchw(x, w, b, 1, 1, 1, 1, dtype, epi, scale=scale, shift=shift)
        _check(y, x, w, b, scale, shift, 1, 1, 1, 1, dtype, epi, mode, f"bn nchw {dtype} {mode}")


def test_bn_with_unit_scale_equals_plain_entry():
    """scale = 1, shift = 0 gives the plain entry's output bit for bit on the
    workload's 3x3 bias+ReLU layer (reduced size)."""
    ly = ci.layer(2, 0)
    x, w, b = ci.layer_tensors(2, 0, N=1, H=21, W=23)
    one, zero = np.ones(ly.Cout, np.float32), np.zeros(ly.Cout, np.float32)
    a = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue)
    bn = run_nhwc(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, ly.dtype, ly.epilogue, scale=one, shift=zero)
    np.testing.assert_array_equal(a, bn)
