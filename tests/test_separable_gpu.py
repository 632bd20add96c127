"""GPU parity of the fused depthwise-separable entry against the fp64 oracle.

The oracle is the block as the pages define it (lincklin.cn lesson 9,
section 25): 3x3 depthwise with bias and ReLU, the intermediate rounded to
bf16, then the 1x1 convolution.  Tolerances, element by element:
  random data       |y - yref| <= 1e-2 * S + 1e-3, S = sum_c |t_c * w_pw[co,c]|
                    (the kernel's intermediate may differ from the oracle's
                    by one bf16 step, 2**-8 relative, where the exact value
                    lies near a rounding boundary; that moves y by at most
                    0.4% of S, inside the bound)
  exact-integer     x in {-2..2}, weights in {-1,0,1}, integer biases: the
                    depthwise sums are small integers (exact in bf16), the
                    1x1 sums integers below 2**24, so y must equal
                    round-to-nearest-even(yref) bit for bit.
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import check_bf16, ensure_built, gpu_available, run_nhwc, run_separable

pytestmark = pytest.mark.gpu

if gpu_available():
    ensure_built()
    import torch
    import cnn_convolution_conv2d_amd as c2

B, R = ci.EPI_BIAS, ci.EPI_RELU


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _tensors(seed, N, C, H, W, Cout, dw_epi, pw_epi, mode):
    """Seeded block inputs with the depthwise-separable workload's
    distributions: x uniform[-1, 1], Kaiming-normal weights, biases N(0, 0.01)."""
    rng = np.random.default_rng(seed)
    if mode == "int":
        x = rng.integers(-2, 3, size=(N, C, H, W)).astype(np.float32)
        wdw = rng.integers(-1, 2, size=(C, 1, 3, 3)).astype(np.float32)
        wpw = rng.integers(-1, 2, size=(Cout, C, 1, 1)).astype(np.float32)
        bdw = rng.integers(-4, 5, size=C).astype(np.float32)
        bpw = rng.integers(-4, 5, size=Cout).astype(np.float32)
    else:
        x = ci.to_storage(rng.uniform(-1, 1, (N, C, H, W)), ci.BF16)
        wdw = ci.to_storage(rng.standard_normal((C, 1, 3, 3)) * np.sqrt(2 / 9), ci.BF16)
        wpw = ci.to_storage(rng.standard_normal((Cout, C, 1, 1)) * np.sqrt(2 / C), ci.BF16)
        bdw = (rng.standard_normal(C) * 0.01).astype(np.float32)
        bpw = (rng.standard_normal(Cout) * 0.01).astype(np.float32)
    return x, wdw, (bdw if dw_epi & B else None), wpw, (bpw if pw_epi & B else None)


def _check(y, x, wdw, bdw, wpw, bpw, stride, pad, dw_epi, pw_epi, mode, what):
    yref, s = oracle.separable(x, wdw, wpw, bdw, bpw, stride, pad, dw_relu=bool(dw_epi & R),
                               pw_relu=bool(pw_epi & R))
    assert y.shape == yref.shape, (y.shape, yref.shape)
    if mode == "int":
        np.testing.assert_array_equal(y, oracle.round_to_bf16(yref), err_msg=what)
    else:
        check_bf16(y, yref, s, what)


# (N, C, H, W, Cout, stride, pad, dw epilogue, pw epilogue): channel counts of
# the workload pair and ragged, chunked, strided and degenerate shapes
CASES = [
    (2, 144, 19, 21, 24, 1, 1, B | R, 0),    # the workload's channels, ragged bands and tiles
    (1, 8, 5, 7, 4, 1, 1, B | R, 0),         # fewest channels; Cout % 8 != 0 (8-byte stores)
    (2, 40, 9, 13, 36, 2, 1, B, B | R),      # stride 2; two output-channel blocks
    (1, 136, 6, 70, 20, 1, 1, B | R, B),     # wide rows split into column chunks; C % 16 == 8
    (1, 256, 7, 9, 128, 1, 1, R, B | R),     # widest input, four output blocks, one block per CU
    (1, 64, 11, 11, 64, 2, 0, 0, 0),         # no epilogues, no padding
    (2, 16, 3, 3, 8, 1, 2, B | R, R),        # padding 2: output larger than the input
    (1, 24, 1, 1, 12, 1, 1, B | R, 0),       # one-pixel image
    (3, 32, 33, 5, 96, 1, 1, B | R, B | R),  # tall and narrow; three of four output blocks used
]


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}c{c[1]}h{c[2]}w{c[3]}o{c[4]}s{c[5]}p{c[6]}" for c in CASES])
def test_separable_small(case, mode):
    N, C, H, W, Cout, stride, pad, dwe, pwe = case
    say(f"[separable] {case} {mode}")
    x, wdw, bdw, wpw, bpw = _tensors(hash(case) % 2**31, N, C, H, W, Cout, dwe, pwe, mode)
    y = run_separable(x, wdw, bdw, wpw, bpw, stride, pad, dwe, pwe)
    _check(y, x, wdw, bdw, wpw, bpw, stride, pad, dwe, pwe, mode, f"separable {case} {mode}")


def _workload(mode, **shrink):
    x, wdw, bdw = ci.layer_tensors(3, 0, mode=mode, **shrink)
    _, wpw, bpw = ci.layer_tensors(3, 1, N=1, H=1, W=1, mode=mode)
    return x, wdw, bdw, wpw, bpw


@pytest.mark.parametrize("mode", ["random", "int"])
def test_separable_workload_full_size(mode):
    """The depthwise-separable workload at full size (N=32, 144x56x56 ->
    24), every output compared, through the entry and launch the benchmark
    times."""
    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    x, wdw, bdw, wpw, bpw = _workload(mode)
    say(f"[separable] workload full size {mode} x{x.shape}")
    y = run_separable(x, wdw, bdw, wpw, bpw, dw.stride, dw.pad, dw.epilogue, pw.epilogue)
    _check(y, x, wdw, bdw, wpw, bpw, dw.stride, dw.pad, dw.epilogue, pw.epilogue, mode,
           f"separable workload {mode}")


def test_separable_equals_two_layer_chain():
    """At stride 1 the fused kernel does the two layers' arithmetic in the
    same order (bias-first depthwise sums, the same bf16 intermediate, the
    same matrix-op sequence), so its output equals the depthwise layer
    followed by the 1x1 layer through the per-layer entry, bit for bit."""
    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    x, wdw, bdw, wpw, bpw = _workload("random", N=2, H=23, W=25)
    say(f"[separable] fused vs two layers x{x.shape}")
    y = run_separable(x, wdw, bdw, wpw, bpw, dw.stride, dw.pad, dw.epilogue, pw.epilogue)
    t = run_nhwc(x, wdw, bdw, dw.stride, dw.pad, 1, dw.groups, ci.BF16, dw.epilogue)
    y2 = run_nhwc(t.astype(np.float32), wpw, bpw, 1, 0, 1, 1, ci.BF16, pw.epilogue)
    np.testing.assert_array_equal(y, y2)


def test_separable_repeat_calls_are_identical():
    """Two launches on the same inputs give the same bits (no state carried
    between calls)."""
    x, wdw, bdw, wpw, bpw = _workload("random", N=2, H=17, W=29)
    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    a = run_separable(x, wdw, bdw, wpw, bpw, dw.stride, dw.pad, dw.epilogue, pw.epilogue)
    b = run_separable(x, wdw, bdw, wpw, bpw, dw.stride, dw.pad, dw.epilogue, pw.epilogue)
    np.testing.assert_array_equal(a, b)
