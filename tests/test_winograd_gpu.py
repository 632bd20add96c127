"""GPU parity of the Winograd F(2x2, 3x3) path ("lpnh.cn/news/2674933"
section 3.3; "lnrq.cn/news/4475" section 2.2) against the fp64 oracle's
direct convolution.  Winograd computes the convolution exactly in exact
arithmetic; its only roundings are the bf16 transformed input and filter,
the fp32 sums, and the final bf16 output.

Tolerances, element by element, S = sum |x w| over the valid taps:
  bf16 random data  |y - yref| <= 1e-2 S + 1e-3
  exact-integer mode (x in {-2..2}, w in {-1,0,1}, integer bias): the
  transformed input holds integers up to 8 and the transformed filter
  multiples of 1/4 up to 9/4 -- all exact in bf16 -- so every product and sum
  is a multiple of 1/4 far below 2^20, exact in fp32, and the output equals
  round-to-nearest-even(yref) bit for bit.
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import check_bf16, compare_full, ensure_built, gpu_available, run_winograd

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


# (N, Cin, H, W, Cout, pad, epilogue)
CASES = [
    (1, 16, 16, 16, 64, 1, 3),     # one workgroup exactly
    (2, 32, 19, 21, 72, 1, 3),     # ragged block groups and a partial 64-channel group
    (1, 8, 7, 9, 4, 0, 1),         # half a channel chunk, 4 output channels, odd output
    (1, 24, 33, 17, 100, 2, 2),    # padding 2, a channel chunk tail, Cout not a multiple of 64
    (2, 128, 23, 23, 256, 1, 3),   # the 3x3 workload's channels, reduced image
    (1, 16, 3, 3, 8, 0, 0),        # a single output
    (1, 16, 2, 2, 8, 1, 3),        # output smaller than one 2x2 block in neither direction
    (3, 40, 12, 5, 36, 1, 3),      # narrow image
]


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_winograd_matches_oracle(case, mode):
    N, Cin, H, W, Cout, P, epi = case
    x, w, b = ci.random_tensors(1100 + CASES.index(case), N, Cin, H, W, Cout, 3, 3, mode=mode, bias=bool(epi & 1))
    say(f"[wino] {case} {mode}")
    y = run_winograd(x, w, b, P, epi)
    yref, s = oracle.conv2d(x, w, b, 1, P, 1, 1, relu=bool(epi & 2))
    if mode == "int":
        np.testing.assert_array_equal(y, oracle.round_to_bf16(yref))
    else:
        worst = check_bf16(y, yref, s, f"winograd {case}")
        say(f"[wino]   worst |err| / tolerance = {worst:.3f}")


@pytest.mark.parametrize("mode", ["random", "int"])
def test_winograd_full_workload(mode):
    """The 3x3 workload layer (N=32, 128x112x112 -> 256, pad 1, bias+ReLU) at
    full size through the launch the benchmark times; every output element
    against the direct-loop oracle."""
    ly = ci.layer(2, 0)
    x, w, b = ci.layer_tensors(2, 0, mode=mode)
    say(f"[wino] full workload {mode}")
    yd = run_winograd(x, w, b, ly.pad, ly.epilogue, return_dev=True)
    assert not torch.isnan(yd.float()).any().item()
    worst = compare_full(yd, x, w, b, 1, ly.pad, 1, 1, True, ci.BF16, mode, "winograd full")
    say(f"[wino]   worst |err| / tolerance = {worst:.3f}")
