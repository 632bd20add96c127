"""GPU parity of the persistent kernels' cross-tile schedule.

The halo-tile implicit GEMMs, the streaming 1x1 kernel and the fused
separable kernel launch at most as many workgroups as fit on the device and
walk their tiles in a grid-stride loop; while one tile finishes, the next
tile's weights, first halo chunk and bias are already being loaded.  That
hand-over only runs when a workgroup owns two or more tiles.  These tests
reach it two ways, and compare every output element with the fp64 oracle
(random data within the bf16 tolerance, exact-integer data bit for bit):

- small problems under a workgroup cap (conv2d_set_grid_limit), so each
  workgroup walks many tiles, with a partial last round and, for the unrolled
  3x3 kernel, the spread assignment of the last round's tiles;
- problems with more tiles than the device holds workgroups at once (no cap),
  at the launch configuration a caller gets.

The halo tile is the input block plus its (K-1)*D border staged once per
channel chunk and shared by all taps (lincklin.cn lesson 9, sections 12-13).
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import compare_full, ensure_built, gpu_available, run_nhwc, run_separable

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
    c2.conv2d_set_grid_limit(0)
    c2.conv2d_set_path_override(c2.PATH_AUTO)


def _check_path(case, want):
    """The path the calls of this case will take; a 3x3 stride-2 case is sent
    to the staged-window kernel by forcing the halo path (the automatic
    choice gives stride 2 to the gather kernel)."""
    N, Cin, H, W, Cout, Kh, Kw, S, P, D, G = case
    if want == c2.PATH_IGEMM_HALO and S == 2:
        c2.conv2d_set_path_override(c2.PATH_IGEMM_HALO)
    got = c2.conv2d_select_path(N, Cin, H, W, Cout, Kh, Kw, S, P, D, G, c2.BF16)
    assert got == want, f"{case}: path {c2.PATH_NAMES.get(got, got)}, expected {c2.PATH_NAMES[want]}"


def _run_case(case, mode, epi, seed, cap):
    N, Cin, H, W, Cout, Kh, Kw, S, P, D, G = case
    x, w, b = ci.random_tensors(seed, N, Cin, H, W, Cout, Kh, Kw, G, mode=mode, bias=epi & 1)
    prev = c2.conv2d_set_grid_limit(cap)
    try:
        yd = run_nhwc(x, w, b, S, P, D, G, ci.BF16, epi, return_dev=True)
    finally:
        c2.conv2d_set_grid_limit(prev)
    assert not torch.isnan(yd.float()).any().item()
    return compare_full(yd, x, w, b, S, P, D, G, bool(epi & 2), ci.BF16, mode, f"{case} cap {cap} {mode}")


HALO = "igemm_halo"
GEMM1X1 = "gemm1x1"

# (N, Cin, H, W, Cout, Kh, Kw, S, P, D, G), expected path, workgroup caps.
# Filters other than 3x3 (d1, d2) run the generic halo kernel (runtime tap
# loop); 3x3 runs the unrolled one.  Output-channel tiles are 128 wide when
# Cout/G > 64, else 64.
CAPPED = [
    # generic halo kernel: 5x5 (25 taps), 4x4, 5x3, 2x4 and 2x5; Cin/G not a
    # multiple of the 32-channel chunk; Cout/G not a multiple of the tile
    ((2, 64, 40, 36, 256, 5, 5, 1, 2, 1, 1), HALO, (1, 5, 16)),
    ((2, 32, 23, 29, 96, 4, 4, 1, 1, 1, 1), HALO, (1, 3, 8)),
    ((1, 48, 30, 45, 72, 5, 3, 1, 2, 1, 1), HALO, (2, 7)),
    ((2, 64, 17, 50, 64, 2, 4, 1, 1, 1, 1), HALO, (1, 6)),
    ((2, 48, 21, 26, 128, 2, 5, 1, 1, 1, 2), HALO, (3, 11)),
    # unrolled 3x3 kernel: 128- and 64-channel tiles, dilation 2 with
    # 128-channel tiles (5x5-span halo buffers), Cin/G % 32 != 0, the 8x32
    # pixel block, groups
    ((2, 128, 33, 40, 64, 3, 3, 1, 1, 1, 1), HALO, (4, 16)),
    ((2, 64, 30, 34, 256, 3, 3, 1, 2, 2, 2), HALO, (1, 9, 20, 32)),
    ((2, 256, 21, 19, 256, 3, 3, 1, 2, 2, 4), HALO, (5, 40)),
    ((2, 40, 25, 27, 128, 3, 3, 1, 1, 1, 1), HALO, (3, 8)),
    ((2, 72, 25, 27, 96, 3, 3, 1, 1, 1, 1), HALO, (2, 13)),
    ((2, 64, 8, 60, 128, 3, 3, 1, 1, 1, 1), HALO, (1, 3)),
    # 72 tiles of 128 channels x 16x16 pixels: a cap of 64 leaves a last
    # round of 8 tiles, which the spread assignment gives to every fourth
    # workgroup of each XCD; 40 leaves 32 (no spread); 27 is not a multiple
    # of 8 (plain round-robin)
    ((2, 64, 96, 96, 128, 3, 3, 1, 1, 1, 1), HALO, (27, 40, 64)),
    # two or four 128-channel tiles per pixel block: 36 tiles (2 images x 3 x
    # 3 blocks x 2), a last round of 1, 1, 4 and 12 tiles under caps 5, 7, 8
    # and 24, none under 12; dilation 2 with 256 channels per group (cap 40:
    # a last round of 8 tiles on 40 workgroups); Cin/G % 32 != 0; the 8x32
    # block (8 tiles, cap 7)
    ((2, 64, 37, 35, 256, 3, 3, 1, 1, 1, 1), HALO, (1, 5, 7, 8, 12, 24)),
    ((2, 64, 30, 34, 512, 3, 3, 1, 2, 2, 2), HALO, (1, 5, 8, 40)),
    ((4, 64, 8, 64, 128, 3, 3, 1, 1, 1, 1), HALO, (3, 7)),
    # one image of 3 x 3 blocks, two channel tiles: 18 tiles, a last round of
    # 3 or 2 tiles under caps 3 and 4
    ((1, 64, 37, 35, 256, 3, 3, 1, 1, 1, 1), HALO, (1, 3, 4)),
    ((2, 40, 25, 27, 256, 3, 3, 1, 1, 1, 1), HALO, (2, 3, 6)),
    ((1, 64, 20, 22, 512, 3, 3, 1, 1, 1, 1), HALO, (1, 3)),
    # 3x3 stride 2 on the phase-split window (4x32 pixel blocks; the halo
    # path forced): 128- and 64-channel tiles, ragged output channels,
    # Cin/G % 32 != 0, padding 0 and 2, groups, more than one 32-wide block
    # per row
    ((2, 64, 29, 57, 128, 3, 3, 2, 1, 1, 1), HALO, (1, 3)),
    ((2, 72, 30, 70, 96, 3, 3, 2, 1, 1, 1), HALO, (2, 5)),
    ((3, 64, 23, 40, 64, 3, 3, 2, 1, 1, 1), HALO, (1, 4)),
    ((2, 32, 21, 33, 48, 3, 3, 2, 0, 1, 1), HALO, (1, 3)),
    ((1, 64, 16, 16, 128, 3, 3, 2, 2, 1, 1), HALO, (1, 2)),
    ((2, 128, 20, 20, 256, 3, 3, 2, 1, 1, 2), HALO, (3, 7)),
    # streaming 1x1 kernel: half tiles (256 in), whole tiles (64 in, 144 in),
    # straight operand loads (40 in, 136 out)
    ((3, 256, 20, 23, 64, 1, 1, 1, 0, 1, 1), GEMM1X1, (1, 5)),
    ((3, 64, 20, 23, 256, 1, 1, 1, 0, 1, 1), GEMM1X1, (1, 7)),
    ((3, 144, 20, 21, 24, 1, 1, 1, 0, 1, 1), GEMM1X1, (2, 9)),
    ((2, 40, 17, 19, 136, 1, 1, 1, 0, 1, 1), GEMM1X1, (1, 4)),
]


def _id(c):
    case, path, caps = c
    N, Cin, H, W, Cout, Kh, Kw, S, P, D, G = case
    return f"{path}-n{N}c{Cin}h{H}w{W}o{Cout}k{Kh}x{Kw}p{P}d{D}g{G}"


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("spec", CAPPED, ids=[_id(c) for c in CAPPED])
def test_capped_grid(spec, mode):
    """Each workgroup walks several tiles; every element against the oracle."""
    case, path, caps = spec
    _check_path(case, getattr(c2, "PATH_" + path.upper()))
    for k, cap in enumerate(caps):
        epi = 3 if k % 2 == 0 else 1
        say(f"[multitile] {case} cap {cap} {mode} epi {epi}")
        worst = _run_case(case, mode, epi, 4000 + 17 * k + CAPPED.index(spec), cap)
        say(f"[multitile]   worst err/tol {worst:.3g}")


def test_capped_grid_matches_uncapped_bitwise():
    """The cap changes which workgroup computes a tile, not the arithmetic:
    capped and uncapped outputs are identical bit for bit."""
    case = (2, 64, 37, 35, 256, 3, 3, 1, 1, 1, 1)
    N, Cin, H, W, Cout, Kh, Kw, S, P, D, G = case
    x, w, b = ci.random_tensors(4242, N, Cin, H, W, Cout, Kh, Kw, G, bias=1)
    ref = run_nhwc(x, w, b, S, P, D, G, ci.BF16, 3)
    for cap in (1, 6, 50):
        c2.conv2d_set_grid_limit(cap)
        say(f"[multitile] bitwise cap {cap}")
        np.testing.assert_array_equal(run_nhwc(x, w, b, S, P, D, G, ci.BF16, 3), ref)
    c2.conv2d_set_grid_limit(0)


# More tiles than resident workgroups (two per CU on 256 CUs): each workgroup
# walks two or three tiles at the launch a caller gets.
NATURAL = [
    # generic kernel, 5x5: 10 images x 64 blocks x 2 channel tiles = 1280 tiles
    (10, 64, 128, 128, 256, 5, 5, 1, 2, 1, 1),
    # unrolled 3x3, dilation 2, 128 channels per group: 10 x 64 x 2 groups
    (10, 64, 128, 128, 256, 3, 3, 1, 2, 2, 2),
    # unrolled 3x3, 72 input channels (chunks of 32, 32, 8): 20 x 64 tiles
    (20, 72, 128, 128, 128, 3, 3, 1, 1, 1, 1),
    # the 3x3 workload's shape at 6 images: 6 x 49 blocks x 2 channel tiles
    (6, 64, 112, 112, 256, 3, 3, 1, 1, 1, 1),
    # 3x3 stride 2, 128 -> 128 at 56x56 -> 28x28: 80 images x 7 blocks
    (80, 128, 56, 56, 128, 3, 3, 2, 1, 1, 1),
]


@pytest.mark.parametrize("mode", ["random", "int"])
@pytest.mark.parametrize("case", NATURAL, ids=[f"n{c[0]}c{c[1]}o{c[4]}k{c[5]}s{c[7]}d{c[9]}g{c[10]}" for c in NATURAL])
def test_more_tiles_than_workgroups(case, mode):
    _check_path(case, c2.PATH_IGEMM_HALO)
    say(f"[multitile] natural {case} {mode}")
    worst = _run_case(case, mode, 3, 5000 + NATURAL.index(case), 0)
    say(f"[multitile]   worst err/tol {worst:.3g}")


@pytest.mark.parametrize("mode", ["random", "int"])
def test_separable_capped_grid(mode):
    """The fused separable kernel with each workgroup walking several bands."""
    N, C, H, W, Cout = 2, 144, 29, 31, 24
    rng = np.random.default_rng(4321 if mode == "random" else 4322)
    if mode == "int":
        x = rng.integers(-2, 3, size=(N, C, H, W)).astype(np.float32)
        wdw = rng.integers(-1, 2, size=(C, 1, 3, 3)).astype(np.float32)
        wpw = rng.integers(-1, 2, size=(Cout, C, 1, 1)).astype(np.float32)
        bdw = rng.integers(-4, 5, size=C).astype(np.float32)
    else:
        x = ci.to_storage(rng.uniform(-1, 1, (N, C, H, W)), ci.BF16)
        wdw = ci.to_storage(rng.standard_normal((C, 1, 3, 3)) * np.sqrt(2 / 9), ci.BF16)
        wpw = ci.to_storage(rng.standard_normal((Cout, C, 1, 1)) * np.sqrt(2 / C), ci.BF16)
        bdw = (rng.standard_normal(C) * 0.01).astype(np.float32)
    yref, s = oracle.separable(x, wdw, wpw, bdw, None, 1, 1, dw_relu=True, pw_relu=False)
    for cap in (1, 3, 10):
        c2.conv2d_set_grid_limit(cap)
        say(f"[multitile] separable cap {cap} {mode}")
        y = run_separable(x, wdw, bdw, wpw, None, 1, 1, ci.EPI_BIAS | ci.EPI_RELU, 0)
        if mode == "int":
            np.testing.assert_array_equal(y, oracle.round_to_bf16(yref))
        else:
            from helpers import check_bf16
            check_bf16(y, yref, s, f"separable cap {cap}")
    c2.conv2d_set_grid_limit(0)
