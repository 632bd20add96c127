"""Pins of the fp64 oracle to facts the pages and mathematics fix (CPU only).

Each test ties the oracle to something other than itself: a matrix or a shape
the pages print, a closed form, a library routine (torch CPU float64), or an
independent formulation (explicit im2col x GEMM).  The planted-mistake tests
at the end build mutated copies of the oracle source and check that these pins
reject each mutation.
"""
import json
import math
import os
import re
import shutil
import tempfile

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import conv_inputs as ci
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FIG = json.load(open(os.path.join(GOLDEN, "page_figures.json")))


def _torch_conv(x, w, b, stride, pad, dil, groups, relu=False):
    y = F.conv2d(torch.from_numpy(np.asarray(x, np.float64)), torch.from_numpy(np.asarray(w, np.float64)),
                 None if b is None else torch.from_numpy(np.asarray(b, np.float64)),
                 stride=stride, padding=pad, dilation=dil, groups=groups)
    if relu:
        y = torch.relu(y)
    return y.numpy()


# ------------------------------------------------------------- p1: im2col matrix

def test_p1_im2col_matches_printed_matrix():
    """3x3 input a..i, 2x2 kernel, stride 1 -> the 4x4 X_col printed on the
    lincklin.cn page, section 8.  Entries are distinct powers of two so each
    cell identifies exactly one input symbol."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "im2col_3x3_input_2x2_kernel.txt"))
            if ln.strip() and not ln.startswith("#")]
    sym = "abcdefghi"
    val = {s: float(2 ** i) for i, s in enumerate(sym)}
    x = np.array([val[s] for s in sym]).reshape(1, 1, 3, 3)
    xcol = oracle.im2col(x, 2, 2, stride=1, pad=0)
    expect = np.array([[val[s] for s in r] for r in rows])
    assert xcol.shape == (4, 4)
    np.testing.assert_array_equal(xcol, expect)
    # columns are windows: column j is window j flattened row-major
    np.testing.assert_array_equal(xcol[:, 0], [val[s] for s in "abde"])
    np.testing.assert_array_equal(xcol[:, 3], [val[s] for s in "efhi"])


# ------------------------------------------------------------- p2: small case

def test_p2_small_im2col_shapes_and_gemm_equivalence():
    f = FIG["small_im2col"]
    rng = np.random.default_rng(7)
    x = rng.integers(-3, 4, size=(1, f["C"], f["H"], f["W"])).astype(np.float64)
    w = rng.integers(-3, 4, size=(1, f["C"], f["K"], f["K"])).astype(np.float64)
    xcol = oracle.im2col(x, f["K"], f["K"], f["stride"], f["pad"])
    assert xcol.shape == (f["xcol_rows"], f["xcol_cols"])
    y, _ = oracle.conv2d(x, w, stride=f["stride"], pad=f["pad"])
    assert y.shape[2:] == (f["Ho"], f["Wo"])
    # direct loop == W_row @ X_col exactly on integer data (lpnh.cn section 3.1)
    np.testing.assert_array_equal(y.reshape(-1), (w.reshape(1, -1) @ xcol).reshape(-1))
    # each column is the flattened window at that output position
    np.testing.assert_array_equal(xcol[:, 1], x[0, 0, 0:3, 1:4].reshape(-1))
    np.testing.assert_array_equal(xcol[:, 2], x[0, 0, 1:4, 0:3].reshape(-1))


# ------------------------------------------------------------- p3: first layer

def test_p3_first_layer_shape_and_impulse_response():
    """224x224x3 -> 112x112x32, stride 2, pad 1 (lpnh.cn section 2.1).
    A unit impulse at input (c=1, h=113, w=57) reaches exactly the outputs
    whose window covers it, each with the weight of the covering tap:
    2*ho + kh - 1 = 113 and 2*wo + kw - 1 = 57."""
    f = FIG["first_layer"]
    x = np.zeros((1, f["Cin"], f["H"], f["W"]))
    x[0, 1, 113, 57] = 1.0
    rng = np.random.default_rng(3)
    w = rng.standard_normal((f["Cout"], f["Cin"], f["K"], f["K"]))
    y, s = oracle.conv2d(x, w, stride=f["stride"], pad=f["pad"])
    assert y.shape == (1, f["Cout"], f["Ho"], f["Wo"])
    expect = np.zeros_like(y)
    # 2*57 + 0 - 1 = 113, 2*56 + 2 - 1 = 113; 2*29 + 0 - 1 = 57, 2*28 + 2 - 1 = 57
    expect[0, :, 57, 29] = w[:, 1, 0, 0]
    expect[0, :, 57, 28] = w[:, 1, 0, 2]
    expect[0, :, 56, 29] = w[:, 1, 2, 0]
    expect[0, :, 56, 28] = w[:, 1, 2, 2]
    np.testing.assert_array_equal(y, expect)


def test_p3_first_layer_single_point_hand_check():
    """The page computes one output by hand: the 27 input values of the 3x3
    neighbourhood over 3 channels times the 27 weights, summed, plus the bias.
    Interior point (ho, wo) = (56, 56): window rows/cols 111..113."""
    x, w, b = ci.layer_tensors(1, 0)
    y, s = oracle.conv2d(x, w, b, stride=2, pad=1)
    for co in (0, 13, 31):
        terms = [float(x[0, c, 111 + dh, 111 + dw]) * float(w[co, c, dh, dw])
                 for c in range(3) for dh in range(3) for dw in range(3)]
        assert len(terms) == FIG["first_layer"]["products_per_output"]
        hand = math.fsum(terms) + float(b[co])
        assert abs(y[0, co, 56, 56] - hand) <= 1e-14 * (s[0, co, 56, 56] + abs(b[co]))


def test_p3_corner_and_far_edge_tap_counts():
    """With |x| = |w| = 1, S counts the valid taps: the (0,0) corner of the
    stride-2 pad-1 layer sees 2x2 taps per channel (12), and the last output
    row/col never reads the bottom/right padding (last hi = 2*111 + 2 - 1 = 223)."""
    x = np.ones((1, 3, 224, 224))
    w = np.ones((32, 3, 3, 3))
    _, s = oracle.conv2d(x, w, stride=2, pad=1)
    assert s[0, 0, 0, 0] == 12
    assert s[0, 0, 111, 111] == 27
    assert s[0, 0, 0, 111] == 18


# ------------------------------------------------------------- p4: tap counts

@pytest.mark.parametrize("entry", FIG["macs_per_output"], ids=lambda e: str(e["macs"]))
def test_p4_macs_per_interior_output(entry):
    Cin, K = entry["Cin"], entry["K"]
    x = np.ones((1, Cin, 5, 5))
    w = -np.ones((2, Cin, K, K))
    y, s = oracle.conv2d(x, w, stride=1, pad=1)
    assert s[0, 0, 2, 2] == entry["macs"]
    assert y[0, 1, 2, 2] == -entry["macs"]


# ------------------------------------------------------------- p5: output size

def test_p5_output_sizes():
    assert oracle.out_dim(224, 3, 2, 1, 1) == FIG["first_layer"]["Ho"]
    assert oracle.out_dim(4, 3, 1, 0, 1) == FIG["small_im2col"]["Ho"]
    assert oracle.out_dim(3, 2, 1, 0, 1) == 2            # lincklin.cn section 8 example
    d = FIG["dilation"]
    assert oracle.effective_kernel(d["K"], d["dilation"]) == d["K_eff"]
    # a dilated 3x3 spans exactly as far as a 5x5: identical output sizes
    for n in (5, 6, 7, 64, 65):
        for s in (1, 2, 3):
            for p in (0, 1, 2):
                assert oracle.out_dim(n, 3, s, p, 2) == oracle.out_dim(n, 5, s, p, 1)
    # the workloads' output sizes (the first is stated as 1x32x112x112)
    expected = {(1, 0): 112, (2, 0): 112, (3, 0): 56, (3, 1): 56, (4, 0): 64,
                (5, 0): 56, (5, 1): 56, (5, 2): 56, (5, 3): 28}
    for (cid, li), ho in expected.items():
        ly = ci.layer(cid, li)
        assert oracle.out_dim(ly.H, ly.Kh, ly.stride, ly.pad, ly.dilation) == ho
    # too-small inputs give an empty output, which the oracle rejects
    assert oracle.out_dim(2, 3, 1, 0, 1) <= 0
    assert oracle.out_dim(3, 3, 1, 0, 2) <= 0
    with pytest.raises(ValueError):
        oracle.conv2d(np.ones((1, 1, 2, 2)), np.ones((1, 1, 3, 3)))


def test_p5_floor_division():
    # (7 + 2 - 2 - 1)/2 = 3 -> 4 outputs; (6 + 0 - 2 - 1)/2 = 1.5 -> floor 1 -> 2 outputs
    assert oracle.out_dim(7, 3, 2, 1, 1) == 4
    assert oracle.out_dim(6, 3, 2, 0, 1) == 2
    assert oracle.out_dim(9, 3, 3, 0, 1) == 3
    assert oracle.out_dim(10, 3, 3, 0, 1) == 3


# ------------------------------------------------------------- p6: dilation

@pytest.mark.parametrize("dil,pad,stride", [(2, 2, 1), (2, 0, 1), (3, 1, 2), (2, 1, 2)])
def test_p6_dilation_equals_zero_inserted_kernel(dil, pad, stride):
    """A dilated KxK filter is a K_eff x K_eff filter with zeros between taps
    (lpnh.cn section 4.2); on integer data the results agree exactly."""
    rng = np.random.default_rng(11)
    x = rng.integers(-3, 4, size=(2, 4, 13, 11)).astype(np.float64)
    w = rng.integers(-3, 4, size=(6, 2, 3, 3)).astype(np.float64)
    ke = oracle.effective_kernel(3, dil)
    we = np.zeros((6, 2, ke, ke))
    we[:, :, ::dil, ::dil] = w
    y1, s1 = oracle.conv2d(x, w, stride=stride, pad=pad, dilation=dil, groups=2)
    y2, _ = oracle.conv2d(x, we, stride=stride, pad=pad, dilation=1, groups=2)
    np.testing.assert_array_equal(y1, y2)
    # only the K*K taps are gathered: S counts at most 2*9 products per output
    xs = np.ones_like(x)
    _, s3 = oracle.conv2d(xs, np.ones_like(w), stride=stride, pad=pad, dilation=dil, groups=2)
    assert s3.max() == 2 * FIG["dilation"]["valid_taps"]


# ------------------------------------------------------------- p7: groups

@pytest.mark.parametrize("G", [2, 4])
def test_p7_groups_equal_independent_convs(G):
    rng = np.random.default_rng(5)
    Cin, Cout = 8, 12
    x = rng.standard_normal((2, Cin, 9, 10))
    w = rng.standard_normal((Cout, Cin // G, 3, 3))
    b = rng.standard_normal(Cout)
    y, _ = oracle.conv2d(x, w, b, stride=1, pad=1, groups=G, relu=True)
    ci_g, co_g = Cin // G, Cout // G
    parts = [oracle.conv2d(x[:, g * ci_g:(g + 1) * ci_g], w[g * co_g:(g + 1) * co_g],
                           b[g * co_g:(g + 1) * co_g], stride=1, pad=1, relu=True)[0]
             for g in range(G)]
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=1))


# ------------------------------------------------------------- p8: depthwise

def test_p8_depthwise_is_per_channel_conv():
    rng = np.random.default_rng(8)
    C = 6
    x = rng.standard_normal((2, C, 8, 7))
    wdw = rng.standard_normal((C, 1, 3, 3))
    y, _ = oracle.conv2d(x, wdw, stride=1, pad=1, groups=C)
    for c in range(C):
        yc, _ = oracle.conv2d(x[:, c:c + 1], wdw[c:c + 1], stride=1, pad=1)
        np.testing.assert_array_equal(y[:, c:c + 1], yc)


def test_p8_separable_equals_factorised_standard_conv():
    """Depthwise then pointwise (lnrq.cn section 3.1, no nonlinearity between)
    is one standard conv whose weight factorises W[co,ci,kh,kw] =
    Wpw[co,ci] * Wdw[ci,kh,kw] (linearity)."""
    rng = np.random.default_rng(9)
    Cin, Cout = 5, 7
    x = rng.integers(-3, 4, size=(2, Cin, 9, 8)).astype(np.float64)
    wdw = rng.integers(-3, 4, size=(Cin, 1, 3, 3)).astype(np.float64)
    wpw = rng.integers(-3, 4, size=(Cout, Cin, 1, 1)).astype(np.float64)
    t, _ = oracle.conv2d(x, wdw, stride=2, pad=1, groups=Cin)
    y, _ = oracle.conv2d(t, wpw)
    wstd = wpw[:, :, 0, 0][:, :, None, None] * wdw[:, 0][None, :, :, :]
    y2, _ = oracle.conv2d(x, wstd, stride=2, pad=1)
    np.testing.assert_array_equal(y, y2)


# ------------------------------------------------------------- p8: the separable block

@pytest.mark.parametrize("v,want", [
    (1 + 2.0**-8, 1.0),                       # midpoint of 1 and 1 + 2**-7: ties to the even 1
    (1 + 3 * 2.0**-8, 1 + 2.0**-6),           # midpoint of 1 + 2**-7 and 1 + 2**-6: even is 1 + 2**-6
    (1 + 2.0**-8 + 2.0**-30, 1 + 2.0**-7),    # a hair above the midpoint rounds up (one rounding)
    (-(1 + 2.0**-8 + 2.0**-30), -(1 + 2.0**-7)),
    (3.0, 3.0), (0.0, 0.0), (-0.0, -0.0),
    (2.0**-130, 2.0**-130),                   # subnormal, a multiple of the spacing 2**-133
    (2.0**-134, 0.0), (3 * 2.0**-134, 2.0**-132),  # subnormal ties to even
    ((2 - 2.0**-7) * 2.0**127, (2 - 2.0**-7) * 2.0**127),  # largest finite bf16
    ((2 - 2.0**-8) * 2.0**127, math.inf),     # its upper midpoint ties to the even 2**128: overflow
])
def test_bf16_round_cases(v, want):
    """bf16 keeps 8 significant bits and fp32's exponent range; rounding is to
    nearest, ties to even, taken once from the exact value."""
    got = float(oracle.bf16_round(np.array([v]))[0])
    assert got == want and math.copysign(1, got) == math.copysign(1, want), (v, got, want)


def test_bf16_round_agrees_with_bit_level_rounding_on_fp32_values():
    """On fp32 values the fp64 rounding equals the bit-level fp32 -> bf16
    rounding of the input generator (an independent formulation)."""
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000)).astype(np.float32)
    a = a[np.isfinite(a)]
    want = ci.bf16_bits_to_f32(ci.f32_to_bf16_bits(a)).astype(np.float64)
    np.testing.assert_array_equal(oracle.bf16_round(a.astype(np.float64)), want)


@pytest.mark.parametrize("stride,pad,dw_relu,pw_relu", [(1, 1, True, False), (2, 1, True, True),
                                                        (1, 0, False, True), (2, 2, True, False)])
def test_p8_separable_block_matches_torch(stride, pad, dw_relu, pw_relu):
    """The block composed from torch's own float64 convolutions: depthwise
    (groups = C) + bias, ReLU, bf16 rounding of the intermediate, then the
    1x1 convolution + bias (and ReLU)."""
    rng = np.random.default_rng(20 + 4 * stride + pad)
    N, C, H, W, Cout = 2, 16, 9, 11, 12
    x = ci.to_storage(rng.uniform(-1, 1, (N, C, H, W)), ci.BF16)
    wdw = ci.to_storage(rng.standard_normal((C, 1, 3, 3)) * 0.47, ci.BF16)
    bdw = rng.standard_normal(C) * 0.01
    wpw = ci.to_storage(rng.standard_normal((Cout, C, 1, 1)) * 0.35, ci.BF16)
    bpw = rng.standard_normal(Cout) * 0.01
    y, s = oracle.separable(x, wdw, wpw, bdw, bpw, stride, pad, dw_relu=dw_relu, pw_relu=pw_relu)
    t = _torch_conv(x, wdw, bdw, stride, pad, 1, C, relu=dw_relu)
    yt = _torch_conv(oracle.bf16_round(t), wpw, bpw, 1, 0, 1, 1, relu=pw_relu)
    assert y.shape == (N, Cout, (H + 2 * pad - 3) // stride + 1, (W + 2 * pad - 3) // stride + 1)
    np.testing.assert_allclose(y, yt, rtol=0, atol=1e-12 * float(s.max()))
    # S is the sum of |t * w_pw| over the C products of each output
    st = _torch_conv(np.abs(oracle.bf16_round(t)), np.abs(wpw), None, 1, 0, 1, 1)
    np.testing.assert_allclose(s, st, rtol=1e-12)


def test_p8_separable_block_without_relu_is_a_factorised_conv():
    """On integers (the bf16 rounding is exact) and with no ReLU the block is
    one standard convolution with W[co,c,kh,kw] = w_pw[co,c] * w_dw[c,kh,kw]
    and bias b_pw + w_pw @ b_dw."""
    rng = np.random.default_rng(21)
    C, Cout = 6, 5
    x = rng.integers(-2, 3, size=(2, C, 8, 9)).astype(np.float64)
    wdw = rng.integers(-1, 2, size=(C, 1, 3, 3)).astype(np.float64)
    wpw = rng.integers(-1, 2, size=(Cout, C, 1, 1)).astype(np.float64)
    bdw = rng.integers(-4, 5, size=C).astype(np.float64)
    bpw = rng.integers(-4, 5, size=Cout).astype(np.float64)
    for stride in (1, 2):
        y, _ = oracle.separable(x, wdw, wpw, bdw, bpw, stride, 1, dw_relu=False, pw_relu=False)
        wstd = wpw[:, :, 0, 0][:, :, None, None] * wdw[:, 0][None, :, :, :]
        # the depthwise bias is added after its sum, so it reaches every
        # output as w_pw @ b_dw
        yb, _ = oracle.conv2d(x, wstd, bpw + wpw[:, :, 0, 0] @ bdw, stride, 1)
        np.testing.assert_array_equal(y, yb)


# ------------------------------------------------------------- folded batch normalisation

@pytest.mark.parametrize("relu,with_bias,groups", [(True, True, 1), (False, True, 2), (True, False, 1)])
def test_bn_epilogue_matches_torch_batch_norm(relu, with_bias, groups):
    """conv (+ bias), then torch's own batch normalisation in inference mode,
    then ReLU, against the oracle given the folded per-channel scale and
    shift: scale = gamma / sqrt(var + eps), shift = beta - mean * scale."""
    rng = np.random.default_rng(31 + groups + 2 * relu)
    N, Cin, H, W, Cout = 2, 8, 9, 7, 6
    x = rng.standard_normal((N, Cin, H, W))
    w = rng.standard_normal((Cout, Cin // groups, 3, 3)) * 0.3
    b = rng.standard_normal(Cout) * 0.1 if with_bias else None
    mean, var = rng.standard_normal(Cout), rng.uniform(0.2, 2.0, Cout)
    gamma, beta, eps = rng.standard_normal(Cout), rng.standard_normal(Cout), 1e-5
    scale = gamma / np.sqrt(var + eps)
    shift = beta - mean * scale
    y, s = oracle.conv2d_bn(x, w, scale, shift, b, 1, 1, 1, groups, relu=relu)
    t = F.conv2d(torch.from_numpy(x), torch.from_numpy(w), None if b is None else torch.from_numpy(b),
                 padding=1, groups=groups)
    t = F.batch_norm(t, torch.from_numpy(mean), torch.from_numpy(var), torch.from_numpy(gamma),
                     torch.from_numpy(beta), training=False, eps=eps)
    if relu:
        t = torch.relu(t)
    np.testing.assert_allclose(y, t.numpy(), rtol=0, atol=1e-12 * float(s.max()))
    # the tolerance scale: |scale| (sum |x w| + |b|) + |shift|
    s0 = _torch_conv(np.abs(x), np.abs(w), None, 1, 1, 1, groups)
    bb = 0 if b is None else np.abs(b)[None, :, None, None]
    np.testing.assert_allclose(s, np.abs(scale)[None, :, None, None] * (s0 + bb) + np.abs(shift)[None, :, None, None],
                               rtol=1e-12)


# ------------------------------------------------------------- p9: 1x1 = GEMM

def test_p9_pointwise_is_gemm():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 16, 7, 9))
    w = rng.standard_normal((24, 16, 1, 1))
    b = rng.standard_normal(24)
    y, s = oracle.conv2d(x, w, b)
    for n in range(3):
        g = w[:, :, 0, 0] @ x[n].reshape(16, -1) + b[:, None]
        assert np.all(np.abs(y[n].reshape(24, -1) - g) <= 1e-12 * (s[n].reshape(24, -1) + 1))


# ------------------------------------------------------------- p10: padding

def test_p10_all_ones_input_border_closed_form():
    """All-ones input (lpnh.cn section 6.4): each output is the bias plus the
    sum of the weights whose tap lands inside the image; at a 3x3 pad-1 border
    the zero ring removes a row and/or column of the filter (lincklin.cn
    section 26)."""
    rng = np.random.default_rng(12)
    w = rng.integers(-5, 6, size=(1, 1, 3, 3)).astype(np.float64)
    b = np.array([0.5])
    y, _ = oracle.conv2d(np.ones((1, 1, 5, 6)), w, b, stride=1, pad=1)
    k = w[0, 0]
    Y = y[0, 0] - 0.5
    assert Y[0, 0] == k[1:, 1:].sum() and Y[0, 5] == k[1:, :2].sum()
    assert Y[4, 0] == k[:2, 1:].sum() and Y[4, 5] == k[:2, :2].sum()
    assert Y[0, 3] == k[1:, :].sum() and Y[4, 2] == k[:2, :].sum()
    assert Y[2, 0] == k[:, 1:].sum() and Y[1, 5] == k[:, :2].sum()
    assert np.all(Y[1:4, 1:5] == k.sum())


def test_p10_dilated_border_closed_form():
    """Dilation 2, pad 2: the zero border is two pixels thick, and a border
    output loses the whole first (or last) tap row/column."""
    rng = np.random.default_rng(13)
    w = rng.integers(-5, 6, size=(1, 1, 3, 3)).astype(np.float64)
    y, _ = oracle.conv2d(np.ones((1, 1, 8, 8)), w, stride=1, pad=2, dilation=2)
    k, Y = w[0, 0], y[0, 0]
    for i in (0, 1):
        assert Y[i, 4] == k[1:, :].sum() and Y[4, i] == k[:, 1:].sum()
        assert Y[7 - i, 4] == k[:2, :].sum() and Y[4, 7 - i] == k[:, :2].sum()
    assert Y[0, 0] == k[1:, 1:].sum() and Y[1, 7] == k[1:, :2].sum()
    assert np.all(Y[2:6, 2:6] == k.sum())


# ------------------------------------------------------------- p11: sweep

def _sweep_cases():
    cases = []
    rng = np.random.default_rng(2024)
    for S in (1, 2, 3):
        for P in (0, 1, 2):
            for D in (1, 2, 3):
                for K in (1, 2, 3, 5):
                    Gs = (1, 2, 4)
                    G = Gs[int(rng.integers(0, 3))]
                    H = int(rng.integers(5, 12)) | 1
                    W = int(rng.integers(4, 13))
                    cases.append((S, P, D, K, G, H, W))
    return cases


def test_p11_direct_equals_im2col_gemm_and_torch_sweep():
    rng = np.random.default_rng(99)
    checked = 0
    for S, P, D, K, G, H, W in _sweep_cases():
        Kh, Kw = K, max(1, K - 1) if K > 2 else K
        if oracle.out_dim(H, Kh, S, P, D) < 1 or oracle.out_dim(W, Kw, S, P, D) < 1:
            continue
        Cin, Cout = 4, 8 if G != 4 else 4
        x = rng.standard_normal((2, Cin, H, W))
        w = rng.standard_normal((Cout, Cin // G, Kh, Kw))
        b = rng.standard_normal(Cout)
        y, s = oracle.conv2d(x, w, b, S, P, D, G, relu=False)
        tol = 1e-12 * (s + np.abs(b)[None, :, None, None] + 1e-300)
        yg = oracle.conv2d_by_gemm(x, w, b, S, P, D, G)
        yt = _torch_conv(x, w, b, S, P, D, G)
        assert yg.shape == y.shape == yt.shape
        assert np.all(np.abs(y - yg) <= tol), (S, P, D, K, G, H, W)
        assert np.all(np.abs(y - yt) <= tol), (S, P, D, K, G, H, W)
        checked += 1
    assert checked > 60


def test_p11_depthwise_groups_equal_channels():
    rng = np.random.default_rng(77)
    x = rng.standard_normal((2, 8, 9, 7))
    w = rng.standard_normal((8, 1, 3, 3))
    b = rng.standard_normal(8)
    for S, P, D in ((1, 1, 1), (2, 1, 1), (1, 2, 2), (2, 0, 1)):
        y, s = oracle.conv2d(x, w, b, S, P, D, 8, relu=True)
        yt = _torch_conv(x, w, b, S, P, D, 8, relu=True)
        assert np.all(np.abs(y - yt) <= 1e-12 * (s + 1))


# ------------------------------------------------------------- p12: torch at workload shapes

@pytest.mark.parametrize("cid,li", [(1, 0), (2, 0), (3, 0), (3, 1), (4, 0), (5, 0), (5, 1), (5, 2), (5, 3)])
def test_p12_torch_float64_at_workload_shapes(cid, li):
    """Every workload layer at its real channel/spatial shape (batch 1) agrees
    with torch's CPU float64 convolution within 1e-12 * S."""
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li, N=1)
    relu = bool(ly.epilogue & ci.EPI_RELU)
    y, s = oracle.conv2d(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, relu=relu)
    yt = _torch_conv(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, relu=relu)
    bb = 0 if b is None else np.abs(b.astype(np.float64))[None, :, None, None]
    assert y.shape == yt.shape
    assert np.all(np.abs(y - yt) <= 1e-12 * (s + bb) + 1e-300)


def test_p12_points_match_full_convolution():
    x, w, b = ci.layer_tensors(4, 0, N=2, H=17, W=13)
    y, s = oracle.conv2d(x, w, None, 1, 2, 2, 4)
    rng = np.random.default_rng(1)
    idx = rng.integers(0, y.size, size=500)
    yp, sp = oracle.conv2d_points(x, w, idx, None, 1, 2, 2, 4)
    np.testing.assert_array_equal(yp, y.reshape(-1)[idx])
    np.testing.assert_array_equal(sp, s.reshape(-1)[idx])


# ------------------------------------------------------------- p13: size arithmetic

def test_p13_big_im2col_size_figures():
    """X_col of a 112x112x128 input under a 3x3 filter is 1152 x 12544,
    about 14.47 million entries / 55 MB in fp32, about 9x the 6.3 MB input
    (lpnh.cn sections 3.2-3.3)."""
    f = FIG["big_im2col"]
    x = np.zeros((1, f["Cin"], f["H"], f["W"]))
    xcol = oracle.im2col(x, f["K"], f["K"], f["stride"], f["pad"])
    assert xcol.shape == (f["xcol_rows"], f["xcol_cols"])
    assert f["weight_cols"] == f["Cin"] * f["K"] * f["K"]
    n = xcol.size
    assert abs(n - f["elements_approx"]) / f["elements_approx"] < 2e-3
    mib = n * 4 / 2 ** 20
    assert abs(mib - f["xcol_fp32_MB_approx"]) < 0.5
    in_mb = f["Cin"] * f["H"] * f["W"] * 4 / 1e6
    assert abs(in_mb - f["input_fp32_MB_approx"]) < 0.2
    assert n / (f["Cin"] * f["H"] * f["W"]) == f["inflation_approx"]


def test_p13_flop_counts():
    """Nominal FLOPs = 2*N*Ho*Wo*Cout*(Cin/G)*Kh*Kw; depthwise drops the
    Cout*Cin channel product to Cin (lincklin.cn section 23)."""
    def flops(ly):
        Ho = oracle.out_dim(ly.H, ly.Kh, ly.stride, ly.pad, ly.dilation)
        Wo = oracle.out_dim(ly.W, ly.Kw, ly.stride, ly.pad, ly.dilation)
        return 2 * ly.N * Ho * Wo * ly.Cout * (ly.Cin // ly.groups) * ly.Kh * ly.Kw
    assert flops(ci.layer(2, 0)) == 2 * 32 * 112 * 112 * 256 * 1152
    dw = ci.layer(3, 0)
    assert flops(dw) == 2 * 32 * 56 * 56 * 144 * 9


# ------------------------------------------------------------- generator

def test_generator_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9,
                     -2.5, 3.0e38, np.inf], np.float32)
    got = ci.bf16_bits_to_f32(ci.f32_to_bf16_bits(vals))
    # ties at 1 + 2^-8 go to even (1.0); 1 + 3*2^-8 ties up to 1 + 2^-6
    np.testing.assert_array_equal(got[:3], np.array([1.0, 1.0, 1.0 + 2 ** -6], np.float32))
    assert got[3] == np.float32(1.0 + 2 ** -7)
    assert got[4] == -2.5 and np.isinf(got[6])
    assert np.all(oracle.round_to_bf16(vals[:6].astype(np.float64)) == got[:6])


def test_generator_is_deterministic_and_bf16_exact():
    a = ci.layer_tensors(5, 1, N=2, H=6, W=6)
    b = ci.layer_tensors(5, 1, N=2, H=6, W=6)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    x, w, bias = a
    np.testing.assert_array_equal(ci.bf16_bits_to_f32(ci.f32_to_bf16_bits(x)), x)
    np.testing.assert_array_equal(ci.bf16_bits_to_f32(ci.f32_to_bf16_bits(w)), w)
    assert abs(w.std() - ci.layer(5, 1).weight_std) < 0.01
    assert bias is not None and bias.dtype == np.float32


# ------------------------------------------------------------- t: transposed convolution
# "lpnh.cn/news/2674933" sections 2.3 and 4.2: a transposed convolution
# upsamples; it is the stride-1 convolution of the input with S-1 zeros
# inserted between neighbouring pixels, and in matrix form Y = W^T X, the
# transpose of the standard convolution's matrix.

def _torch_convT(x, w, b, stride, pad, out_pad, dil, groups, relu=False):
    y = F.conv_transpose2d(torch.from_numpy(np.asarray(x, np.float64)), torch.from_numpy(np.asarray(w, np.float64)),
                           None if b is None else torch.from_numpy(np.asarray(b, np.float64)),
                           stride=stride, padding=pad, output_padding=out_pad, groups=groups, dilation=dil)
    if relu:
        y = torch.relu(y)
    return y.numpy()


# (N, Cin, H, W, Cout, K, stride, pad, out_pad, dil, groups)
T_CASES = [
    (2, 4, 5, 6, 6, 4, 2, 1, 0, 1, 1),   # 2x upsampling, kernel divisible by the stride
    (1, 6, 4, 4, 4, 2, 2, 0, 0, 1, 2),   # kernel = stride: non-overlapping blocks, grouped
    (2, 3, 5, 4, 5, 3, 2, 1, 1, 1, 1),   # odd kernel, output padding
    (1, 4, 3, 5, 2, 3, 3, 0, 2, 1, 1),   # stride 3, output padding 2
    (1, 2, 6, 5, 4, 3, 1, 1, 0, 1, 2),   # stride 1
    (2, 4, 4, 3, 4, 3, 2, 2, 1, 2, 2),   # dilation 2, padding larger than the stride
    (1, 3, 4, 4, 3, 5, 2, 3, 0, 1, 1),   # padding 3 with a 5x5 kernel
    (1, 2, 3, 3, 2, 1, 2, 0, 1, 1, 1),   # 1x1 kernel, stride 2: odd outputs receive nothing
    (1, 4, 5, 3, 4, 3, 2, 0, 1, 3, 1),   # dilation 3 with stride 2 (output padding < dilation)
]


def _t_tensors(case, seed, integer=False):
    N, Cin, H, W, Cout, K, S, P, OP, D, G = case
    rng = np.random.default_rng(seed)
    if integer:
        x = rng.integers(-3, 4, (N, Cin, H, W)).astype(np.float64)
        w = rng.integers(-2, 3, (Cin, Cout // G, K, K)).astype(np.float64)
        b = rng.integers(-4, 5, Cout).astype(np.float64)
    else:
        x = rng.standard_normal((N, Cin, H, W))
        w = rng.standard_normal((Cin, Cout // G, K, K))
        b = rng.standard_normal(Cout)
    return x, w, b


def test_t1_transposed_output_size():
    """(H-1)S - 2P + D(K-1) + OP + 1; a standard convolution with the same
    (K, S, P, D) maps every such output size back onto H (the transposed
    convolution is that convolution's adjoint), and 2x upsampling layers give
    twice the input."""
    assert oracle.transpose_out_dim(28, 4, 2, 1) == 56
    assert oracle.transpose_out_dim(56, 2, 2, 0) == 112
    assert oracle.transpose_out_dim(7, 3, 2, 1, 1, 1) == 14
    assert oracle.transpose_out_dim(5, 3, 1, 1) == 5
    for H in range(1, 9):
        for K in range(1, 6):
            for S in range(1, 4):
                for D in range(1, 3):
                    for P in range(0, 3):
                        for OP in range(0, S):   # the S sizes the strided convolution folds together
                            Ho = oracle.transpose_out_dim(H, K, S, P, D, OP)
                            if Ho >= 1 and Ho + 2 * P >= D * (K - 1) + 1:
                                assert oracle.out_dim(Ho, K, S, P, D) == H, (H, K, S, P, D, OP)
    assert oracle.transpose_out_dim(5, 3, 2, 1, 1, 2) == -1   # OP must stay below max(S, D)
    assert oracle.transpose_out_dim(5, 3, 2, 1, 3, 2) == 5 * 2 - 2 + 6 + 2 - 1


@pytest.mark.parametrize("case", T_CASES)
def test_t2_transposed_equals_zero_insertion_then_stride1_conv(case):
    """The page's own construction: insert S-1 zeros between neighbouring
    input pixels, pad by D(K-1)-P (OP more at the far edge; a negative pad
    crops), then a stride-1 convolution (the pinned direct loop) with the
    kernel rotated by 180 degrees and, per group, input and output channel
    roles swapped."""
    N, Cin, H, W, Cout, K, S, P, OP, D, G = case
    x, w, b = _t_tensors(case, 7)
    y, s = oracle.conv_transpose2d(x, w, b, S, P, OP, D, G, relu=True)
    z = np.zeros((N, Cin, (H - 1) * S + 1, (W - 1) * S + 1))
    z[:, :, ::S, ::S] = x
    e = D * (K - 1) - P
    lo, hi = e, e + OP
    z = np.pad(z, ((0, 0), (0, 0), (max(lo, 0), max(hi, 0)), (max(lo, 0), max(hi, 0))))
    if lo < 0:
        z = z[:, :, -lo:, -lo:]
    if hi < 0:
        z = z[:, :, :hi, :hi]
    cin_g, cout_g = Cin // G, Cout // G
    wc = np.zeros((Cout, cin_g, K, K))
    for g in range(G):
        blk = w[g * cin_g:(g + 1) * cin_g]                    # [cin_g][cout_g][K][K]
        wc[g * cout_g:(g + 1) * cout_g] = blk.transpose(1, 0, 2, 3)[:, :, ::-1, ::-1]
    yc, _ = oracle.conv2d(z, wc, b, 1, 0, D, G, relu=True)
    assert yc.shape == y.shape
    np.testing.assert_allclose(y, yc, rtol=0, atol=1e-12 * (float(s.max()) + 1))


@pytest.mark.parametrize("case", T_CASES)
def test_t3_transposed_is_the_adjoint_of_the_convolution(case):
    """Y = W^T X: for integer tensors <conv(u), v> equals <u, convT(v)>
    exactly, with the same weight read as the standard convolution's
    [C_out'][C_in'/G][K][K] weight (Cin of the transposed convolution = the
    standard convolution's output channels)."""
    N, Cin, H, W, Cout, K, S, P, OP, D, G = case
    v, w, _ = _t_tensors(case, 11, integer=True)
    t, _ = oracle.conv_transpose2d(v, w, None, S, P, OP, D, G)
    u = np.random.default_rng(13).integers(-3, 4, t.shape).astype(np.float64)
    cu, _ = oracle.conv2d(u, w, None, S, P, D, G)
    assert cu.shape == v.shape
    assert float(np.sum(cu * v)) == float(np.sum(u * t))


@pytest.mark.parametrize("case", T_CASES)
def test_t4_transposed_matches_torch(case):
    N, Cin, H, W, Cout, K, S, P, OP, D, G = case
    x, w, b = _t_tensors(case, 17)
    y, s = oracle.conv_transpose2d(x, w, b, S, P, OP, D, G, relu=True)
    yt = _torch_convT(x, w, b, S, P, OP, D, G, relu=True)
    assert y.shape == yt.shape
    np.testing.assert_allclose(y, yt, rtol=0, atol=1e-12 * (float(s.max()) + 1))
    sa, _ = oracle.conv_transpose2d(np.abs(x), np.abs(w), None, S, P, OP, D, G)
    np.testing.assert_allclose(s, sa, rtol=1e-12, atol=0)


def test_t5_kernel_equal_to_stride_is_blockwise_outer_product():
    """K = S, P = 0: windows do not overlap, so output block (ih, iw) is
    exactly sum_ci x[ci, ih, iw] * w[ci, co, :, :] plus the bias."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 5, 3, 4))
    w = rng.standard_normal((5, 3, 2, 2))
    b = rng.standard_normal(3)
    y, _ = oracle.conv_transpose2d(x, w, b, 2, 0, 0, 1, 1)
    want = np.einsum("nchw,cokl->nohkwl", x, w).reshape(2, 3, 6, 8) + b[None, :, None, None]
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12)


def test_t6_transposed_points_match_full():
    case = (2, 4, 5, 6, 6, 4, 2, 1, 1, 1, 2)
    N, Cin, H, W, Cout, K, S, P, OP, D, G = case
    x, w, b = _t_tensors(case, 23)
    y, s = oracle.conv_transpose2d(x, w, b, S, P, OP, D, G, relu=True)
    idx = np.random.default_rng(3).choice(y.size, 300, replace=False)
    yp, sp = oracle.conv_transpose2d_points(x, w, idx, b, S, P, OP, D, G, relu=True)
    np.testing.assert_allclose(yp, y.reshape(-1)[idx], rtol=0, atol=1e-12 * (float(s.max()) + 1))
    np.testing.assert_allclose(sp, s.reshape(-1)[idx], rtol=1e-12, atol=1e-300)


# ------------------------------------------------------------- planted mistakes

_MUTATIONS = {
    "drop_last_kw_tap": ("for (long kw = 0; kw < Kw; ++kw)", "for (long kw = 0; kw < Kw - (Kw > 1); ++kw)"),
    "flipped_kernel": ("const long hi = ho * stride + kh * dil - pad;",
                       "const long hi = ho * stride + (Kh - 1 - kh) * dil - pad;"),
    "pad_sign": ("const long wi = wo * stride + kw * dil - pad;",
                 "const long wi = wo * stride + kw * dil + pad;"),
    "no_dilation": ("const long hi = ho * stride + kh * dil - pad;",
                    "const long hi = ho * stride + kh - pad;"),
    "wrong_group_base": ("const long c = g * cin_g + ci;", "const long c = ci;"),
    "relu_before_bias": ("double v = acc + (bias ? bias[co] : 0.0);\n    if (relu && v < 0.0) v = 0.0;",
                         "double v = (relu && acc < 0.0) ? 0.0 : acc;\n    v += (bias ? bias[co] : 0.0);"),
}
# the same kinds of mistakes in the transposed convolution's scatter
_T_MUTATIONS = {
    "t_drop_last_tap": ("for (long kw = 0; kw < Kw; ++kw) {\n                                const long ow",
                        "for (long kw = 0; kw < Kw - (Kw > 1); ++kw) {\n                                const long ow"),
    "t_unflipped_scatter": ("const long oh = ih * stride - pad + kh * dil;",
                            "const long oh = ih * stride - pad + (Kh - 1 - kh) * dil;"),
    "t_pad_sign": ("const long ow = iw * stride - pad + kw * dil;",
                   "const long ow = iw * stride + pad + kw * dil;"),
    "t_weight_roles_swapped": ("w[((c * cout_g + col) * Kh + kh) * Kw + kw];\n                                yp",
                               "w[((col * cin_g + ci) * Kh + kh) * Kw + kw];\n                                yp"),
    "t_stride_ignored": ("const long oh = ih * stride - pad + kh * dil;", "const long oh = ih - pad + kh * dil;"),
    "t_wrong_group_base": ("const long c = g * cin_g + ci;\n                for (long ih",
                           "const long c = ci;\n                for (long ih"),
}


@pytest.fixture(scope="module")
def mutant_libs():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "conv2d_oracle.c")).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    libs = {}
    try:
        for name, (a, b) in {**_MUTATIONS, **_T_MUTATIONS}.items():
            assert src.count(a) >= 1, name
            path = os.path.join(tmp, f"{name}.c")
            open(path, "w").write(src.replace(a, b, 1))
            libs[name] = oracle.load_library(oracle.build(src=path, out=os.path.join(tmp, f"lib{name}.so")))
        yield libs
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("name", list(_MUTATIONS))
def test_planted_mistake_is_caught(name, mutant_libs):
    """Each planted mistake makes the torch cross-check of a small
    dilated/grouped/padded conv with bias+ReLU fail."""
    lib = mutant_libs[name]
    rng = np.random.default_rng(31)
    x = rng.standard_normal((2, 4, 9, 8))
    w = rng.standard_normal((6, 2, 3, 3))
    b = rng.standard_normal(6)
    y, s = oracle.conv2d(x, w, b, 1, 2, 2, 2, relu=True, lib=lib)
    yt = _torch_conv(x, w, b, 1, 2, 2, 2, relu=True)
    assert not np.all(np.abs(y - yt) <= 1e-12 * (s + np.abs(b)[None, :, None, None]))


@pytest.mark.parametrize("name", list(_T_MUTATIONS))
def test_planted_transposed_mistake_is_caught(name, mutant_libs):
    """Each planted mistake in the scatter makes the torch cross-check of a
    small grouped, padded stride-2 transposed convolution fail."""
    lib = mutant_libs[name]
    case = (2, 4, 5, 4, 6, 3, 2, 1, 1, 1, 2)
    N, Cin, H, W, Cout, K, S, P, OP, D, G = case
    x, w, b = _t_tensors(case, 41)
    y, s = oracle.conv_transpose2d(x, w, b, S, P, OP, D, G, relu=True, lib=lib)
    yt = _torch_convT(x, w, b, S, P, OP, D, G, relu=True)
    assert not np.all(np.abs(y - yt) <= 1e-12 * (s + 1))
