"""The allocation-free NCHW entry, conv2d_fwd_noalloc, against conv2d_fwd.

conv2d_fwd_noalloc stages through a static device array instead of memory it
allocates; the kernels and the arithmetic are the same, so its output must
equal conv2d_fwd's bit for bit, and both must meet the oracle's tolerance
(bf16: |y - yref| <= 1e-2 * S + 1e-3; fp32: |y - yref| <= 1e-5 * (S + |b|);
exact-integer data bit for bit).  Two calls run back to back, the second on a
smaller input, so the second reads an array the first left full of its own
data.
"""
import sys

import numpy as np
import pytest

import conv_inputs as ci
import oracle
from helpers import check_bf16, check_f32, ensure_built, gpu_available, lib_dtype, to_dev, torch_dtype

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


def _both(x, w, b, ly):
    """(conv2d_fwd_noalloc output, conv2d_fwd output), NCHW float64."""
    N, Cin, H, W = x.shape
    Cout, _, Kh, Kw = w.shape
    Ho = c2.conv2d_out_dim(H, Kh, ly.stride, ly.pad, ly.dilation)
    Wo = c2.conv2d_out_dim(W, Kw, ly.stride, ly.pad, ly.dilation)
    xd, wd = to_dev(x, ly.dtype), to_dev(w, ly.dtype)
    bd = None if b is None else torch.from_numpy(np.asarray(b, np.float32)).cuda()
    outs = []
    for fn in (c2.conv2d_fwd_noalloc, c2.conv2d_fwd):
        yd = torch.full((N, Cout, Ho, Wo), float("nan"), dtype=torch_dtype(ly.dtype), device="cuda")
        fn(xd, wd, bd, yd, N, Cin, H, W, Cout, Kh, Kw, ly.stride, ly.pad, ly.dilation, ly.groups,
           lib_dtype(ly.dtype), ly.epilogue)
        torch.cuda.synchronize()
        outs.append(yd.float().cpu().numpy().astype(np.float64))
    return outs


def _check(y, x, w, b, ly, mode, what):
    yref, s = oracle.conv2d(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups,
                            relu=bool(ly.epilogue & ci.EPI_RELU))
    if mode == "int":
        want = yref if ly.dtype == ci.F32 else oracle.round_to_bf16(yref)
        np.testing.assert_array_equal(y, want, err_msg=what)
    elif ly.dtype == ci.F32:
        check_f32(y, yref, s, np.abs(b.astype(np.float64))[None, :, None, None], what)
    else:
        check_bf16(y, yref, s, what)


@pytest.mark.parametrize("mode", ["random", "int"])
def test_noalloc_matches_conv2d_fwd_two_calls(mode):
    # first: the bottleneck 3x3 layer at full size (51.5 MB of staging), then
    # the 3x3 128 -> 256 layer on a smaller input (0.9 MB), then the
    # depthwise layer (another kernel, 56.6 MB of staging)
    calls = [(5, 1, {}), (2, 0, dict(N=2, H=23, W=23)), (3, 0, dict(N=31))]
    for cid, li, shrink in calls:
        ly = ci.layer(cid, li)
        x, w, b = ci.layer_tensors(cid, li, mode=mode, **shrink)
        say(f"[noalloc] cfg{cid} {ly.name} {mode} x{x.shape}")
        got, ref = _both(x, w, b, ly)
        np.testing.assert_array_equal(got, ref, err_msg=f"cfg{cid} {ly.name}: noalloc != conv2d_fwd")
        _check(got, x, w, b, ly, mode, f"cfg{cid} {ly.name} noalloc")


def test_noalloc_fp32_direct_path():
    ly = ci.layer(1, 0)
    x, w, b = ci.layer_tensors(1, 0)
    say("[noalloc] cfg1 fp32 direct")
    got, ref = _both(x, w, b, ly)
    np.testing.assert_array_equal(got, ref)
    _check(got, x, w, b, ly, "random", "cfg1 noalloc")


def test_noalloc_rejects_staging_beyond_its_array():
    """The 3x3 128 -> 256 layer at full size needs 308 MB of staging: the call
    fails before enqueuing anything and leaves y untouched."""
    ly = ci.layer(2, 0)
    N, Cin, H, W, Cout = ly.N, ly.Cin, ly.H, ly.W, ly.Cout
    x = torch.zeros((N, Cin, H, W), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((Cout, Cin, 3, 3), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(Cout, dtype=torch.float32, device="cuda")
    y = torch.full((N, Cout, H, W), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(c2.Conv2dError) as e:
        c2.conv2d_fwd_noalloc(x, w, b, y, N, Cin, H, W, Cout, 3, 3, 1, 1, 1, 1, c2.BF16, ly.epilogue)
    assert e.value.code == c2.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all().item())
