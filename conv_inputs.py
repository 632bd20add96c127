"""Seeded synthetic inputs for the conv2d forward workloads.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark.  It draws random tensors and rounds them to the storage type; it
holds none of the convolution's arithmetic (no output sizes, no sums, no
epilogue), so neither side of a parity check can lean on the other through it.

Workloads (shapes and distributions) follow the five conv2d configurations of
the benchmark description: a 224x224x3 -> 112x112x32 stride-2 first layer in
fp32 (the single-point example of "lpnh.cn/news/2674933" section 2.1), a
112x112x128 -> 256 3x3 layer (that page's section 3.2 GEMM example, batched),
a MobileNetV2-style depthwise + pointwise pair ("lnrq.cn/news/4475" section
3.1), a dilated and grouped layer (lpnh.cn sections 2.2, 4.2) and
ResNet-50-bottleneck-shaped layers (lnrq.cn section 5.3); a sixth workload
holds the transposed-convolution layers of a decoder's upsampling stage.

Storage types: fp32 tensors are drawn in fp64 and rounded to the nearest fp32;
bf16 tensors are drawn in fp64, rounded to fp32, then to bf16 with
round-to-nearest-even.  Every returned array is float32 whose values are exactly
representable in the storage type, so the same numbers can be fed to the GPU
and, promoted to fp64, to the oracle.

Seeds: seed = 1000*config + 100*layer + tensor, tensor 1 = x, 2 = w, 3 = bias,
each drawn from ``numpy.random.default_rng(seed)`` (PCG64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"

EPI_NONE = 0
EPI_BIAS = 1
EPI_RELU = 2


@dataclass(frozen=True)
class Layer:
    """One convolution layer of a workload (NCHW shapes, OIHW weights)."""
    name: str
    N: int
    Cin: int
    H: int
    W: int
    Cout: int
    Kh: int
    Kw: int
    stride: int = 1
    pad: int = 0
    dilation: int = 1
    groups: int = 1
    dtype: str = BF16
    epilogue: int = EPI_NONE
    x_dist: tuple = ("normal", 1.0)
    w_std: float | None = None      # None: Kaiming normal, sqrt(2 / fan_in)
    bias_std: float = 0.01
    chained_from: str | None = None  # name of the layer whose output is this layer's x
    transposed: bool = False         # transposed convolution: w is [Cin][Cout/G][Kh][Kw]
    out_pad: int = 0                 # extra output rows/columns of a transposed layer

    @property
    def fan_in(self) -> int:
        if self.transposed:
            # products each output receives when the kernel is a multiple of
            # the stride: (Cin/G) * (Kh/S) * (Kw/S)
            return max(1, (self.Cin // self.groups) * -(-self.Kh // self.stride) * -(-self.Kw // self.stride))
        return (self.Cin // self.groups) * self.Kh * self.Kw

    @property
    def w_shape(self) -> tuple:
        if self.transposed:
            return (self.Cin, self.Cout // self.groups, self.Kh, self.Kw)
        return (self.Cout, self.Cin // self.groups, self.Kh, self.Kw)

    @property
    def weight_std(self) -> float:
        return self.w_std if self.w_std is not None else math.sqrt(2.0 / self.fan_in)

    def scaled(self, **kw) -> "Layer":
        d = dict(self.__dict__)
        d.update(kw)
        return Layer(**d)


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    layers: tuple = field(default_factory=tuple)


def _kaiming(fan_in: int) -> float:
    return math.sqrt(2.0 / fan_in)


WORKLOADS = {
    1: Workload(1, "conv3x3s2_fp32_nchw_1x3x224x224_to_32", (
        Layer("conv1", 1, 3, 224, 224, 32, 3, 3, stride=2, pad=1, dtype=F32,
              epilogue=EPI_BIAS, x_dist=("uniform", 1.0), w_std=_kaiming(27)),
    )),
    2: Workload(2, "conv3x3_bf16_n32_128x112x112_to_256_bias_relu", (
        Layer("conv3x3", 32, 128, 112, 112, 256, 3, 3, stride=1, pad=1,
              epilogue=EPI_BIAS | EPI_RELU, x_dist=("normal", 1.0), w_std=_kaiming(1152)),
    )),
    3: Workload(3, "mobilenetv2_dw3x3_pw1x1_bf16_n32_144x56x56", (
        Layer("depthwise", 32, 144, 56, 56, 144, 3, 3, stride=1, pad=1, groups=144,
              epilogue=EPI_BIAS | EPI_RELU, x_dist=("uniform", 1.0)),
        Layer("pointwise", 32, 144, 56, 56, 24, 1, 1, epilogue=EPI_NONE,
              x_dist=("uniform", 1.0), chained_from="depthwise"),
    )),
    4: Workload(4, "conv3x3_d2_g4_bf16_n16_256x64x64", (
        Layer("dilated_grouped", 16, 256, 64, 64, 256, 3, 3, stride=1, pad=2, dilation=2,
              groups=4, epilogue=EPI_NONE, x_dist=("normal", 1.0), w_std=_kaiming(576)),
    )),
    5: Workload(5, "resnet50_bottleneck_bf16_n64_56x56", (
        Layer("L1_1x1_256_64", 64, 256, 56, 56, 64, 1, 1, epilogue=EPI_BIAS | EPI_RELU),
        Layer("L2_3x3_64_64", 64, 64, 56, 56, 64, 3, 3, pad=1, epilogue=EPI_BIAS | EPI_RELU,
              chained_from="L1_1x1_256_64"),
        Layer("L3_1x1_64_256", 64, 64, 56, 56, 256, 1, 1, epilogue=EPI_BIAS | EPI_RELU,
              chained_from="L2_3x3_64_64"),
        Layer("L4_3x3s2_128_128", 64, 128, 56, 56, 128, 3, 3, stride=2, pad=1,
              epilogue=EPI_BIAS | EPI_RELU),
    )),
    # A decoder's 2x upsampling stage built from transposed convolutions
    # (lpnh.cn sections 2.3 and 4.2: upsampling in generative networks, with
    # the kernel a multiple of the stride): 4x4 stride 2 pad 1 (28 -> 56) and
    # 2x2 stride 2 (56 -> 112).  Inputs are post-ReLU activations.
    6: Workload(6, "decoder_upsampling_transposed_bf16_n32", (
        Layer("up4x4s2_256_128", 32, 256, 28, 28, 128, 4, 4, stride=2, pad=1,
              epilogue=EPI_BIAS | EPI_RELU, x_dist=("halfnormal", 1.0), transposed=True),
        Layer("up2x2s2_128_64", 32, 128, 56, 56, 64, 2, 2, stride=2, pad=0,
              epilogue=EPI_BIAS | EPI_RELU, x_dist=("halfnormal", 1.0), transposed=True),
    )),
}


def layer(cid: int, name_or_index=0) -> Layer:
    wl = WORKLOADS[cid]
    if isinstance(name_or_index, int):
        return wl.layers[name_or_index]
    for ly in wl.layers:
        if ly.name == name_or_index:
            return ly
    raise KeyError(name_or_index)


def layer_index(cid: int, name: str) -> int:
    for i, ly in enumerate(WORKLOADS[cid].layers):
        if ly.name == name:
            return i
    raise KeyError(name)


def seed_of(cid: int, layer_idx: int, tensor: int) -> int:
    return 1000 * cid + 100 * layer_idx + tensor


# ---------------------------------------------------------------- rounding

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> fp32 (nearest) -> storage type; returned as float32 values."""
    a32 = np.asarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return a32
    if dtype == BF16:
        return bf16_bits_to_f32(f32_to_bf16_bits(a32))
    raise ValueError(dtype)


# ---------------------------------------------------------------- draws

def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    kind, scale = dist
    if kind == "normal":
        return rng.standard_normal(size=shape) * scale
    if kind == "uniform":
        return rng.uniform(-scale, scale, size=shape)
    if kind == "halfnormal":
        return np.abs(rng.standard_normal(size=shape)) * scale
    raise ValueError(kind)


def layer_tensors(cid: int, layer_idx: int, *, N: int | None = None, H: int | None = None,
                  W: int | None = None, mode: str = "random", ly: Layer | None = None):
    """Seeded (x, w, bias) for one layer as float32 arrays (NCHW, OIHW, [Cout]).

    ``N``, ``H``, ``W`` shrink the activation for fast tests without changing
    the weights.  ``mode="int"`` is the exact-integer mode: x in {-2..2},
    w in {-1,0,1}, integer bias in [-4, 4]; every partial sum is then an
    integer well below 2**24, exact in fp32 and bf16-storable inputs.
    Bias is None when the layer's epilogue has no bias.
    """
    ly = ly if ly is not None else WORKLOADS[cid].layers[layer_idx]
    n = ly.N if N is None else N
    h = ly.H if H is None else H
    w_ = ly.W if W is None else W
    xs = (n, ly.Cin, h, w_)
    ws = ly.w_shape
    rx = np.random.default_rng(seed_of(cid, layer_idx, 1))
    rw = np.random.default_rng(seed_of(cid, layer_idx, 2))
    rb = np.random.default_rng(seed_of(cid, layer_idx, 3))
    if mode == "int":
        x = rx.integers(-2, 3, size=xs).astype(np.float32)
        w = rw.integers(-1, 2, size=ws).astype(np.float32)
        b = rb.integers(-4, 5, size=(ly.Cout,)).astype(np.float32)
    elif mode == "random":
        x = to_storage(_draw(rx, ly.x_dist, xs), ly.dtype)
        w = to_storage(rw.standard_normal(size=ws) * ly.weight_std, ly.dtype)
        b = rb.standard_normal(size=(ly.Cout,)).astype(np.float64) * ly.bias_std
        b = b.astype(np.float32)
    else:
        raise ValueError(mode)
    if not (ly.epilogue & EPI_BIAS):
        b = None
    return x, w, b


def random_tensors(seed: int, N, Cin, H, W, Cout, Kh, Kw, groups=1, dtype=BF16,
                   mode="random", bias=True):
    """(x, w, bias) of an arbitrary shape for sweep tests, from one seed."""
    rng = np.random.default_rng(seed)
    xs = (N, Cin, H, W)
    ws = (Cout, Cin // groups, Kh, Kw)
    if mode == "int":
        x = rng.integers(-2, 3, size=xs).astype(np.float32)
        w = rng.integers(-1, 2, size=ws).astype(np.float32)
        b = rng.integers(-4, 5, size=(Cout,)).astype(np.float32)
    else:
        x = to_storage(rng.standard_normal(size=xs), dtype)
        fan = max(1, (Cin // groups) * Kh * Kw)
        w = to_storage(rng.standard_normal(size=ws) * math.sqrt(2.0 / fan), dtype)
        b = (rng.standard_normal(size=(Cout,)) * 0.01).astype(np.float32)
    return x, w, (b if bias else None)


def nchw_to_nhwc(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.transpose(a, (0, 2, 3, 1)))


def nhwc_to_nchw(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.transpose(a, (0, 3, 1, 2)))
