"""Seeded synthetic inputs for the fused NHWC convolution.

This module only draws random tensors; it holds none of the convolution's
arithmetic, and both the GPU path's tests/benchmark and the CPU oracle take
their inputs from it.  Each workload is a ResNet-shaped layer (shapes and value
distributions below); there is no dataset: the synthetic tensors are the
workload.

Conventions: integer ranges are inclusive; ``normal(mu, sd)`` takes the
standard deviation; every tensor has its own stream spawned from
``numpy.random.SeedSequence(seed)``.  Shapes: x NHWC, filter HWIO [R,S,C,K],
side input NHWC with the output's shape, per-channel vectors [K].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Epilogue op codes (same numbering as the C header's fconv_op enum).
OP_SCALE, OP_SIDE, OP_BIAS, OP_BN, OP_RELU = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    dtype: str  # "int8" | "bf16" | "fp32"
    N: int
    H: int
    W: int
    C: int
    K: int
    R: int
    S: int
    stride: int
    padding: str  # "SAME" | "VALID"
    Ho: int  # output size as the workload states it (checked by the tests)
    Wo: int
    ops: tuple
    seed: int
    x_range: tuple = (-127, 127)
    w_range: tuple = (-127, 127)
    side_range: tuple = (-127, 127)
    bias_sd: float = 16.0
    conv_input_scale: float = 1.0
    side_input_scale: float = 0.0
    description: str = ""

    @property
    def relu(self) -> bool:
        return OP_RELU in self.ops

    @property
    def has_side(self) -> bool:
        return OP_SIDE in self.ops

    def ops_count(self) -> int:
        """2*N*Ho*Wo*K*R*S*C, the throughput numerator."""
        return 2 * self.N * self.Ho * self.Wo * self.K * self.R * self.S * self.C


LAYERS = {
    "tiny_int8_3x3": Layer(
        "tiny_int8_3x3", "int8", N=1, H=8, W=8, C=8, K=8, R=3, S=3, stride=1,
        padding="SAME", Ho=8, Wo=8, ops=(OP_SCALE, OP_SIDE, OP_BIAS, OP_RELU), seed=0,
        bias_sd=16.0, conv_input_scale=2.0 ** -8, side_input_scale=0.5,
        description="N=1 8x8x8 -> 8, 3x3 s1 SAME, side+bias+ReLU"),
    "resnet_3x3_int8": Layer(
        "resnet_3x3_int8", "int8", N=32, H=56, W=56, C=64, K=64, R=3, S=3,
        stride=1, padding="SAME", Ho=56, Wo=56,
        ops=(OP_SCALE, OP_SIDE, OP_BIAS, OP_RELU), seed=1, x_range=(0, 127), side_range=(0, 127), bias_sd=64.0,
        conv_input_scale=2.0 ** -11, side_input_scale=0.25,
        description="N=32 56x56x64 -> 64, 3x3 s1 SAME, side+bias+ReLU"),
    "resnet_1x1_int8": Layer(
        "resnet_1x1_int8", "int8", N=32, H=56, W=56, C=256, K=64, R=1, S=1,
        stride=1, padding="VALID", Ho=56, Wo=56, ops=(OP_SCALE, OP_BIAS), seed=2,
        bias_sd=16.0, conv_input_scale=2.0 ** -11,
        description="N=32 56x56x256 -> 64, 1x1 VALID, bias only"),
    "resnet_3x3s2_int8": Layer(
        "resnet_3x3s2_int8", "int8", N=64, H=56, W=56, C=128, K=128, R=3, S=3,
        stride=2, padding="SAME", Ho=28, Wo=28,
        ops=(OP_SCALE, OP_SIDE, OP_BIAS, OP_RELU), seed=3, bias_sd=16.0, conv_input_scale=2.0 ** -12, side_input_scale=1.0,
        description="N=64 56x56x128 -> 128, 3x3 s2 SAME (pads 0/1), side+bias+ReLU"),
    "resnet_3x3_bf16_bn": Layer(
        "resnet_3x3_bf16_bn", "bf16", N=16, H=28, W=28, C=256, K=256, R=3, S=3,
        stride=1, padding="SAME", Ho=28, Wo=28, ops=(OP_BIAS, OP_BN, OP_RELU),
        seed=4, description="N=16 28x28x256 -> 256, 3x3 s1 SAME, bf16, bias+BN+ReLU"),
    "resnet_3x3_fp32_bn": Layer(
        "resnet_3x3_fp32_bn", "fp32", N=16, H=28, W=28, C=256, K=256, R=3, S=3,
        stride=1, padding="SAME", Ho=28, Wo=28, ops=(OP_BIAS, OP_BN, OP_RELU),
        seed=4, description="N=16 28x28x256 -> 256, 3x3 s1 SAME, fp32, bias+BN+ReLU"),
    # Two more filter sizes of the CBNA "Direct" row of MIOpen's bf16 fusion
    # table (3x3 .. 11x11, stride 1 and 2), drawn like the 3x3 bf16 layer.
    "cbna_5x5_bf16": Layer(
        "cbna_5x5_bf16", "bf16", N=16, H=28, W=28, C=128, K=128, R=5, S=5,
        stride=1, padding="SAME", Ho=28, Wo=28, ops=(OP_BIAS, OP_BN, OP_RELU),
        seed=5, description="N=16 28x28x128 -> 128, 5x5 s1 SAME, bf16, bias+BN+ReLU"),
    "cbna_7x7s2_bf16": Layer(
        "cbna_7x7s2_bf16", "bf16", N=16, H=56, W=56, C=64, K=128, R=7, S=7,
        stride=2, padding="SAME", Ho=28, Wo=28, ops=(OP_BIAS, OP_BN, OP_RELU),
        seed=6, description="N=16 56x56x64 -> 128, 7x7 s2 SAME (pads 2/3), bf16, bias+BN+ReLU"),
    # A filter as large as the image, VALID: one output pixel per image, the
    # GEMM special case of the fused op ([N, H*W*C] x [H*W*C, K]), shaped like
    # a network's last 7x7x512 feature map feeding 1024 outputs.
    "valid_7x7_int8": Layer(
        "valid_7x7_int8", "int8", N=32, H=7, W=7, C=512, K=1024, R=7, S=7,
        stride=1, padding="VALID", Ho=1, Wo=1, ops=(OP_SCALE, OP_BIAS, OP_RELU), seed=9,
        x_range=(0, 127), bias_sd=16.0, conv_input_scale=2.0 ** -13,
        description="N=32 7x7x512 -> 1024, 7x7 VALID (full-size filter), bias+ReLU"),
    "valid_7x7_bf16": Layer(
        "valid_7x7_bf16", "bf16", N=32, H=7, W=7, C=512, K=1024, R=7, S=7,
        stride=1, padding="VALID", Ho=1, Wo=1, ops=(OP_BIAS, OP_BN, OP_RELU), seed=10,
        description="N=32 7x7x512 -> 1024, 7x7 VALID (full-size filter), bf16, bias+BN+ReLU"),
}


# Weight-gradient workloads: the filter gradient of a layer's convolution,
# given its input x and an output gradient dy.  Shapes are those of the
# forward layers above (the 3x3 bf16/fp32 layer and the 3x3 int8 benchmark
# layer's geometry run in bf16); ops are empty.
WGRAD_LAYERS = {
    "wgrad_3x3_bf16": Layer(
        "wgrad_3x3_bf16", "bf16", N=16, H=28, W=28, C=256, K=256, R=3, S=3,
        stride=1, padding="SAME", Ho=28, Wo=28, ops=(), seed=7,
        description="dW of N=16 28x28x256 -> 256, 3x3 s1 SAME, bf16 in, fp32 dW"),
    "wgrad_3x3_fp32": Layer(
        "wgrad_3x3_fp32", "fp32", N=16, H=28, W=28, C=256, K=256, R=3, S=3,
        stride=1, padding="SAME", Ho=28, Wo=28, ops=(), seed=7,
        description="dW of N=16 28x28x256 -> 256, 3x3 s1 SAME, fp32"),
    "wgrad_3x3_64_bf16": Layer(
        "wgrad_3x3_64_bf16", "bf16", N=32, H=56, W=56, C=64, K=64, R=3, S=3,
        stride=1, padding="SAME", Ho=56, Wo=56, ops=(), seed=8,
        description="dW of N=32 56x56x64 -> 64, 3x3 s1 SAME, bf16 in, fp32 dW"),
}


@dataclasses.dataclass
class WgradInputs:
    layer: Layer
    x: np.ndarray   # NHWC, uint16 (bf16 bits) or float32
    dy: np.ndarray  # NHWC with the output's shape, same dtype


def make_wgrad_inputs(layer: Layer, N: Optional[int] = None) -> WgradInputs:
    """x ~ N(0, 1/sqrt(R*S*C)) as the forward layers draw it, dy ~ N(0, 1);
    both drawn in fp32 and, for bf16, rounded to bf16 (nearest even).  ``N``
    keeps the first N images."""
    L = layer
    rx, rd = (np.random.default_rng(s) for s in np.random.SeedSequence(L.seed).spawn(2))
    n_keep = L.N if N is None else N
    sd = 1.0 / np.sqrt(L.R * L.S * L.C)
    x = rx.normal(0.0, sd, size=(L.N, L.H, L.W, L.C)).astype(np.float32)[:n_keep]
    dy = rd.normal(0.0, 1.0, size=(L.N, L.Ho, L.Wo, L.K)).astype(np.float32)[:n_keep]
    if L.dtype == "bf16":
        x, dy = float_to_bf16_bits(x), float_to_bf16_bits(dy)
    return WgradInputs(L, np.ascontiguousarray(x), np.ascontiguousarray(dy))


def float_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 samples -> bf16 bit patterns (uint16), round to nearest even.

    Used only to turn drawn samples into bf16 inputs (all finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    layer: Layer
    x: np.ndarray  # int8 / uint16 (bf16 bits) / float32, NHWC
    w: np.ndarray  # same dtype, HWIO
    bias: Optional[np.ndarray]  # float32 [K]
    side: Optional[np.ndarray] = None  # int8 NHWC, output shape
    bn: Optional[dict] = None  # gamma, beta, mean, var (float32 [K]), eps


def make_inputs(layer: Layer, N: Optional[int] = None) -> Inputs:
    """Draw the layer's seeded inputs.  ``N`` (optional) keeps the first N
    images of the full batch, so a sample is a prefix of the full workload."""
    L = layer
    ss = np.random.SeedSequence(L.seed)
    rx, rw, rb, rs, rbn = (np.random.default_rng(s) for s in ss.spawn(5))
    Ho, Wo = L.Ho, L.Wo
    n_keep = L.N if N is None else N
    if L.dtype == "int8":
        x = rx.integers(L.x_range[0], L.x_range[1], size=(L.N, L.H, L.W, L.C),
                        endpoint=True, dtype=np.int8)
        w = rw.integers(L.w_range[0], L.w_range[1], size=(L.R, L.S, L.C, L.K),
                        endpoint=True, dtype=np.int8)
        bias = rb.normal(0.0, L.bias_sd, size=L.K).astype(np.float32)
        side = None
        if L.has_side:
            side = rs.integers(L.side_range[0], L.side_range[1],
                               size=(L.N, Ho, Wo, L.K), endpoint=True, dtype=np.int8)
            side = side[:n_keep]
        return Inputs(L, x[:n_keep], w, bias, side)
    sd = 1.0 / np.sqrt(L.R * L.S * L.C)
    x = rx.normal(0.0, sd, size=(L.N, L.H, L.W, L.C)).astype(np.float32)[:n_keep]
    w = rw.normal(0.0, sd, size=(L.R, L.S, L.C, L.K)).astype(np.float32)
    bias = rb.normal(0.0, 0.1, size=L.K).astype(np.float32)
    bn = dict(mean=rbn.normal(0.0, 0.1, size=L.K).astype(np.float32),
              var=rbn.uniform(0.5, 1.5, size=L.K).astype(np.float32),
              gamma=rbn.uniform(0.5, 1.5, size=L.K).astype(np.float32),
              beta=rbn.normal(0.0, 0.1, size=L.K).astype(np.float32),
              eps=1e-5)
    if L.dtype == "bf16":
        x, w = float_to_bf16_bits(x), float_to_bf16_bits(w)
    return Inputs(L, np.ascontiguousarray(x), np.ascontiguousarray(w), bias, None, bn)


def random_small_case(rng: np.random.Generator):
    """Shape parameters of a random small layer for fuzz-style tests: shapes
    that cross tile boundaries and leave ragged tails (C and K not multiples of
    16 included).  The caller sizes the side input from its own geometry."""
    N = int(rng.integers(1, 4))
    H = int(rng.integers(1, 18))
    W = int(rng.integers(1, 18))
    C = int(rng.integers(1, 41))
    K = int(rng.integers(1, 41))
    R = int(rng.choice([1, 2, 3, 5]))
    S = int(rng.choice([1, 2, 3, 5]))
    stride = int(rng.integers(1, 4))
    padding = "SAME" if rng.random() < 0.6 or H < R or W < S else "VALID"
    return dict(N=N, H=H, W=W, C=C, K=K, R=R, S=S, stride=stride, padding=padding)


def draw_int8(rng, shape, lo=-127, hi=127):
    return rng.integers(lo, hi, size=shape, endpoint=True, dtype=np.int8)
