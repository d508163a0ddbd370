"""GPU parity of the int8 epilogue variants (TensorFlow conv_ops_fused_int8.cc,
BiasActivationOutputKernel): a conv_input_scale per output channel, and the
cuDNN 7 order (scale and bias in one fused multiply-add, then the side
input).  Bit-exact against the oracle on every kernel family that runs
them."""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import make_plan, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu


def _scales(L, seed):
    """Per-channel scales around the layer's scalar (x0.5 .. x2, fp32)."""
    rng = np.random.default_rng(seed)
    return (np.float32(L.conv_input_scale) *
            rng.uniform(0.5, 2.0, size=L.K)).astype(np.float32)


def _check(name, N, per_channel, order, variant=None, monkeypatch=None, expect=None):
    if variant:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", variant)
    L = wl.LAYERS[name]
    inp = wl.make_inputs(L, N=N)
    n = inp.x.shape[0]
    plan = make_plan(n, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops,
                     cudnn7_order=(order == 7))
    cis = _scales(L, 7 + (N or 0)) if per_channel else L.conv_input_scale
    say("%s N=%d per_channel=%s order=%d kernel=%s" % (name, n, per_channel, order,
                                                      plan.kernel_name))
    if expect:
        assert plan.kernel_name in expect, plan.kernel_name
    y, guards = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, inp.side, cis,
                        L.side_input_scale, guard=128)
    assert guards, "write outside y"
    r = oracle_out(L.dtype, inp.x, inp.w, L.stride, L.padding, inp.bias, inp.side, cis,
                   L.side_input_scale, L.relu, order=order)
    bad = np.count_nonzero(y != r)
    assert bad == 0, "%d of %d int8 outputs differ" % (bad, r.size)


@pytest.mark.parametrize("name,expect", [
    ("resnet_3x3_int8", ("conv_halo_i8",)), ("resnet_1x1_int8", ("conv_stream_i8",)),
    ("resnet_3x3s2_int8", ("conv_halo_s2_i8",)), ("tiny_int8_3x3", ("conv_general_i8",))])
def test_per_channel_scale(name, expect):
    _check(name, 4, True, 8, expect=expect)


@pytest.mark.parametrize("name,variant", [
    ("resnet_3x3_int8", "general"), ("resnet_3x3_int8", "rf"), ("resnet_3x3_int8", "stream"),
    ("resnet_1x1_int8", "tile"), ("resnet_3x3s2_int8", "tile")])
def test_per_channel_scale_forced_variant(name, variant, monkeypatch):
    _check(name, 2, True, 8, variant, monkeypatch, expect=("conv_%s_i8" % variant,))


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("name,expect", [
    ("resnet_3x3_int8", ("conv_halo_i8",)), ("resnet_1x1_int8", ("conv_stream_i8",)),
    ("resnet_3x3s2_int8", ("conv_halo_s2_i8",)), ("tiny_int8_3x3", ("conv_general_i8",))])
def test_cudnn7_order(name, expect, per_channel):
    _check(name, 4, per_channel, 7, expect=expect)


@pytest.mark.parametrize("name,variant", [
    ("resnet_3x3_int8", "general"), ("resnet_3x3_int8", "rf"), ("resnet_3x3_int8", "stream"),
    ("resnet_1x1_int8", "tile"), ("resnet_3x3s2_int8", "general"), ("resnet_3x3s2_int8", "tile")])
def test_cudnn7_order_forced_variant(name, variant, monkeypatch):
    _check(name, 2, True, 7, variant, monkeypatch, expect=("conv_%s_i8" % variant,))


def test_full_size_variants():
    """The benchmark layer at full size on the halo kernel: per-channel
    scales, and the cuDNN 7 order with per-channel scales."""
    _check("resnet_3x3_int8", None, True, 8, expect=("conv_halo_i8",))
    _check("resnet_3x3_int8", None, True, 7, expect=("conv_halo_i8",))


def test_cudnn7_crafted_fused_scale_and_bias():
    """Single-pixel 1x1 case whose result flips with the fused scale-and-bias
    step: 5 * 838860.9375 - 4194304 = 0.6875 exactly -> 1 (cuDNN 7), while
    the separate steps of the cuDNN 8 order round 4194304.6875 to 4194304.5
    first -> 0.5 -> 0."""
    x = np.full((1, 1, 1, 1), 5, np.int8)
    w = np.full((1, 1, 1, 1), 1, np.int8)
    bias = np.array([-4194304.0], np.float32)
    for order, exp in ((8, 0), (7, 1)):
        plan = make_plan(1, 1, 1, 1, 1, 1, 1, 1, "VALID", "int8",
                         [wl.OP_SCALE, wl.OP_BIAS], cudnn7_order=(order == 7))
        y, _ = run_gpu(plan, "int8", x, w, bias, None, np.float32(838860.9375), 0.0)
        assert int(y.reshape(-1)[0]) == exp, (order, plan.kernel_name)
