"""GPU parity of the float (bf16 / fp32) path beyond the benchmark layers:
the activations of MIOpen's fusion tables (Leaky Relu, Clipped Relu, CLAMP,
after bias and batch norm) on every float kernel family, and the filter sizes
and strides of its CBNA "Direct" row (3x3 .. 11x11, stride 1 and 2).
Normwise tolerances as for the benchmark layers (fp32 1e-5, bf16 2e-2)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import TOL, float_error, run_gpu, say
import convolution_implicit_gemm_nhwc_amd as fc

pytestmark = pytest.mark.gpu


def _inputs(rng, dtype, N, H, W, C, K, R, S):
    sd = 1.0 / np.sqrt(R * S * C)
    x = rng.normal(0, sd * 8, size=(N, H, W, C)).astype(np.float32)
    w = rng.normal(0, sd, size=(R, S, C, K)).astype(np.float32)
    if dtype == "bf16":
        x, w = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(w)
    bias = rng.normal(0, 0.1, K).astype(np.float32)
    bn = dict(mean=rng.normal(0, 0.1, K).astype(np.float32),
              var=rng.uniform(0.5, 1.5, K).astype(np.float32),
              gamma=rng.uniform(0.5, 1.5, K).astype(np.float32),
              beta=rng.normal(0, 0.1, K).astype(np.float32), eps=1e-5)
    return x, w, bias, bn


def _widen(a, dtype):
    return wl.bf16_bits_to_float(a) if dtype == "bf16" else a


def _check(dtype, shape, stride, padding, act, alpha, beta, use_bn=True, expect=None,
           seed=0):
    N, H, W, C, K, R, S = shape
    rng = np.random.default_rng(seed)
    x, w, bias, bn = _inputs(rng, dtype, N, H, W, C, K, R, S)
    ops = ["bias"] + (["bn"] if use_bn else []) + ([act] if act else [])
    plan = fc.Plan(N, H, W, C, K, R, S, stride, padding, dtype, ops=ops)
    say("%s %s s%d %s act=%s(%g, %g) kernel=%s" % (dtype, shape, stride, padding, act, alpha,
                                                  beta, plan.kernel_name))
    if expect:
        assert plan.kernel_name in expect, plan.kernel_name
    y, guards = run_gpu(plan, dtype, x, w, bias, None, bn=bn if use_bn else None, guard=128,
                        activ=(alpha, beta))
    assert guards, "write outside y"
    r = oracle.fused_conv_float(_widen(x, dtype), _widen(w, dtype), bias,
                                bn if use_bn else None, stride=stride, padding=padding,
                                act=act, alpha=alpha, beta=beta)
    e = float_error(y, r)
    say("  normwise error %.3e (tolerance %.0e)" % (e, TOL[dtype]))
    assert e <= TOL[dtype]


ACTS = [("relu", 0.0, 0.0), ("leaky_relu", 0.1, 0.0), ("clipped_relu", 0.5, 0.0),
        ("clamp", -0.3, 0.4)]


@pytest.mark.parametrize("act,alpha,beta", ACTS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant,shape", [
    (None, (2, 14, 14, 256, 256, 3, 3)),      # tiled kernel (the benchmark layer's shape)
    ("rf", (2, 9, 11, 32, 64, 3, 3)),          # resident-filter kernel
    ("general", (2, 7, 5, 24, 20, 3, 3))])     # general kernel, ragged C and K
def test_activations(variant, shape, dtype, act, alpha, beta, monkeypatch):
    if variant:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", variant)
    expect = None if variant is None else ("conv_%s_%s" % (variant, dtype.replace("p", "")),)
    _check(dtype, shape, 1, "SAME", act, alpha, beta, expect=expect)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("R,stride", [(3, 2), (5, 1), (5, 2), (7, 1), (7, 2), (9, 1), (11, 2)])
def test_cbna_direct_filter_sizes(R, stride, dtype):
    """The filter sizes and strides of MIOpen's CBNA Direct row, with a
    leaky ReLU activation, on 64 and 128 channels."""
    _check(dtype, (2, 23, 19, 64, 128, R, R), stride, "SAME", "leaky_relu", 0.2, 0.0,
           seed=R * 10 + stride)
