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


# Round-to-nearest-even of the bf16 output, bit for bit.  Output channel k of
# a 1x1 convolution with a one-hot filter (w[c][k] = 1 for c = k) is exactly
# x[k] + bias[k] in fp32; (x, bias, expected bf16 bits) below put that sum on
# a tie, just past one, at the overflow edge and in the denormal range, with
# the expected bits worked out by hand from IEEE 754 round-to-nearest-even
# (bf16: 8 significant bits, fp32's exponent range).
_TIES = [
    (1.0, 2.0 ** -8, 0x3F80),                       # 1 + half an ulp: tie, to even (down)
    (1.0 + 2.0 ** -7, 2.0 ** -8, 0x3F82),           # odd + half an ulp: tie, to even (up)
    (1.0, 2.0 ** -8 + 2.0 ** -20, 0x3F81),          # just past the tie: up
    (1.0, 2.0 ** -8 - 2.0 ** -20, 0x3F80),          # just below the tie: down
    (-1.0, -(2.0 ** -8), 0xBF80),                   # negative tie, to even
    (-(1.0 + 2.0 ** -7), -(2.0 ** -8), 0xBF82),     # negative odd tie, to even
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** 119, 0x7F80),   # largest bf16 + half an ulp: Inf
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** 118, 0x7F7F),   # a quarter ulp: stays finite
    (0.0, 2.0 ** -134, 0x0000),                     # half the smallest denormal: tie, to 0
    (0.0, 3 * 2.0 ** -134, 0x0002),                 # 1.5 denormal steps: tie, to even (2)
    (0.0, 2.0 ** -133 + 2.0 ** -140, 0x0001),       # just past one step: down to 1
    (3.0, -(2.0 ** -7), 0x4040),                    # 3 - half an ulp: tie, to even (3.0)
    (3.0, -(2.0 ** -7) - 2.0 ** -20, 0x403F),       # just past it: down to 2.984375
]


@pytest.mark.parametrize("variant,roles", [(None, None), ("tile", "1"), ("tile", "0"),
                                           ("general", None), ("rf", None)])
def test_bf16_output_rounding_is_round_to_nearest_even(variant, roles, monkeypatch):
    if variant:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", variant)
    if roles:
        monkeypatch.setenv("FCONV_TILE_ROLES", roles)
    N, H, W, C, K = 1, 1, 16, 128, 64
    xs = np.zeros(C, np.float32)
    bias = np.zeros(K, np.float32)
    for k, (xv, bv, _) in enumerate(_TIES):
        xs[k], bias[k] = xv, bv
    xbits = wl.float_to_bf16_bits(xs)
    assert np.array_equal(wl.bf16_bits_to_float(xbits), xs)  # every x is a bf16 value
    x = np.broadcast_to(xbits, (N, H, W, C)).copy()
    w = np.zeros((1, 1, C, K), np.uint16)
    w[0, 0, np.arange(K), np.arange(K)] = 0x3F80
    plan = fc.Plan(N, H, W, C, K, 1, 1, 1, "VALID", "bf16", ops=["bias"])
    if variant:
        assert plan.kernel_name.startswith("conv_" + variant), plan.kernel_name
    say("bf16 rounding on %s (roles %s)" % (plan.kernel_name, roles))
    y, guards = run_gpu(plan, "bf16", x, w, bias, None, guard=128, raw_bits=True)
    assert guards
    got = y.reshape(W, K)[:, :len(_TIES)]
    want = np.array([e for _, _, e in _TIES], np.uint16)
    for p in range(W):
        bad = [(hex(int(got[p, i])), hex(int(want[i]))) for i in range(len(_TIES)) if got[p, i] != want[i]]
        assert not bad, "pixel %d: %s" % (p, bad)
