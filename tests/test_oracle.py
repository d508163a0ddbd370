"""Pins of the CPU oracle against things other than itself.

Each test fixes part of the oracle by a library routine (numpy, torch), a
closed form, an invariant stated on the pages, or values worked out by hand
(tests/golden).  A plausible slip anywhere in oracle.c -- a dropped tap, a
wrong pad side, a transposed filter, a fused multiply-add in the wrong place,
the wrong rounding direction -- fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _numpy_conv_int64(x, w, stride, pads):
    """Library form of the contraction: pad, sliding windows, einsum in int64."""
    pt, pb, pl, pr = pads
    xp = np.pad(x.astype(np.int64), ((0, 0), (pt, pb), (pl, pr), (0, 0)))
    R, S = w.shape[:2]
    win = np.lib.stride_tricks.sliding_window_view(xp, (R, S), axis=(1, 2))
    win = win[:, ::stride[0], ::stride[1]]  # N, Ho, Wo, C, R, S
    return np.einsum("nhwcrs,rsck->nhwk", win, w.astype(np.int64))


def _torch_conv_f64(x, w, stride, pads):
    """torch.nn.functional.conv2d (cross-correlation) in float64, NHWC in/out."""
    pt, pb, pl, pr = pads
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64)).permute(0, 3, 1, 2)
    xt = F.pad(xt, (pl, pr, pt, pb))
    wt = torch.from_numpy(np.asarray(w, dtype=np.float64)).permute(3, 2, 0, 1)
    y = F.conv2d(xt, wt.contiguous(), stride=stride)
    return y.permute(0, 2, 3, 1).numpy()


# ------------------------------------------------------------------ P-1


def test_brute_force_tiny_shapes_both_forms():
    """Direct and im2col forms equal a numpy einsum and torch conv2d on 500
    random tiny shapes (strides 1-3, SAME and VALID, 1-5 channels)."""
    rng = np.random.default_rng(1234)
    for _ in range(500):
        N = int(rng.integers(1, 3))
        H, W = (int(v) for v in rng.integers(1, 8, size=2))
        C, K = (int(v) for v in rng.integers(1, 6, size=2))
        R, S = (int(v) for v in rng.integers(1, 4, size=2))
        sh, sw = (int(v) for v in rng.integers(1, 4, size=2))
        same = bool(rng.random() < 0.5) or H < R or W < S
        x = wl.draw_int8(rng, (N, H, W, C), -128, 127)
        w = wl.draw_int8(rng, (R, S, C, K), -128, 127)
        g = oracle.geometry(H, W, R, S, sh, sw, same)
        pads = g[2:]
        ref = _numpy_conv_int64(x, w, (sh, sw), pads)
        assert ref.shape == (N, g[0], g[1], K)
        a1 = oracle.conv_acc(x, w, (sh, sw), "SAME" if same else "VALID")
        a2 = oracle.conv_acc(x, w, (sh, sw), "SAME" if same else "VALID", form="im2col")
        np.testing.assert_array_equal(a1, ref)
        np.testing.assert_array_equal(a2, ref)
        np.testing.assert_array_equal(a1, _torch_conv_f64(x, w, (sh, sw), pads))


def test_brute_force_float_paths():
    rng = np.random.default_rng(77)
    for _ in range(60):
        N, H, W = 2, int(rng.integers(2, 9)), int(rng.integers(2, 9))
        C, K = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        R, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        s = int(rng.integers(1, 3))
        same = bool(rng.random() < 0.5) or H < R or W < S
        pads = oracle.geometry(H, W, R, S, s, s, same)[2:]
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        w = rng.standard_normal((R, S, C, K)).astype(np.float32)
        pad = "SAME" if same else "VALID"
        ref = _torch_conv_f64(x, w, (s, s), pads)
        np.testing.assert_allclose(oracle.conv_acc(x, w, s, pad), ref, rtol=1e-12,
                                   atol=1e-12)
        xb, wb = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(w)
        refb = _torch_conv_f64(wl.bf16_bits_to_float(xb), wl.bf16_bits_to_float(wb),
                               (s, s), pads)
        np.testing.assert_allclose(oracle.conv_acc(xb, wb, s, pad), refb,
                                   rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ P-2, P-3


def test_1x1_stride1_is_gemm():
    """conv_ops_fused_int8.cc: a 1x1 stride-1 conv is the [N*H*W, C] x [C, K]
    contraction."""
    rng = np.random.default_rng(5)
    x = wl.draw_int8(rng, (3, 9, 7, 40))
    w = wl.draw_int8(rng, (1, 1, 40, 24))
    acc = oracle.conv_acc(x, w, 1, "VALID")
    ref = x.reshape(-1, 40).astype(np.int64) @ w.reshape(40, 24).astype(np.int64)
    np.testing.assert_array_equal(acc.reshape(-1, 24), ref)
    np.testing.assert_array_equal(oracle.conv_acc(x, w, 1, "SAME"), acc)


def test_full_size_valid_is_gemm():
    """conv_ops_fused_int8.cc: a VALID filter as large as the image is the
    [N, H*W*C] x [H*W*C, K] contraction (fixes the (r, s, c) reduction order)."""
    rng = np.random.default_rng(6)
    x = wl.draw_int8(rng, (4, 5, 3, 7))
    w = wl.draw_int8(rng, (5, 3, 7, 9))
    for form in ("direct", "im2col"):
        acc = oracle.conv_acc(x, w, 1, "VALID", form=form)
        assert acc.shape == (4, 1, 1, 9)
        ref = x.reshape(4, -1).astype(np.int64) @ w.reshape(-1, 9).astype(np.int64)
        np.testing.assert_array_equal(acc.reshape(4, 9), ref)


# ------------------------------------------------------------------ P-4, P-5, P-6


def test_identity_filter_passes_through():
    rng = np.random.default_rng(7)
    x = wl.draw_int8(rng, (2, 6, 5, 16), -128, 127)
    w = np.eye(16, dtype=np.int8).reshape(1, 1, 16, 16)
    bias = np.zeros(16, np.float32)
    y = oracle.fused_conv_i8(x, w, bias, 1.0, padding="VALID")
    np.testing.assert_array_equal(y, x)
    y = oracle.fused_conv_i8(x, w, bias, 1.0, relu=True, padding="VALID")
    np.testing.assert_array_equal(y, np.maximum(x, 0))


@pytest.mark.parametrize("H,W,R,S,stride", [(8, 8, 3, 3, 1), (56, 56, 3, 3, 2),
                                            (7, 9, 5, 3, 2), (6, 6, 2, 4, 1)])
def test_delta_filters_shift_the_image(H, W, R, S, stride):
    """w[r,s,c,k] = [r==dr][s==ds][c==k] copies x shifted by (dr - pt, ds - pl),
    zero where the tap leaves the image: pins pad placement and stride."""
    rng = np.random.default_rng(8)
    C = 4
    x = wl.draw_int8(rng, (1, H, W, C))
    Ho, Wo, pt, pb, pl, pr = oracle.geometry(H, W, R, S, stride, stride, True)
    for dr in range(R):
        for ds in range(S):
            w = np.zeros((R, S, C, C), np.int8)
            for c in range(C):
                w[dr, ds, c, c] = 1
            acc = oracle.conv_acc(x, w, stride, "SAME")
            for ho in range(Ho):
                for wo in range(Wo):
                    i, j = ho * stride - pt + dr, wo * stride - pl + ds
                    inside = 0 <= i < H and 0 <= j < W
                    exp = x[0, i, j] if inside else np.zeros(C, np.int8)
                    np.testing.assert_array_equal(acc[0, ho, wo], exp)


def test_delta_filter_strided_asymmetric_pad():
    """56x56 stride-2 SAME has pads (0, 1): the last output row's third tap
    reads row 56, which is the zero bottom pad."""
    x = np.ones((1, 56, 56, 1), np.int8)
    w = np.zeros((3, 3, 1, 1), np.int8)
    w[2, 1, 0, 0] = 1
    acc = oracle.conv_acc(x, w, 2, "SAME")
    assert acc.shape == (1, 28, 28, 1)
    assert acc[0, 27, 5, 0] == 0 and acc[0, 26, 5, 0] == 1


def test_constant_closed_form():
    """x = a, w = b: acc = a*b*C*nr(ho)*ns(wo), nr counting in-image taps."""
    for (H, W, R, S, st) in [(10, 7, 3, 3, 1), (11, 11, 5, 5, 2), (56, 56, 3, 3, 2),
                             (4, 9, 7, 2, 3)]:
        a, b, C, K = 3, -5, 6, 2
        x = np.full((1, H, W, C), a, np.int8)
        w = np.full((R, S, C, K), b, np.int8)
        Ho, Wo, pt, _, pl, _ = oracle.geometry(H, W, R, S, st, st, True)
        acc = oracle.conv_acc(x, w, st, "SAME")
        for ho in range(Ho):
            nr = sum(1 for r in range(R) if 0 <= ho * st - pt + r < H)
            for wo in range(Wo):
                ns = sum(1 for s in range(S) if 0 <= wo * st - pl + s < W)
                assert acc[0, ho, wo, 0] == a * b * C * nr * ns


def test_linearity():
    rng = np.random.default_rng(9)
    x1 = wl.draw_int8(rng, (2, 9, 9, 8), -60, 60)
    x2 = wl.draw_int8(rng, (2, 9, 9, 8), -60, 60)
    w = wl.draw_int8(rng, (3, 3, 8, 5))
    s = (x1.astype(np.int16) + x2).astype(np.int8)
    np.testing.assert_array_equal(
        oracle.conv_acc(x1, w, 2, "SAME").astype(np.int64)
        + oracle.conv_acc(x2, w, 2, "SAME"),
        oracle.conv_acc(s, w, 2, "SAME"))


# ------------------------------------------------------------------ P-7


def test_size_formulas_grid():
    """SAME: Ho = ceil(H/stride); the padding total and its split follow the
    TensorFlow SAME comment (half before, the odd rest after), and the Im2col
    size expression returns Ho again.  VALID: zero pads, (H-R)/stride + 1.
    Stride 1 SAME also matches torch's padding='same' (odd rest after)."""
    for H in range(1, 65):
        for R in range(1, 8):
            for st in range(1, 5):
                Ho, _, pt, pb, _, _ = oracle.geometry(H, 5, R, 1, st, 1, True)
                assert Ho == math.ceil(H / st)
                assert pb - pt in (0, 1) and pt >= 0
                assert (H + pt + pb - R) // st + 1 == Ho
                # taps of the last output row stay within the bottom pad
                assert (Ho - 1) * st - pt + R - 1 <= H - 1 + pb
                if H >= R:
                    Hv, _, a, b, _, _ = oracle.geometry(H, 5, R, 1, st, 1, False)
                    assert (a, b) == (0, 0) and Hv == (H - R) // st + 1
                else:
                    with pytest.raises(oracle.OracleError):
                        oracle.geometry(H, 5, R, 1, st, 1, False)
    rng = np.random.default_rng(3)
    for R in range(1, 7):
        x = rng.standard_normal((1, 1, 9, 9))
        w = rng.standard_normal((1, 1, R, R))
        ref = F.conv2d(torch.from_numpy(x), torch.from_numpy(w), padding="same")
        ours = oracle.conv_acc(np.ascontiguousarray(x.transpose(0, 2, 3, 1), np.float32),
                               np.ascontiguousarray(w.transpose(2, 3, 1, 0), np.float32),
                               1, "SAME")
        np.testing.assert_allclose(
            ours[..., 0],
            F.conv2d(torch.from_numpy(x.astype(np.float32)).double(),
                     torch.from_numpy(w.astype(np.float32)).double(),
                     padding="same")[:, 0].numpy(), rtol=1e-12, atol=1e-12)
        assert ref.shape[-2:] == (9, 9)


def test_workload_geometries():
    """Output sizes and pads the workloads state: 56x56 stride-2 SAME gives 28
    with pads top/left 0, bottom/right 1; the stride-1 3x3 layers pad 1/1."""
    for L in wl.LAYERS.values():
        Ho, Wo, pt, pb, pl, pr = oracle.geometry(L.H, L.W, L.R, L.S, L.stride,
                                                 L.stride, L.padding == "SAME")
        assert (Ho, Wo) == (L.Ho, L.Wo)
    assert oracle.geometry(56, 56, 3, 3, 2, 2, True) == (28, 28, 0, 1, 0, 1)
    assert oracle.geometry(8, 8, 3, 3, 1, 1, True) == (8, 8, 1, 1, 1, 1)
    assert oracle.geometry(56, 56, 1, 1, 1, 1, False) == (56, 56, 0, 0, 0, 0)


# ------------------------------------------------------------------ P-8, P-9, P-10


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _single_pixel(acc_value, K=1):
    return np.full((1, 1, 1, K), acc_value, np.int32)


def test_epilogue_hand_values():
    rows = _read_rows("epilogue_i8_hand.txt")
    assert len(rows) >= 15
    for r in rows:
        acc, cis, side, sis, bias, relu, exp = r[:7]
        side_arr = None if side == "-" else np.full((1, 1, 1, 1), int(side), np.int8)
        y = oracle.epilogue_i8(_single_pixel(int(acc)), float(cis),
                               np.array([float(bias)], np.float32), side_arr,
                               float(sis), relu == "1")
        assert int(y[0, 0, 0, 0]) == int(exp), r


def test_epilogue_crafted_fma_and_contraction_cases():
    """T1 needs the side step fused; T2 needs scale and bias unfused.  Run
    through the full oracle convolution (1x1, single pixel)."""
    for name, C, xv, wv, cis, side, sis, bias, relu, exp in _read_rows(
            "epilogue_i8_crafted.txt"):
        C = int(C)
        x = np.full((1, 1, 1, C), int(xv), np.int8)
        w = np.full((1, 1, C, 1), int(wv), np.int8)
        side_arr = None if side == "-" else np.full((1, 1, 1, 1), int(side), np.int8)
        y = oracle.fused_conv_i8(x, w, np.array([float(bias)], np.float32),
                                 np.float32(float(cis)), side_arr,
                                 np.float32(float(sis)), relu == "1",
                                 padding="VALID")
        assert int(y[0, 0, 0, 0]) == int(exp), name


def test_epilogue_variant_hand_values():
    """Per-channel scale vectors and the cuDNN 7 order, hand-worked values
    (tests/golden/epilogue_i8_variants.txt)."""
    rows = _read_rows("epilogue_i8_variants.txt")
    assert len(rows) >= 7
    f32 = lambda t: np.array([float(v) for v in t.split(",")], np.float32)
    for r in rows:
        order, relu, sis, accs, scales, biases, sides, exp = r[:8]
        acc = np.array([int(v) for v in accs.split(",")], np.int32).reshape(1, 1, 1, -1)
        side = None if sides == "-" else np.array(
            [int(v) for v in sides.split(",")], np.int8).reshape(acc.shape)
        y = oracle.epilogue_i8(acc, f32(scales), f32(biases), side, float(sis),
                               relu == "1", order=int(order))
        assert y.reshape(-1).tolist() == [int(v) for v in exp.split(",")], r


def test_epilogue_cudnn7_order_fuses_scale_and_bias():
    """Crafted case T2 (epilogue_i8_crafted.txt) rounds differently when scale
    and bias are one fused multiply-add: 0 in the cuDNN 8 order, 1 in the
    cuDNN 7 order (5 * 838860.9375 - 4194304 = 0.6875 exactly)."""
    for name, C, xv, wv, cis, side, sis, bias, relu, exp in _read_rows(
            "epilogue_i8_crafted.txt"):
        if name != "T2":
            continue
        x = np.full((1, 1, 1, int(C)), int(xv), np.int8)
        w = np.full((1, 1, int(C), 1), int(wv), np.int8)
        b = np.array([float(bias)], np.float32)
        y8 = oracle.fused_conv_i8(x, w, b, np.float32(float(cis)), padding="VALID", order=8)
        y7 = oracle.fused_conv_i8(x, w, b, np.float32(float(cis)), padding="VALID", order=7)
        assert int(y8[0, 0, 0, 0]) == int(exp) == 0
        assert int(y7[0, 0, 0, 0]) == 1


def test_per_channel_scale_of_equal_values_is_the_scalar():
    rng = np.random.default_rng(14)
    x = wl.draw_int8(rng, (2, 7, 6, 24))
    w = wl.draw_int8(rng, (3, 3, 24, 20))
    side = wl.draw_int8(rng, (2, 7, 6, 20))
    acc = oracle.conv_acc(x, w, 1, "SAME")
    bias = rng.normal(0, 16, size=20).astype(np.float32)
    for order in (7, 8):
        for cis in (np.float32(2.0 ** -11), np.float32(0.0123)):
            ys = oracle.epilogue_i8(acc, cis, bias, side, 0.25, True, order)
            yv = oracle.epilogue_i8(acc, np.full(20, cis, np.float32), bias, side, 0.25,
                                    True, order)
            np.testing.assert_array_equal(ys, yv)


def _round_f32(q: Fraction) -> Fraction:
    """Exact value of the binary32 nearest to q (ties to even), from scratch."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 23, -149)
    n = round(a / quantum)  # Fraction.__round__: half to even
    v = n * quantum
    return v if q > 0 else -v


def _epilogue_exact(acc, cis, side, sis, bias, relu, order=8):
    t = _round_f32(Fraction(int(acc)))
    if order == 7:
        t = _round_f32(t * Fraction(float(cis)) + Fraction(float(bias)))
        if side is not None and sis != 0:
            t = _round_f32(Fraction(int(side)) * Fraction(float(sis)) + t)
    else:
        t = _round_f32(t * Fraction(float(cis)))
        if side is not None and sis != 0:
            t = _round_f32(Fraction(int(side)) * Fraction(float(sis)) + t)
        t = _round_f32(t + Fraction(float(bias)))
    v = round(t)  # half to even
    lo = 0 if relu else -128
    return max(lo, min(127, v))


def test_epilogue_against_exact_rational_model():
    """The oracle's fp32 steps equal exact rational arithmetic rounded to
    binary32 at each step, on random and tie-heavy data with scales that are
    not powers of two (so the rounding points matter)."""
    rng = np.random.default_rng(11)
    n = 4000
    acc = rng.integers(-2 ** 26, 2 ** 26, size=n).astype(np.int32)
    acc[: n // 4] = rng.integers(-600, 600, size=n // 4)
    side = wl.draw_int8(rng, (n,), -128, 127)
    cis = np.float32(rng.choice([2.0 ** -8, 0.0123, 1 / 3, 2.0 ** -11]))
    sis = np.float32(rng.choice([0.5, 0.377, 1 / 6, 0.0]))
    bias = rng.normal(0, 40, size=n).astype(np.float32)
    bias[: n // 8] = np.round(bias[: n // 8] * 2) / 2  # half-integers
    for relu in (False, True):
        for with_side in (False, True):
            y = np.empty(n, np.int8)
            for i in range(n):
                y[i] = oracle.epilogue_i8(_single_pixel(acc[i]), cis, bias[i:i + 1],
                                          side[i].reshape(1, 1, 1, 1) if with_side else None,
                                          sis, relu)[0, 0, 0, 0]
            exp = [_epilogue_exact(acc[i], cis, side[i] if with_side else None, sis,
                                   bias[i], relu) for i in range(n)]
            np.testing.assert_array_equal(y, np.array(exp, np.int8))


def test_epilogue_large_accumulators_against_exact_rational_model():
    """Accumulators between 2^24 and 2^31, where the int32 -> fp32 conversion
    rounds (odd values above 2^24 are ties), with biases that bring t back
    into the int8 range so that every rounding step shows in the output;
    both orders, against exact rational arithmetic rounded to binary32."""
    rng = np.random.default_rng(16)
    n = 3000
    mag = rng.integers(2 ** 24, 2 ** 27, size=n)
    mag[: n // 3] = rng.integers(2 ** 24, 2 ** 24 + 64, size=n // 3)
    mag[n // 3: n // 2] = rng.integers(2 ** 31 - 2 ** 20, 2 ** 31, size=n // 2 - n // 3)
    acc = (mag * rng.choice([-1, 1], size=n)).astype(np.int64)
    acc = np.clip(acc, -2 ** 31, 2 ** 31 - 1).astype(np.int32)
    side = wl.draw_int8(rng, (n,), -128, 127)
    for cis in (np.float32(0.5), np.float32(1.0), np.float32(0.7), np.float32(2.0 ** -3)):
        # bias = -(acc * cis) in fp32 plus a small offset: t lands near the
        # int8 range, so the conversion's rounding decides the result.
        off = rng.choice([0.0, 0.5, -0.5, 1.0, 3.25, -7.0, 100.0], size=n)
        bias = (-(acc.astype(np.float64) * float(cis)) + off).astype(np.float32)
        sis = np.float32(0.377)
        for order in (7, 8):
            for relu in (False, True):
                for with_side in (False, True):
                    y = oracle.epilogue_i8(acc.reshape(1, 1, 1, n), cis, bias,
                                           side.reshape(1, 1, 1, n) if with_side else None,
                                           sis, relu, order)
                    # bias is per channel: one channel per value here
                    exp = [_epilogue_exact(acc[i], cis, side[i] if with_side else None, sis,
                                           bias[i], relu, order) for i in range(n)]
                    np.testing.assert_array_equal(y.reshape(-1), np.array(exp, np.int8))
    # the construction puts most outputs strictly inside the range
    y = oracle.epilogue_i8(acc.reshape(1, 1, 1, n), np.float32(1.0),
                           (-acc.astype(np.float64)).astype(np.float32), None, 0.0, False)
    assert np.mean(np.abs(y.astype(int)) < 127) > 0.9


def test_epilogue_variants_against_exact_rational_model():
    """Both orders with a per-channel scale vector: the oracle's fp32 steps
    equal exact rational arithmetic rounded to binary32 at each step (in the
    cuDNN 7 order, scale and bias round once together)."""
    rng = np.random.default_rng(15)
    K, P = 16, 150
    acc = rng.integers(-2 ** 26, 2 ** 26, size=(P, K)).astype(np.int32)
    acc[: P // 3] = rng.integers(-600, 600, size=(P // 3, K))
    side = wl.draw_int8(rng, (P, K), -128, 127)
    scales = rng.choice([2.0 ** -8, 0.0123, 1 / 3, 2.0 ** -11, 0.7071], size=K).astype(np.float32)
    scales[0] = np.float32(838860.9375) / np.float32(2.0 ** 20)
    bias = rng.normal(0, 40, size=K).astype(np.float32)
    bias[: K // 4] = np.round(bias[: K // 4] * 2) / 2
    sis = np.float32(0.377)
    for order in (7, 8):
        for relu in (False, True):
            for with_side in (False, True):
                y = oracle.epilogue_i8(acc.reshape(1, 1, P, K), scales, bias,
                                       side.reshape(1, 1, P, K) if with_side else None,
                                       sis, relu, order).reshape(P, K)
                exp = [[_epilogue_exact(acc[p, k], scales[k], side[p, k] if with_side else None,
                                        sis, bias[k], relu, order) for k in range(K)]
                       for p in range(P)]
                np.testing.assert_array_equal(y, np.array(exp, np.int8))


def test_tie_dense_rounding_is_half_even():
    """bias 0, scale 0.5, no side: every odd accumulator is an exact .5 tie;
    the result is numpy's half-to-even rounding of acc/2, clipped."""
    rng = np.random.default_rng(12)
    x = wl.draw_int8(rng, (2, 6, 6, 8), -3, 3)
    w = wl.draw_int8(rng, (3, 3, 8, 16), -3, 3)
    acc = oracle.conv_acc(x, w, 1, "SAME")
    assert np.mean(acc % 2 != 0) > 0.3
    y = oracle.epilogue_i8(acc, 0.5, np.zeros(16, np.float32))
    np.testing.assert_array_equal(y, np.clip(np.round(acc / 2.0), -128, 127).astype(np.int8))


# ------------------------------------------------------------------ P-12


def test_float_epilogue_against_torch_batch_norm():
    """bias -> batch-norm inference -> ReLU equals torch's eval-mode
    batch_norm (float64) applied to acc + bias, then relu."""
    rng = np.random.default_rng(13)
    K = 12
    acc = rng.standard_normal((2, 3, 4, K))
    bias = rng.normal(0, 0.1, K).astype(np.float32)
    bn = dict(mean=rng.normal(0, 0.1, K).astype(np.float32),
              var=rng.uniform(0.5, 1.5, K).astype(np.float32),
              gamma=rng.uniform(0.5, 1.5, K).astype(np.float32),
              beta=rng.normal(0, 0.1, K).astype(np.float32), eps=1e-5)
    y = oracle.epilogue_float(acc, bias, bn, relu=True)
    t = torch.from_numpy(acc + bias.astype(np.float64)).permute(0, 3, 1, 2)
    ref = F.batch_norm(t, torch.from_numpy(bn["mean"]).double(),
                       torch.from_numpy(bn["var"]).double(),
                       torch.from_numpy(bn["gamma"]).double(),
                       torch.from_numpy(bn["beta"]).double(), training=False,
                       eps=bn["eps"])
    ref = torch.relu(ref).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # no ops at all: identity; bias only: plain add
    np.testing.assert_array_equal(oracle.epilogue_float(acc), acc)
    np.testing.assert_array_equal(oracle.epilogue_float(acc, bias),
                                  acc + bias.astype(np.float64))


@pytest.mark.parametrize("act,alpha,beta", [
    ("leaky_relu", 0.1, 0.0), ("leaky_relu", 0.0, 0.0), ("clipped_relu", 0.75, 0.0),
    ("clamp", -0.4, 0.6)])
def test_float_activations_against_torch(act, alpha, beta):
    """bias -> batch norm -> activation equals torch's eval-mode batch_norm
    followed by torch's own leaky_relu / hardtanh(0, alpha) / clamp, in
    float64, on data that crosses every threshold."""
    rng = np.random.default_rng(16)
    K = 10
    acc = rng.standard_normal((2, 5, 3, K)) * 2
    acc[0, 0, 0, :4] = [0.0, -0.0, alpha, beta]  # values on the thresholds
    bias = rng.normal(0, 0.1, K).astype(np.float32)
    bn = dict(mean=rng.normal(0, 0.1, K).astype(np.float32),
              var=rng.uniform(0.5, 1.5, K).astype(np.float32),
              gamma=rng.uniform(0.5, 1.5, K).astype(np.float32),
              beta=rng.normal(0, 0.1, K).astype(np.float32), eps=1e-5)
    for with_bn in (False, True):
        y = oracle.epilogue_float(acc, bias, bn if with_bn else None, act=act, alpha=alpha,
                                  beta=beta)
        t = torch.from_numpy(acc + bias.astype(np.float64)).permute(0, 3, 1, 2)
        if with_bn:
            t = F.batch_norm(t, torch.from_numpy(bn["mean"]).double(),
                             torch.from_numpy(bn["var"]).double(),
                             torch.from_numpy(bn["gamma"]).double(),
                             torch.from_numpy(bn["beta"]).double(), training=False,
                             eps=bn["eps"])
        a32 = float(np.float32(alpha))
        b32 = float(np.float32(beta))
        if act == "leaky_relu":
            ref = F.leaky_relu(t, negative_slope=a32)
        elif act == "clipped_relu":
            ref = F.hardtanh(t, 0.0, a32)
        else:
            ref = torch.clamp(t, a32, b32)
        ref = ref.permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_workload_accumulators_fit_int32():
    """The largest possible |acc| of the strided layer (127*127*1152) exceeds
    2^24 but fits int32; the oracle flags sums outside int32."""
    L = wl.LAYERS["resnet_3x3s2_int8"]
    assert 127 * 127 * L.R * L.S * L.C < 2 ** 31
    x = np.full((1, 1, 1, 140000), -128, np.int8)
    w = np.full((1, 1, 140000, 1), -128, np.int8)
    with pytest.raises(oracle.OracleError):
        oracle.conv_acc(x, w, 1, "VALID")


def test_workload_inputs_are_seeded_and_in_range():
    for L in wl.LAYERS.values():
        a = wl.make_inputs(L, N=1)
        b = wl.make_inputs(L, N=1)
        np.testing.assert_array_equal(a.x, b.x)
        assert a.x.shape == (1, L.H, L.W, L.C) and a.w.shape == (L.R, L.S, L.C, L.K)
        if L.dtype == "int8":
            assert a.x.min() >= L.x_range[0] and a.x.max() <= L.x_range[1]
            if L.has_side:
                assert a.side.shape == (1, L.Ho, L.Wo, L.K)


# ------------------------------------------------------ weight gradient


def _torch_wgrad(x64, dy64, R, S, stride, pads):
    """torch's conv2d_weight in float64 (NCHW); asymmetric pads by F.pad."""
    pt, pb, pl, pr = pads
    xt = F.pad(torch.from_numpy(x64).permute(0, 3, 1, 2), (pl, pr, pt, pb))
    gt = torch.from_numpy(dy64).permute(0, 3, 1, 2)
    g = torch.nn.grad.conv2d_weight(xt, (dy64.shape[-1], x64.shape[-1], R, S), gt,
                                    stride=stride, padding=0)
    return g.permute(2, 3, 1, 0).numpy()  # KCRS -> RSCK


@pytest.mark.parametrize("seed", range(12))
def test_wgrad_against_torch(seed):
    """The filter gradient equals torch.nn.grad.conv2d_weight (float64) on
    random shapes: strides 1-3, SAME (odd pads after) and VALID, filters
    larger than the image, float32 and bf16 inputs."""
    rng = np.random.default_rng(100 + seed)
    N, H, W = int(rng.integers(1, 3)), int(rng.integers(1, 9)), int(rng.integers(1, 9))
    C, K = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    R, S = int(rng.choice([1, 2, 3, 5])), int(rng.choice([1, 3, 4]))
    st = int(rng.integers(1, 4))
    same = seed % 3 != 0 or H < R or W < S
    g = oracle.geometry(H, W, R, S, st, st, same)
    x = rng.standard_normal((N, H, W, C)).astype(np.float32)
    dy = rng.standard_normal((N, g[0], g[1], K)).astype(np.float32)
    if seed % 2:
        x, dy = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(dy)
    dw = oracle.wgrad(x, dy, R, S, st, "SAME" if same else "VALID")
    ref = _torch_wgrad(oracle._as_f64(x), oracle._as_f64(dy), R, S, st, g[2:])
    np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-12)


def test_wgrad_of_a_delta_gradient_is_the_patch():
    """dY = 1 at one output position and channel, 0 elsewhere: dW[:, :, :, k]
    is the input patch under that position (zeros in the padding)."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((1, 6, 7, 3)).astype(np.float32)
    Ho, Wo, pt, pb, pl, pr = oracle.geometry(6, 7, 3, 3, 2, 2, True)
    for (ho, wo, k) in [(0, 0, 1), (Ho - 1, Wo - 1, 0), (1, 2, 2)]:
        dy = np.zeros((1, Ho, Wo, 3), np.float32)
        dy[0, ho, wo, k] = 1.0
        dw = oracle.wgrad(x, dy, 3, 3, 2, "SAME")
        xp = np.pad(x[0].astype(np.float64), ((pt, pb), (pl, pr), (0, 0)))
        patch = xp[2 * ho:2 * ho + 3, 2 * wo:2 * wo + 3, :]
        np.testing.assert_array_equal(dw[:, :, :, k], patch)
        assert not np.any(np.delete(dw, k, axis=3))
