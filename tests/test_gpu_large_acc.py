"""GPU parity of the int8 epilogue at the ends of the accumulator range.

Random data keeps |acc| near 10^5, where every int32 converts to fp32
exactly and t stays small.  These crafted layers push the accumulators as far
as each kernel family's reduction allows:

  * above 2^24 (3x3 over 128 channels, 1x1 over 1152), where the int32 ->
    fp32 conversion rounds and every odd accumulator is a tie, so a
    conversion that does not round half to even changes outputs;
  * close to the family's maximum otherwise (3x3 over 64 channels and 1x1
    over 512 stay below 2^24);

with biases that bring t back into the int8 range (so the conversion's
rounding decides the result) or that leave |t| far beyond 2^22 (the clip
path).  Every family, both epilogue orders, with and without ReLU and the
side input; int8 outputs bit-exact against the oracle (TensorFlow
conv_ops_fused_int8.cc, BiasActivationOutputKernel).

Construction: x is -128 in every channel except channel c0, which is -128 or
-127 at random; w is in {-128, -127} (positive products) or {127, 126}
(negative products) per output channel, except w[..., c0, :] = 1.  Every
product outside c0 is even, so the parity of acc is that of the number of
taps whose c0 value is -127, and interior pixels of one channel differ by at
most R*S: the per-channel bias moves them all near zero at once.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import make_plan, run_gpu, say
import workloads as wl

pytestmark = pytest.mark.gpu


def large_acc_inputs(rng, N, H, W, C, K, R, stride, pad):
    c0 = int(rng.integers(0, C))
    x = np.full((N, H, W, C), -128, np.int8)
    x[..., c0] = rng.choice(np.array([-128, -127], np.int8), size=(N, H, W))
    neg = rng.random(K) < 0.5  # output channels with negative accumulators
    w = rng.choice(np.array([-128, -127], np.int8), size=(R, R, C, K))
    wn = rng.choice(np.array([127, 126], np.int8), size=(R, R, C, K))
    w[..., neg] = wn[..., neg]
    w[:, :, c0, :] = 1
    acc = oracle.conv_acc(x, w, stride, pad)
    return x, w, acc


def biases(rng, acc, cis, mode):
    """Per-channel bias: "centre" moves the channel's median t to a small
    offset (the conversion's rounding shows in the int8 result); "far" leaves
    t beyond 2^22 in magnitude or sets it there explicitly."""
    K = acc.shape[-1]
    med = np.median(acc.reshape(-1, K).astype(np.float64), axis=0)
    if mode == "centre":
        off = rng.choice([0.0, 0.5, -0.5, 1.0, 2.5, -3.0, 60.0, -60.0], size=K)
        return (-(med * float(cis)) + off).astype(np.float32)
    far = rng.choice([0.0, 2.0 ** 22, -(2.0 ** 22), 3 * 2.0 ** 22, -3 * 2.0 ** 22,
                      2.0 ** 24, -(2.0 ** 24)], size=K)
    return (-(med * float(cis)) * (rng.random(K) < 0.5) + far).astype(np.float32)


# (family, shape (N, H, W, C, K, R, stride, padding), forced variant, tile
# height); the kernel name must start with "conv_" + family.
FAMILIES = [
    ("halo", (3, 10, 12, 64, 64, 3, 1, "SAME"), None, None),
    ("stream", (2, 9, 11, 512, 64, 1, 1, "VALID"), None, None),
    ("stream", (3, 10, 12, 64, 64, 3, 1, "SAME"), "stream", None),
    ("halo_s2", (3, 15, 15, 128, 128, 3, 2, "SAME"), None, None),
    ("halo_s2", (3, 15, 15, 64, 128, 3, 2, "SAME"), None, None),
    ("tile", (3, 15, 15, 128, 128, 3, 2, "SAME"), "tile", "64"),
    ("tile", (3, 15, 15, 128, 128, 3, 2, "SAME"), "tile", "128"),
    ("tile", (3, 15, 15, 128, 128, 3, 2, "SAME"), "tile", "256"),
    ("tile", (2, 9, 13, 128, 64, 3, 1, "SAME"), "tile", None),
    ("tile", (2, 7, 9, 1152, 64, 1, 1, "VALID"), None, None),
    ("rf", (3, 15, 15, 128, 128, 3, 2, "SAME"), "rf", None),
    ("rf", (2, 7, 9, 1152, 64, 1, 1, "VALID"), "rf", None),
    ("general", (3, 15, 15, 128, 128, 3, 2, "SAME"), "general", None),
    ("general", (2, 7, 9, 1152, 48, 1, 1, "VALID"), "general", None),
]


@pytest.mark.parametrize("mode", ["centre", "far"])
@pytest.mark.parametrize("order", [8, 7])
@pytest.mark.parametrize("fi", range(len(FAMILIES)),
                         ids=["%s-%s" % (f[0], "x".join(map(str, f[1][:6]))) + (
                             "-bm%s" % f[3] if f[3] else "") for f in FAMILIES])
def test_large_accumulators_bit_exact(fi, order, mode, monkeypatch):
    family, (N, H, W, C, K, R, stride, pad), force, bm = FAMILIES[fi]
    if force:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", force)
    if bm:
        monkeypatch.setenv("FCONV_TILE_BM", bm)
    rng = np.random.default_rng(1000 * fi + 10 * order + (mode == "far"))
    x, w, acc = large_acc_inputs(rng, N, H, W, C, K, R, stride, pad)
    Ho, Wo = acc.shape[1:3]
    amax = int(np.abs(acc.astype(np.int64)).max())
    if C * R * R >= 1152:
        assert amax > 2 ** 24  # the conversion rounds on these layers
        big = np.abs(acc.astype(np.int64)) > 2 ** 24
        assert np.mean(acc[big] % 2 != 0) > 0.2  # odd accumulators are ties there
    for sub, (cis, relu, use_side, sis) in enumerate([
            (0.5, False, False, 0.0), (1.0, True, True, 0.5), (0.7, False, True, 0.377),
            (2.0 ** -3, True, False, 0.0)]):
        cis = np.float32(cis)
        bias = biases(rng, acc, cis, mode)
        side = wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if use_side else None
        ops = [wl.OP_SCALE] + ([wl.OP_SIDE] if use_side else []) + [wl.OP_BIAS] + (
            [wl.OP_RELU] if relu else [])
        plan = make_plan(N, H, W, C, K, R, R, stride, pad, "int8", ops,
                         cudnn7_order=(order == 7))
        assert plan.kernel_name.startswith("conv_" + family), plan.kernel_name
        say("large acc %s %s order %d mode %s sub %d max|acc| %d" % (
            plan.kernel_name, (N, H, W, C, K, R, stride, pad), order, mode, sub, amax))
        y, guards = run_gpu(plan, "int8", x, w, bias, side, cis, np.float32(sis), guard=64)
        assert guards, "write outside y"
        r = oracle.fused_conv_i8(x, w, bias, cis, side, np.float32(sis), relu, stride, pad,
                                 order=order)
        bad = np.count_nonzero(y != r)
        assert bad == 0, "%d of %d outputs differ (sub-case %d)" % (bad, r.size, sub)
        if mode == "centre":  # the rounding shows in the result, not clipped away
            inside = np.mean((r > (0 if relu else -128)) & (r < 127))
            assert inside > 0.1, inside
