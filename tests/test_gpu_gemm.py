"""GPU parity of the full-size VALID path (conv_gemm_*): a filter as large as
the image is the GEMM [N, H*W*C] x [H*W*C, K] of the fused op's second
special case (TensorFlow conv_ops_fused_int8.cc,
LaunchFusedConv2DOpCpuInt8Helper), run as a split reduction plus a
fixed-order sum with the fused epilogue.  int8 bit-exact (both epilogue
orders, side input, per-channel scales), bf16 / fp32 within the normwise
tolerances; several image tiles, ragged image and channel counts, one and
many reduction ranges; the sum of the ranges is deterministic."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import TOL, float_error, make_plan, run_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # N, H(=W=R=S), C, K
    (40, 7, 64, 200),    # two image tiles (ragged), K not a multiple of 64
    (33, 4, 96, 1000),   # K = 1000: ragged last channel tile
    (5, 5, 128, 72),     # few images, K % 16 = 8
    (70, 3, 256, 128),   # three image tiles
    (1, 1, 64, 64),      # 1x1 image: a single k-step per image
    (16, 2, 1024, 48),   # long rows, few channels: many ranges per tile
]


def _inputs(rng, N, H, C, K, dtype):
    if dtype == "int8":
        x = wl.draw_int8(rng, (N, H, H, C), -128, 127)
        w = wl.draw_int8(rng, (H, H, C, K), -128, 127)
        return x, w
    sd = 1.0 / np.sqrt(H * H * C)
    x = rng.normal(0, 1, (N, H, H, C)).astype(np.float32)
    w = rng.normal(0, sd, (H, H, C, K)).astype(np.float32)
    if dtype == "bf16":
        x, w = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(w)
    return x, w


@pytest.mark.parametrize("case", CASES, ids=["x".join(map(str, c)) for c in CASES])
@pytest.mark.parametrize("dtype", ["int8", "bf16", "fp32"])
def test_gemm_valid_shapes(case, dtype):
    N, H, C, K = case
    rng = np.random.default_rng(N * 7919 + H * 101 + C + K)
    x, w = _inputs(rng, N, H, C, K, dtype)
    bias = rng.normal(0, 20 if dtype == "int8" else 0.1, K).astype(np.float32)
    if dtype == "int8":
        ops = [wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS, wl.OP_RELU]
        side = wl.draw_int8(rng, (N, 1, 1, K), -128, 127)
        cis, sis = np.float32(1.0 / (H * H * C * 4)), np.float32(0.5)
        plan = make_plan(N, H, H, C, K, H, H, 1, "VALID", dtype, ops)
        assert plan.kernel_name == "conv_gemm_i8", plan.kernel_name
        say("gemm %s %s ws %d" % (dtype, case, plan.workspace_bytes))
        y, guards = run_gpu(plan, dtype, x, w, bias, side, cis, sis, guard=64)
        r = oracle.fused_conv_i8(x, w, bias, cis, side, sis, True, 1, "VALID")
        assert guards
        assert np.array_equal(y, r), "%d differ" % np.count_nonzero(y != r)
        return
    bn = dict(mean=rng.normal(0, .1, K).astype(np.float32),
              var=rng.uniform(.5, 1.5, K).astype(np.float32),
              gamma=rng.uniform(.5, 1.5, K).astype(np.float32),
              beta=rng.normal(0, .1, K).astype(np.float32), eps=1e-5)
    plan = make_plan(N, H, H, C, K, H, H, 1, "VALID", dtype, [wl.OP_BIAS, wl.OP_BN, wl.OP_RELU])
    assert plan.kernel_name == "conv_gemm_" + ("bf16" if dtype == "bf16" else "f32")
    say("gemm %s %s ws %d" % (dtype, case, plan.workspace_bytes))
    y, guards = run_gpu(plan, dtype, x, w, bias, None, bn=bn, guard=64)
    r = oracle.fused_conv_float(x, w, bias, bn, True, 1, "VALID")
    assert guards
    e = float_error(y, r)
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("order", [8, 7])
def test_gemm_epilogue_variants(order):
    """Per-channel conv_input_scale and both epilogue orders, no ReLU."""
    rng = np.random.default_rng(77 + order)
    N, H, C, K = 24, 6, 64, 320
    x, w = _inputs(rng, N, H, C, K, "int8")
    bias = rng.normal(0, 30, K).astype(np.float32)
    side = wl.draw_int8(rng, (N, 1, 1, K), -128, 127)
    cis = rng.choice([2.0 ** -14, 1.0 / 9000, 2.0 ** -13], size=K).astype(np.float32)
    sis = np.float32(0.377)
    plan = make_plan(N, H, H, C, K, H, H, 1, "VALID", "int8",
                     [wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS], cudnn7_order=(order == 7))
    assert plan.kernel_name == "conv_gemm_i8"
    y, guards = run_gpu(plan, "int8", x, w, bias, side, cis, sis, guard=64)
    r = oracle.fused_conv_i8(x, w, bias, cis, side, sis, False, 1, "VALID", order=order)
    assert guards
    assert np.array_equal(y, r), "%d differ" % np.count_nonzero(y != r)


def test_gemm_is_deterministic():
    """The ranges are summed in a fixed order: two runs give the same bits."""
    L = wl.LAYERS["valid_7x7_bf16"]
    inp = wl.make_inputs(L, N=8)
    plan = make_plan(8, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops)
    a, _ = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, None, bn=inp.bn)
    b, _ = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, None, bn=inp.bn)
    assert np.array_equal(a, b)


def test_gemm_back_to_back_runs():
    """Twelve runs with different inputs queued back to back on one stream,
    no host wait between them, over a workspace filled with garbage before
    the filter was packed (every fourth run repacks it): each run rewrites
    every partial tile it sums, so every run's int8 output must equal the
    oracle's bit for bit."""
    rng = np.random.default_rng(4242)
    N, H, C, K = 64, 4, 256, 512
    dev = torch.device("cuda:0")
    ops = [wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS, wl.OP_RELU]
    plan = make_plan(N, H, H, C, K, H, H, 1, "VALID", "int8", ops)
    assert plan.kernel_name == "conv_gemm_i8"
    w = wl.draw_int8(rng, (H, H, C, K), -128, 127)
    bias = rng.normal(0, 20, K).astype(np.float32)
    cis, sis = np.float32(1.0 / (H * H * C * 4)), np.float32(0.5)
    ws = torch.full((plan.workspace_bytes,), 0x5A, dtype=torch.uint8, device=dev)
    wd = torch.from_numpy(w).to(dev)
    plan.pack_filter(wd, ws)
    bd = torch.from_numpy(bias).to(dev)
    runs = []
    for i in range(12):
        x = wl.draw_int8(rng, (N, H, H, C), -128, 127)
        side = wl.draw_int8(rng, (N, 1, 1, K), -128, 127)
        xd, sd = torch.from_numpy(x).to(dev), torch.from_numpy(side).to(dev)
        y = torch.empty(plan.out_shape, dtype=torch.int8, device=dev)
        plan.run(xd, wd, y, ws, bias=bd, side=sd, conv_input_scale=float(cis),
                 side_input_scale=float(sis), prepacked=(i % 4 != 3))
        runs.append((x, side, xd, sd, y))
    torch.cuda.synchronize()
    say("gemm back-to-back: 12 runs of %s queued, workspace %d B" % ((N, H, C, K), plan.workspace_bytes))
    for i, (x, side, _, _, y) in enumerate(runs):
        r = oracle.fused_conv_i8(x, w, bias, cis, side, sis, True, 1, "VALID")
        got = y.cpu().numpy()
        assert np.array_equal(got, r), "run %d: %d differ" % (i, np.count_nonzero(got != r))
