"""GPU parity: the HIP path through the C ABI against the CPU oracle.

int8 outputs must be bit-exact; bf16 and fp32 must be within the normwise
tolerances in gpu_helpers.TOL of the float64 oracle fed the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import (TOL, device, float_error, make_plan, oracle_out, run_gpu, say,
                         to_dev)

pytestmark = pytest.mark.gpu


def _layer_case(L, N=None):
    inp = wl.make_inputs(L, N=N)
    n = inp.x.shape[0]
    plan = make_plan(n, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops)
    return inp, plan


def _check_layer(L, N=None, prepacked=False):
    inp, plan = _layer_case(L, N)
    say("layer %s N=%d kernel=%s prepacked=%s" % (L.name, inp.x.shape[0], plan.kernel_name,
                                                   prepacked))
    ws = None
    if prepacked:
        dev = device()
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        plan.pack_filter(to_dev(inp.w, dev), ws)
    y, guards = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, inp.side,
                        L.conv_input_scale, L.side_input_scale, inp.bn, prepacked_ws=ws,
                        guard=256)
    assert guards, "write outside y"
    r = oracle_out(L.dtype, inp.x, inp.w, L.stride, L.padding, inp.bias, inp.side,
                   L.conv_input_scale, L.side_input_scale, L.relu, inp.bn,
                   use_bias=wl.OP_BIAS in L.ops)
    if L.dtype == "int8":
        bad = np.count_nonzero(y != r)
        assert bad == 0, "%d of %d int8 outputs differ" % (bad, r.size)
    else:
        e = float_error(y, r)
        say("  normwise error %.3e (tolerance %.0e)" % (e, TOL[L.dtype]))
        assert e <= TOL[L.dtype]
    return y


@pytest.mark.parametrize("name", list(wl.LAYERS))
def test_workload_full_size(name):
    _check_layer(wl.LAYERS[name])


@pytest.mark.parametrize("name", ["resnet_3x3_int8", "resnet_1x1_int8", "resnet_3x3s2_int8",
                                  "resnet_3x3_bf16_bn"])
def test_workload_prepacked_filter(name):
    """The launch configuration the benchmark times: filter packed once."""
    _check_layer(wl.LAYERS[name], prepacked=True)


def _random_case(rng, dtype):
    p = wl.random_small_case(rng)
    N, H, W, C, K, R, S, st, pad = (p[k] for k in ("N", "H", "W", "C", "K", "R", "S",
                                                  "stride", "padding"))
    Ho, Wo = oracle.geometry(H, W, R, S, st, st, pad == "SAME")[:2]
    if dtype == "int8":
        x = wl.draw_int8(rng, (N, H, W, C), -128, 127)
        w = wl.draw_int8(rng, (R, S, C, K), -128, 127)
        bias = rng.normal(0, 30, K).astype(np.float32)
        use_side = rng.random() < 0.5
        side = wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if use_side else None
        relu = bool(rng.random() < 0.5)
        cis = np.float32(rng.choice([2.0 ** -8, 0.0123, 1 / 3, 1.0, 2.0 ** -11]))
        sis = np.float32(rng.choice([0.5, 0.377, 0.0, 1.0])) if use_side else np.float32(0)
        ops = [wl.OP_SCALE] + ([wl.OP_SIDE] if use_side else []) + [wl.OP_BIAS] + (
            [wl.OP_RELU] if relu else [])
        return dict(shape=(N, H, W, C, K, R, S, st, pad), x=x, w=w, bias=bias, side=side,
                    cis=cis, sis=sis, relu=relu, ops=ops, bn=None, use_bias=True)
    sd = 1.0 / np.sqrt(R * S * C)
    x = rng.normal(0, 1, (N, H, W, C)).astype(np.float32)
    w = rng.normal(0, sd, (R, S, C, K)).astype(np.float32)
    if dtype == "bf16":
        x, w = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(w)
    use_bias = bool(rng.random() < 0.7)
    use_bn = bool(rng.random() < 0.6)
    relu = bool(rng.random() < 0.5)
    bias = rng.normal(0, 0.1, K).astype(np.float32)
    bn = dict(mean=rng.normal(0, 0.1, K).astype(np.float32),
              var=rng.uniform(0.5, 1.5, K).astype(np.float32),
              gamma=rng.uniform(0.5, 1.5, K).astype(np.float32),
              beta=rng.normal(0, 0.1, K).astype(np.float32), eps=1e-5) if use_bn else None
    ops = ([wl.OP_BIAS] if use_bias else []) + ([wl.OP_BN] if use_bn else []) + (
        [wl.OP_RELU] if relu else [])
    return dict(shape=(N, H, W, C, K, R, S, st, pad), x=x, w=w, bias=bias, side=None,
                cis=1.0, sis=0.0, relu=relu, ops=ops, bn=bn, use_bias=use_bias)


def _run_case(c, dtype):
    N, H, W, C, K, R, S, st, pad = c["shape"]
    plan = make_plan(N, H, W, C, K, R, S, st, pad, dtype, c["ops"])
    y, guards = run_gpu(plan, dtype, c["x"], c["w"], c["bias"], c["side"], c["cis"], c["sis"],
                        c["bn"], guard=64)
    r = oracle_out(dtype, c["x"], c["w"], st, pad, c["bias"], c["side"], c["cis"], c["sis"],
                   c["relu"], c["bn"], c["use_bias"])
    return y, r, guards, plan


@pytest.mark.parametrize("dtype,count,seed", [("int8", 160, 100), ("bf16", 50, 200),
                                              ("fp32", 50, 300)])
def test_fuzz_small_shapes(dtype, count, seed):
    """Random small layers: C, K not multiples of 16, filters 1-5, strides 1-3,
    SAME/VALID, images smaller than the filter; several tiles and ragged tails."""
    rng = np.random.default_rng(seed)
    say("fuzz %s: %d cases" % (dtype, count))
    for i in range(count):
        c = _random_case(rng, dtype)
        y, r, guards, plan = _run_case(c, dtype)
        where = "case %d %s %s" % (i, c["shape"], plan.kernel_name)
        assert guards, where
        if dtype == "int8":
            assert np.array_equal(y, r), where + ": %d differ" % np.count_nonzero(y != r)
        else:
            tol = TOL[dtype] if dtype == "bf16" else 2e-6
            assert float_error(y, r) <= tol, where


@pytest.mark.parametrize("C,K,H,W,R,stride,pad", [
    (64, 64, 9, 13, 3, 1, "SAME"), (128, 128, 11, 11, 3, 2, "SAME"),
    (256, 64, 7, 9, 1, 1, "VALID"), (16, 32, 17, 5, 3, 1, "SAME"), (48, 80, 6, 6, 5, 2, "SAME"),
    (64, 8, 4, 4, 3, 1, "VALID"), (256, 256, 5, 5, 3, 1, "SAME"), (32, 200, 3, 70, 2, 3, "SAME")])
@pytest.mark.parametrize("dtype", ["int8", "bf16", "fp32"])
def test_tile_shapes(C, K, H, W, R, stride, pad, dtype):
    """Channel counts on and off the vector widths, several 64-channel blocks,
    ragged pixel tails."""
    check_case(tile_case(C, K, H, W, R, stride, pad, dtype), dtype)


def tile_case(C, K, H, W, R, stride, pad, dtype):
    """Seeded inputs of one layer: int8 with side input and bias, or bf16 /
    fp32 with bias, batch norm and ReLU."""
    rng = np.random.default_rng(C * 1000 + K)
    Ho, Wo = oracle.geometry(H, W, R, R, stride, stride, pad == "SAME")[:2]
    N = 3
    if dtype == "int8":
        x = wl.draw_int8(rng, (N, H, W, C), -128, 127)
        w = wl.draw_int8(rng, (R, R, C, K), -128, 127)
        side = wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127)
        c = dict(shape=(N, H, W, C, K, R, R, stride, pad), x=x, w=w,
                 bias=rng.normal(0, 50, K).astype(np.float32), side=side,
                 cis=np.float32(2.0 ** -9), sis=np.float32(0.75), relu=False,
                 ops=[wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS], bn=None, use_bias=True)
    else:
        x = rng.normal(0, 1, (N, H, W, C)).astype(np.float32)
        w = rng.normal(0, 1 / np.sqrt(R * R * C), (R, R, C, K)).astype(np.float32)
        if dtype == "bf16":
            x, w = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(w)
        bn = dict(mean=rng.normal(0, .1, K).astype(np.float32),
                  var=rng.uniform(.5, 1.5, K).astype(np.float32),
                  gamma=rng.uniform(.5, 1.5, K).astype(np.float32),
                  beta=rng.normal(0, .1, K).astype(np.float32), eps=1e-5)
        c = dict(shape=(N, H, W, C, K, R, R, stride, pad), x=x, w=w,
                 bias=rng.normal(0, .1, K).astype(np.float32), side=None, cis=1.0, sis=0.0,
                 relu=True, ops=[wl.OP_BIAS, wl.OP_BN, wl.OP_RELU], bn=bn, use_bias=True)
    return c


def check_case(c, dtype, fp32_tol=2e-6):
    """Run one case on the GPU against the oracle (int8 bit-exact, bf16 2e-2,
    fp32 2e-6 normwise for reductions up to a few thousand terms, else the
    general TOL["fp32"]); returns the plan's kernel."""
    say("tile shape %s %s" % (dtype, c["shape"]))
    y, r, guards, plan = _run_case(c, dtype)
    assert guards
    if dtype == "int8":
        assert np.array_equal(y, r), "%d differ" % np.count_nonzero(y != r)
    else:
        assert float_error(y, r) <= (TOL["bf16"] if dtype == "bf16" else fp32_tol)
    return plan.kernel_name


def test_crafted_fma_and_contraction_cases():
    """T1 (side step must be one fused multiply-add) and T2 (scale and bias
    must not be contracted), single-pixel 1x1 convolutions."""
    for C, xv, wv, cis, side, sis, bias, exp in [
            (2, 64, 64, 1024.0, 3, 0.1666666716337204, -8388608.0, 1),
            (1, 5, 1, 838860.9375, None, 0.0, -4194304.0, 0)]:
        x = np.full((1, 1, 1, C), xv, np.int8)
        w = np.full((1, 1, C, 1), wv, np.int8)
        s = None if side is None else np.full((1, 1, 1, 1), side, np.int8)
        ops = [wl.OP_SCALE] + ([wl.OP_SIDE] if s is not None else []) + [wl.OP_BIAS]
        plan = make_plan(1, 1, 1, C, 1, 1, 1, 1, "VALID", "int8", ops)
        y, _ = run_gpu(plan, "int8", x, w, np.array([bias], np.float32), s, np.float32(cis),
                       np.float32(sis))
        assert int(y[0, 0, 0, 0]) == exp


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("variant", [None, "stream", "rf", "general"])
def test_tie_dense_round_half_even(relu, variant, monkeypatch):
    """scale 0.5, bias 0, no side: every odd accumulator is an exact tie, on
    both sides of zero (ReLU: ties at 0.5 and above round to even, below
    clip to 0), in the default kernel for the shape (row-halo) and the
    others."""
    if variant:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", variant)
    rng = np.random.default_rng(21)
    x = wl.draw_int8(rng, (4, 12, 12, 64), -9, 9)
    w = wl.draw_int8(rng, (3, 3, 64, 64), -9, 9)
    plan = make_plan(4, 12, 12, 64, 64, 3, 3, 1, "SAME", "int8",
                     [wl.OP_SCALE, wl.OP_BIAS] + ([wl.OP_RELU] if relu else []))
    assert plan.kernel_name.startswith("conv_" + (variant or "halo")), plan.kernel_name
    bias = np.zeros(64, np.float32)
    y, _ = run_gpu(plan, "int8", x, w, bias, None, 0.5)
    acc = oracle.conv_acc(x, w, 1, "SAME")
    assert np.mean(acc % 2 != 0) > 0.3
    lo = 0 if relu else -128
    assert np.array_equal(y, np.clip(np.round(acc / 2.0), lo, 127).astype(np.int8))


def test_zero_side_scale_skips_side():
    rng = np.random.default_rng(22)
    x = wl.draw_int8(rng, (2, 9, 9, 32))
    w = wl.draw_int8(rng, (3, 3, 32, 32))
    side = wl.draw_int8(rng, (2, 9, 9, 32))
    bias = rng.normal(0, 20, 32).astype(np.float32)
    plan = make_plan(2, 9, 9, 32, 32, 3, 3, 1, "SAME", "int8",
                     [wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS, wl.OP_RELU])
    y, _ = run_gpu(plan, "int8", x, w, bias, side, 2.0 ** -10, 0.0)
    r = oracle.fused_conv_i8(x, w, bias, 2.0 ** -10, None, 0.0, True, 1, "SAME")
    assert np.array_equal(y, r)


def test_run_twice_is_bit_identical():
    L = wl.LAYERS["resnet_3x3_bf16_bn"]
    inp, plan = _layer_case(L, N=2)
    a, _ = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, None, bn=inp.bn)
    b, _ = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, None, bn=inp.bn)
    assert np.array_equal(a, b)


def test_empty_batch_is_a_no_op():
    dev = device()
    plan = make_plan(0, 8, 8, 16, 16, 3, 3, 1, "SAME", "int8", [wl.OP_SCALE, wl.OP_BIAS])
    x = torch.zeros(16, dtype=torch.int8, device=dev)
    y = torch.full((16,), 7, dtype=torch.int8, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    w = torch.zeros(3 * 3 * 16 * 16, dtype=torch.int8, device=dev)
    b = torch.zeros(16, dtype=torch.float32, device=dev)
    plan.run(x, w, y, ws, bias=b)
    torch.cuda.synchronize()
    assert (y.cpu() == 7).all()


def test_pack_filter_then_prepacked_run_matches():
    rng = np.random.default_rng(23)
    dev = device()
    for dtype in ("int8", "bf16", "fp32"):
        C, K = 48, 72
        plan = make_plan(2, 7, 7, C, K, 3, 3, 1, "SAME", dtype,
                         [wl.OP_SCALE, wl.OP_BIAS] if dtype == "int8" else [wl.OP_BIAS])
        if dtype == "int8":
            x, w = wl.draw_int8(rng, (2, 7, 7, C)), wl.draw_int8(rng, (3, 3, C, K))
        else:
            x = rng.normal(0, 1, (2, 7, 7, C)).astype(np.float32)
            w = rng.normal(0, .1, (3, 3, C, K)).astype(np.float32)
            if dtype == "bf16":
                x, w = wl.float_to_bf16_bits(x), wl.float_to_bf16_bits(w)
        bias = rng.normal(0, 1, K).astype(np.float32)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        plan.pack_filter(to_dev(w, dev), ws)
        a, _ = run_gpu(plan, dtype, x, w, bias, None, 2.0 ** -8, prepacked_ws=ws)
        b, _ = run_gpu(plan, dtype, x, w, bias, None, 2.0 ** -8)
        assert np.array_equal(a, b), dtype


@pytest.mark.parametrize("N,H,W,K,pad,side,rows", [
    (5, 7, 9, 64, "SAME", True, 0),      # one output row per workgroup
    (3, 1, 1, 64, "SAME", True, 0),      # 1x1 images: all but the centre tap in padding
    (2, 13, 62, 128, "SAME", True, 0),   # widest padded row (64 pixels), two channel slices
    (7, 5, 6, 80, "VALID", True, 0),     # K not a multiple of 64, VALID
    (1, 3, 3, 16, "SAME", False, 0),     # K = 16, no side input
    (100, 5, 5, 64, "SAME", True, 0),    # several rows per workgroup, rows span images
    (300, 3, 3, 64, "SAME", True, 0),    # workgroups span up to three images
    (600, 1, 8, 64, "SAME", True, 0),    # one-row images: every workgroup row is a new image
    (2, 3, 20, 64, "VALID", True, 0),    # Ho = 1 with VALID padding
    (6, 9, 11, 64, "SAME", True, 5),     # forced 5 rows per workgroup
    (4, 16, 16, 64, "SAME", True, 13),   # forced 13 rows: ragged last workgroup
])
def test_halo_shapes(N, H, W, K, pad, side, rows, monkeypatch):
    """Row-halo kernel edge cases: padding rows and columns, image changes
    inside a workgroup's rows, ragged pixel and channel tails."""
    if rows:
        monkeypatch.setenv("FCONV_HALO_ROWS", str(rows))
    rng = np.random.default_rng(N * 1000 + H * 10 + K)
    Ho, Wo = oracle.geometry(H, W, 3, 3, 1, 1, pad == "SAME")[:2]
    x = wl.draw_int8(rng, (N, H, W, 64), -128, 127)
    w = wl.draw_int8(rng, (3, 3, 64, K), -128, 127)
    sd = wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if side else None
    ops = [wl.OP_SCALE] + ([wl.OP_SIDE] if side else []) + [wl.OP_BIAS, wl.OP_RELU]
    c = dict(shape=(N, H, W, 64, K, 3, 3, 1, pad), x=x, w=w,
             bias=rng.normal(0, 40, K).astype(np.float32), side=sd,
             cis=np.float32(2.0 ** -10), sis=np.float32(0.5 if side else 0.0), relu=True,
             ops=ops, bn=None, use_bias=True)
    say("halo shape %s side=%s rows=%d" % (c["shape"], side, rows))
    y, r, guards, plan = _run_case(c, "int8")
    assert plan.kernel_name == "conv_halo_i8", plan.kernel_name
    assert guards
    assert np.array_equal(y, r), "%d differ" % np.count_nonzero(y != r)


@pytest.mark.parametrize("N,H,W,C,K,pad,side,relu,rows", [
    (5, 9, 9, 128, 128, "SAME", True, True, 0),      # odd size: top and left pad 1
    (3, 8, 10, 64, 128, "SAME", True, True, 0),      # 64 channels, top pad 0
    (2, 62, 62, 128, 256, "SAME", True, False, 0),   # Wo = 31 (widest), two channel slices
    (7, 11, 6, 128, 128, "VALID", True, True, 0),    # VALID, Wo = 2
    (4, 1, 1, 64, 128, "SAME", False, True, 0),      # 1x1 images: all but one tap in padding
    (300, 3, 3, 128, 128, "SAME", True, True, 0),    # Ho = 2: workgroups span many images
    (6, 13, 13, 128, 128, "SAME", True, False, 5),   # forced 5 rows per workgroup, no ReLU
    (4, 16, 16, 64, 128, "SAME", True, True, 13),    # forced 13 rows: ragged last workgroup
])
def test_halo_s2_shapes(N, H, W, C, K, pad, side, relu, rows, monkeypatch):
    """The stride-2 row kernel's edge cases: both SAME paddings of stride 2
    (top/left 0 or 1), VALID, images smaller than the filter, workgroups whose
    rows span images, ragged last workgroups, both channel counts, with and
    without the side input and ReLU."""
    if rows:
        monkeypatch.setenv("FCONV_HALO_ROWS", str(rows))
    rng = np.random.default_rng(N * 1000 + H * 10 + C + K)
    Ho, Wo = oracle.geometry(H, W, 3, 3, 2, 2, pad == "SAME")[:2]
    x = wl.draw_int8(rng, (N, H, W, C), -128, 127)
    w = wl.draw_int8(rng, (3, 3, C, K), -128, 127)
    sd = wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if side else None
    ops = [wl.OP_SCALE] + ([wl.OP_SIDE] if side else []) + [wl.OP_BIAS] + (
        [wl.OP_RELU] if relu else [])
    c = dict(shape=(N, H, W, C, K, 3, 3, 2, pad), x=x, w=w,
             bias=rng.normal(0, 40, K).astype(np.float32), side=sd,
             cis=np.float32(2.0 ** -11), sis=np.float32(0.5 if side else 0.0), relu=relu,
             ops=ops, bn=None, use_bias=True)
    say("halo_s2 shape %s side=%s relu=%s rows=%d" % (c["shape"], side, relu, rows))
    y, r, guards, plan = _run_case(c, "int8")
    assert plan.kernel_name == "conv_halo_s2_i8", plan.kernel_name
    assert guards
    assert np.array_equal(y, r), "%d differ" % np.count_nonzero(y != r)


def test_halo_s2_falls_back_past_31_output_columns():
    """Wo = 32 needs a 65-pixel input row: the tiled kernel takes it."""
    plan = make_plan(1, 4, 64, 128, 128, 3, 3, 2, "SAME", "int8",
                     [wl.OP_SCALE, wl.OP_BIAS, wl.OP_RELU])
    assert plan.Wo == 32 and plan.kernel_name == "conv_tile_i8", plan.kernel_name


@pytest.mark.parametrize("name,variant", [
    ("resnet_3x3_int8", "general"), ("resnet_3x3_int8", "rf"), ("resnet_3x3_int8", "stream"),
    ("resnet_1x1_int8", "general"), ("resnet_1x1_int8", "rf"), ("resnet_1x1_int8", "tile"),
    ("resnet_3x3s2_int8", "general"), ("resnet_3x3s2_int8", "rf"), ("resnet_3x3s2_int8", "tile")])
def test_workload_forced_variant(name, variant, monkeypatch):
    """Every kernel family stays bit-exact on the layers another family is
    normally chosen for (FCONV_FORCE_VARIANT is read at plan creation; the
    tiled kernel needs channel rows of whole 128-byte stages)."""
    monkeypatch.setenv("FCONV_FORCE_VARIANT", variant)
    L = wl.LAYERS[name]
    inp, plan = _layer_case(L, N=4)
    assert plan.kernel_name.startswith("conv_" + variant), plan.kernel_name
    say("forced %s on %s" % (plan.kernel_name, name))
    y, guards = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, inp.side, L.conv_input_scale,
                        L.side_input_scale, guard=128)
    assert guards
    r = oracle_out(L.dtype, inp.x, inp.w, L.stride, L.padding, inp.bias, inp.side,
                   L.conv_input_scale, L.side_input_scale, L.relu)
    assert np.array_equal(y, r)


@pytest.mark.parametrize("name", ["resnet_3x3_int8", "resnet_1x1_int8", "resnet_3x3s2_int8"])
def test_graph_replay_matches_eager(name):
    """A captured HIP graph of prepacked runs, replayed several times with
    eager work and synchronisation in between, reproduces the eager output
    on every replay."""
    dev = device()
    L = wl.LAYERS[name]
    inp, plan = _layer_case(L, N=4)
    x, w = to_dev(inp.x, dev), to_dev(inp.w, dev)
    bias, side = to_dev(inp.bias, dev), to_dev(inp.side, dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    plan.pack_filter(w, ws)
    y_eager = torch.empty(plan.out_shape, dtype=torch.int8, device=dev)
    plan.run(x, w, y_eager, ws, bias=bias, side=side, conv_input_scale=L.conv_input_scale,
             side_input_scale=L.side_input_scale, prepacked=True)
    torch.cuda.synchronize()
    ref = y_eager.cpu()
    y = torch.zeros(plan.out_shape, dtype=torch.int8, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    args = plan.make_args(x, w, y, ws, bias=bias, side=side,
                          conv_input_scale=L.conv_input_scale,
                          side_input_scale=L.side_input_scale, prepacked=True)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(3):
                assert plan.run_args(args, s.cuda_stream) == 0
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), ref), "replay %d differs" % rep


@pytest.mark.parametrize("C,K,R", [(128, 64, 3), (64, 128, 7), (24, 40, 4), (256, 256, 1)])
@pytest.mark.parametrize("variant", [None, "general", "tile", "rf"])
@pytest.mark.parametrize("dtype", ["int8", "bf16", "fp32"])
def test_full_size_valid(C, K, R, variant, dtype, monkeypatch):
    """Filter as large as the image, VALID: every output is one dot product
    over the whole image, the second GEMM special case of the fused op
    (x viewed as [N, H*W*C] times w viewed as [R*S*C, K]).  Each kernel
    family where the shape allows it."""
    if variant is not None:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", variant)
    c = tile_case(C, K, R, R, R, 1, "VALID", dtype)
    name = check_case(c, dtype, fp32_tol=TOL["fp32"] if R * R * C > 4096 else 2e-6)
    if variant is None:  # whole 64-byte k-steps per image: the split GEMM
        esize = {"int8": 1, "bf16": 2, "fp32": 4}[dtype]
        assert name.startswith("conv_gemm_") == (R * R * C * esize % 64 == 0), name



@pytest.mark.parametrize("roles", ["1", "0"])
@pytest.mark.parametrize("bm", [64, 128, 256])
@pytest.mark.parametrize("K", [64, 256])
@pytest.mark.parametrize("dtype,C,R,stages", [
    ("int8", 128, 1, 1), ("int8", 256, 1, 2), ("fp32", 96, 1, 3), ("int8", 128, 2, 4),
    ("fp32", 160, 1, 5), ("bf16", 384, 1, 6), ("fp32", 224, 1, 7), ("bf16", 64, 3, 9),
    ("fp32", 384, 1, 12), ("bf16", 192, 1, 3), ("int8", 640, 1, 5), ("bf16", 448, 1, 7)])
def test_tile_stage_counts(dtype, C, R, stages, K, bm, roles, monkeypatch):
    """The tiled kernels' loop tails: every stage count from 1 to 9 and 12,
    modulo the 4-buffer ring of the 64- and 128-pixel tiles (one 128-channel
    tile, K = 64: two stages per barrier; two, K = 256: one per barrier; the
    int8 and bf16 kernel with copy waves, FCONV_TILE_ROLES=1, one per barrier)
    and modulo the 6-stage loop trip of the 256-pixel tile's 3-buffer ring."""
    esize = {"int8": 1, "bf16": 2, "fp32": 4}[dtype]
    assert R * R * C * esize // 128 == stages
    if dtype == "fp32" and roles == "0":
        pytest.skip("fp32 always runs the 8-wave tiled kernel")
    monkeypatch.setenv("FCONV_FORCE_VARIANT", "tile")
    monkeypatch.setenv("FCONV_TILE_BM", str(bm))
    monkeypatch.setenv("FCONV_TILE_ROLES", roles)
    name = check_case(tile_case(C, K, 7, 9, R, 1, "SAME", dtype), dtype)
    assert name.startswith("conv_tile_"), name


@pytest.mark.parametrize("name,bm", [("resnet_3x3_bf16_bn", None), ("cbna_5x5_bf16", None),
                                     ("cbna_7x7s2_bf16", None), ("resnet_3x3s2_int8", "128"),
                                     ("resnet_3x3s2_int8", "64")])
def test_tile_roles_bit_identical(name, bm, monkeypatch):
    """The tiled kernel with copy waves and the 8-wave one (FCONV_TILE_ROLES=0)
    add the same products in the same order: the same output bits on the full
    layers (the strided int8 layer with the tiled kernel pinned)."""
    L = wl.LAYERS[name]
    if bm:
        monkeypatch.setenv("FCONV_FORCE_VARIANT", "tile")
        monkeypatch.setenv("FCONV_TILE_BM", bm)
    outs = []
    for roles in ("1", "0"):
        monkeypatch.setenv("FCONV_TILE_ROLES", roles)
        inp, plan = _layer_case(L)
        assert plan.kernel_name.startswith("conv_tile_"), plan.kernel_name
        say("layer %s roles=%s kernel=%s" % (name, roles, plan.kernel_name))
        y, guards = run_gpu(plan, L.dtype, inp.x, inp.w, inp.bias, inp.side, L.conv_input_scale,
                            L.side_input_scale, inp.bn, guard=256)
        assert guards
        outs.append(y)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("C,K,H,W,R,stride,pad", [
    (128, 64, 9, 13, 3, 1, "SAME"), (128, 128, 11, 11, 3, 2, "SAME"),
    (256, 64, 7, 9, 1, 1, "VALID"), (256, 256, 5, 5, 3, 1, "SAME"), (128, 192, 8, 8, 8, 1, "VALID")])
@pytest.mark.parametrize("dtype", ["int8", "bf16", "fp32"])
@pytest.mark.parametrize("bm", [128, 256])
def test_tile_shapes_pinned_heights(C, K, H, W, R, stride, pad, dtype, bm, monkeypatch):
    """Ragged shapes with 128- and 256-pixel tiles pinned (small grids pick
    64-pixel tiles by themselves)."""
    monkeypatch.setenv("FCONV_FORCE_VARIANT", "tile")
    monkeypatch.setenv("FCONV_TILE_BM", str(bm))
    tol = TOL["fp32"] if R * R * C > 4096 else 2e-6
    name = check_case(tile_case(C, K, H, W, R, stride, pad, dtype), dtype, fp32_tol=tol)
    assert name.startswith("conv_tile_"), name


@pytest.mark.parametrize("dtype,roles,seed", [("int8", "1", 410), ("int8", "0", 411),
                                              ("bf16", "1", 420), ("bf16", "0", 421)])
def test_fuzz_tiled_kernels(dtype, roles, seed, monkeypatch):
    """Random layers on the tiled kernels (with copy waves, FCONV_TILE_ROLES=1,
    and the 8-wave one): channels filling whole 128-byte stages, K any
    multiple of 16, filters 1-5 in each direction, strides 1-3, SAME and
    VALID, 64- and 128-pixel tiles, ragged pixel and channel tails."""
    rng = np.random.default_rng(seed)
    monkeypatch.setenv("FCONV_FORCE_VARIANT", "tile")
    monkeypatch.setenv("FCONV_TILE_ROLES", roles)
    count = 48
    say("tiled fuzz %s roles=%s: %d cases" % (dtype, roles, count))
    for i in range(count):
        C = int(rng.choice([128, 256] if dtype == "int8" else [64, 128, 192]))
        K = int(16 * rng.integers(1, 17))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        st = int(rng.integers(1, 4))
        pad = "SAME" if rng.random() < 0.6 else "VALID"
        N = int(rng.integers(1, 4))
        H = int(rng.integers(max(R, 3), 15))
        W = int(rng.integers(max(S, 3), 15))
        bm = str(rng.choice([64, 128]))
        monkeypatch.setenv("FCONV_TILE_BM", bm)
        Ho, Wo = oracle.geometry(H, W, R, S, st, st, pad == "SAME")[:2]
        if dtype == "int8":
            x = wl.draw_int8(rng, (N, H, W, C), -128, 127)
            w = wl.draw_int8(rng, (R, S, C, K), -128, 127)
            use_side = bool(rng.random() < 0.5)
            relu = bool(rng.random() < 0.5)
            c = dict(shape=(N, H, W, C, K, R, S, st, pad), x=x, w=w,
                     bias=rng.normal(0, 30, K).astype(np.float32),
                     side=wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if use_side else None,
                     cis=np.float32(rng.choice([2.0 ** -10, 0.0123, 2.0 ** -13])),
                     sis=np.float32(0.5) if use_side else np.float32(0), relu=relu,
                     ops=[wl.OP_SCALE] + ([wl.OP_SIDE] if use_side else []) + [wl.OP_BIAS] +
                     ([wl.OP_RELU] if relu else []), bn=None, use_bias=True)
        else:
            x = wl.float_to_bf16_bits(rng.normal(0, 1, (N, H, W, C)).astype(np.float32))
            w = wl.float_to_bf16_bits(
                rng.normal(0, 1 / np.sqrt(R * S * C), (R, S, C, K)).astype(np.float32))
            use_bn = bool(rng.random() < 0.6)
            relu = bool(rng.random() < 0.5)
            bn = dict(mean=rng.normal(0, .1, K).astype(np.float32),
                      var=rng.uniform(.5, 1.5, K).astype(np.float32),
                      gamma=rng.uniform(.5, 1.5, K).astype(np.float32),
                      beta=rng.normal(0, .1, K).astype(np.float32), eps=1e-5) if use_bn else None
            c = dict(shape=(N, H, W, C, K, R, S, st, pad), x=x, w=w,
                     bias=rng.normal(0, .1, K).astype(np.float32), side=None, cis=1.0, sis=0.0,
                     relu=relu, ops=[wl.OP_BIAS] + ([wl.OP_BN] if use_bn else []) +
                     ([wl.OP_RELU] if relu else []), bn=bn, use_bias=True)
        y, r, guards, plan = _run_case(c, dtype)
        where = "case %d %s bm=%s %s" % (i, c["shape"], bm, plan.kernel_name)
        assert plan.kernel_name.startswith("conv_tile_"), where
        assert guards, where
        if dtype == "int8":
            assert np.array_equal(y, r), where + ": %d differ" % np.count_nonzero(y != r)
        else:
            assert float_error(y, r) <= TOL["bf16"], where


def test_fuzz_halo_s2():
    """Random layers on the stride-2 row kernel: 64 or 128 input channels, K a
    multiple of 128, Wo up to 31, SAME (either stride-2 padding) and VALID,
    images of one output row and up, ragged last workgroups, rows per
    workgroup from the device size or pinned (FCONV_HALO_ROWS), with and
    without the side input and ReLU; bit-exact against the oracle."""
    import os
    rng = np.random.default_rng(430)
    count = 20
    say("halo_s2 fuzz: %d cases" % count)
    for i in range(count):
        C = int(rng.choice([64, 128]))
        K = int(128 * rng.integers(1, 3))
        N = int(rng.integers(1, 4))
        pad = "SAME" if rng.random() < 0.7 else "VALID"
        H = int(rng.integers(3, 40))
        W = int(rng.integers(3, 62))
        Ho, Wo = oracle.geometry(H, W, 3, 3, 2, 2, pad == "SAME")[:2]
        rows = int(rng.choice([0, 1, 2, 3, 5, 9]))
        if rows:
            os.environ["FCONV_HALO_ROWS"] = str(rows)
        else:
            os.environ.pop("FCONV_HALO_ROWS", None)
        try:
            side = bool(rng.random() < 0.5)
            relu = bool(rng.random() < 0.5)
            x = wl.draw_int8(rng, (N, H, W, C), -128, 127)
            w = wl.draw_int8(rng, (3, 3, C, K), -128, 127)
            c = dict(shape=(N, H, W, C, K, 3, 3, 2, pad), x=x, w=w,
                     bias=rng.normal(0, 40, K).astype(np.float32),
                     side=wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if side else None,
                     cis=np.float32(rng.choice([2.0 ** -11, 2.0 ** -12, 0.0009])),
                     sis=np.float32(0.75 if side else 0.0), relu=relu,
                     ops=[wl.OP_SCALE] + ([wl.OP_SIDE] if side else []) + [wl.OP_BIAS] +
                     ([wl.OP_RELU] if relu else []), bn=None, use_bias=True)
            y, r, guards, plan = _run_case(c, "int8")
        finally:
            os.environ.pop("FCONV_HALO_ROWS", None)
        where = "case %d %s rows=%d %s" % (i, c["shape"], rows, plan.kernel_name)
        if Wo <= 31:
            assert plan.kernel_name == "conv_halo_s2_i8", where
        assert guards, where
        assert np.array_equal(y, r), where + ": %d differ" % np.count_nonzero(y != r)


@pytest.mark.parametrize("cudnn7", [False, True])
def test_fuzz_halo(cudnn7):
    """Random layers on the stride-1 row kernel (the benchmark layer's
    kernel): 3x3 over 64 channels, K any multiple of 16, padded rows of up to
    64 pixels, SAME and VALID, images of one row and up, workgroups spanning
    images, rows per workgroup from the device size or pinned
    (FCONV_HALO_ROWS), with and without the side input and ReLU, in both
    epilogue orders; bit-exact against the oracle."""
    import os
    rng = np.random.default_rng(450 + int(cudnn7))
    count = 24
    say("halo fuzz (cudnn7 order %s): %d cases" % (cudnn7, count))
    for i in range(count):
        K = int(16 * rng.integers(1, 9))
        N = int(rng.integers(1, 12))
        pad = "SAME" if rng.random() < 0.7 else "VALID"
        H = int(rng.integers(1 if pad == "SAME" else 3, 13))
        W = int(rng.integers(1 if pad == "SAME" else 3, 63))
        rows = int(rng.choice([0, 0, 1, 2, 4, 7, 11]))
        side = bool(rng.random() < 0.6)
        relu = bool(rng.random() < 0.5)
        Ho, Wo = oracle.geometry(H, W, 3, 3, 1, 1, pad == "SAME")[:2]
        x = wl.draw_int8(rng, (N, H, W, 64), -128, 127)
        w = wl.draw_int8(rng, (3, 3, 64, K), -128, 127)
        bias = rng.normal(0, 40, K).astype(np.float32)
        sd = wl.draw_int8(rng, (N, Ho, Wo, K), -128, 127) if side else None
        cis = np.float32(rng.choice([2.0 ** -11, 2.0 ** -9, 0.0007]))
        sis = np.float32(0.25 if side else 0.0)
        ops = [wl.OP_SCALE] + ([wl.OP_SIDE] if side else []) + [wl.OP_BIAS] + (
            [wl.OP_RELU] if relu else [])
        if rows:
            os.environ["FCONV_HALO_ROWS"] = str(rows)
        try:
            plan = make_plan(N, H, W, 64, K, 3, 3, 1, pad, "int8", ops, cudnn7_order=cudnn7)
        finally:
            os.environ.pop("FCONV_HALO_ROWS", None)
        where = "case %d %s rows=%d %s" % (i, (N, H, W, K, pad, side, relu), rows,
                                           plan.kernel_name)
        assert plan.kernel_name == "conv_halo_i8", where
        y, guards = run_gpu(plan, "int8", x, w, bias, sd, cis, sis, guard=64)
        r = oracle_out("int8", x, w, 1, pad, bias, sd, cis, sis, relu,
                       order=7 if cudnn7 else 8)
        assert guards, where
        assert np.array_equal(y, r), where + ": %d differ" % np.count_nonzero(y != r)
