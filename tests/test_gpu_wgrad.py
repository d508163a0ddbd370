"""Weight-gradient parity: the HIP path (fconv_wgrad_plan_run through the C
ABI) against the float64 oracle (oracle.wgrad), element by element.

Tolerances on e = max|dw - r| / max|r| (normwise):
  - fp32 dw (fp32 plans, bf16 plans with out_fp32): 1e-4.  Products of the
    inputs are exact in fp32 for bf16 and rounded once for fp32; the sums are
    fp32 over up to 10^5 terms, whose rounding error grows like
    2^-24 * sqrt(terms) (about 2e-5 at 10^5) for these zero-mean inputs.
  - bf16 dw: 4e-3, the bf16 rounding of the result (at most 2^-9 of each
    element, so at most 2^-9 of max|r|) plus the fp32 part.
"""
import zlib

import numpy as np
import pytest
import torch

import convolution_implicit_gemm_nhwc_amd as fc
import oracle
import workloads as wl
from gpu_helpers import device, float_error, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 4e-3}


def draw(rng, shape, dtype):
    a = rng.normal(0.0, 1.0, size=shape).astype(np.float32)
    return wl.float_to_bf16_bits(a) if dtype == "bf16" else a


def run_wgrad(plan, x, dy, dev, fill=None):
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[plan.out_dtype]
    dw = torch.empty(plan.dw_shape, dtype=tdt, device=dev)
    if fill is not None:
        dw.fill_(fill)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    plan.run(to_dev(x, dev), to_dev(dy, dev), dw, ws)
    torch.cuda.synchronize()
    return from_dev(dw, plan.out_dtype)


# (N, H, W, C, K, R, S, stride, padding): several tiles of both kinds, ragged
# tails in k, (r, s, c) and pixels, the element-wise gather (C or K off the
# 16-byte chunk), strides 1-3, SAME and VALID, images smaller than the filter.
CASES = [
    (2, 13, 11, 40, 72, 3, 3, 1, "SAME"),
    (3, 10, 10, 24, 136, 3, 3, 2, "SAME"),
    (2, 9, 9, 16, 64, 1, 1, 1, "VALID"),
    (1, 17, 15, 32, 48, 5, 5, 3, "VALID"),
    (2, 7, 6, 3, 5, 3, 3, 1, "SAME"),
    (2, 8, 9, 6, 10, 2, 3, 2, "SAME"),
    (1, 2, 3, 8, 16, 5, 5, 1, "SAME"),
    (4, 20, 20, 64, 64, 3, 3, 1, "SAME"),
    (1, 1, 1, 8, 8, 1, 1, 1, "VALID"),
    (2, 12, 12, 128, 256, 3, 3, 2, "SAME"),
    # bf16 3x3 stride 1 shapes of the row-halo kernel: one-row steps with two
    # 32-pixel blocks (Wo > 32, the widest 62), two-row steps (Wo <= 32),
    # VALID, three input slices and output blocks, and images of 1 and 3
    # output rows (every step or every other one crosses an image).
    (3, 9, 40, 32, 64, 3, 3, 1, "SAME"),
    (2, 5, 62, 32, 64, 3, 3, 1, "SAME"),
    (5, 7, 30, 64, 128, 3, 3, 1, "SAME"),
    (3, 12, 20, 96, 192, 3, 3, 1, "VALID"),
    (7, 3, 10, 32, 64, 3, 3, 1, "SAME"),
    (9, 1, 40, 32, 64, 3, 3, 1, "SAME"),
]


def _pin(kernel, monkeypatch):
    """'default': the plan's own choice (the row-halo kernel where it applies);
    'halo' pins the row-halo kernel also on rows of at most 32 pixels; the
    others pin the direct-to-LDS kernel's variants or the staged one."""
    if kernel in ("staged", "halo"):
        monkeypatch.setenv("FCONV_WGRAD_KERNEL", kernel)
        return
    if kernel == "default":
        return
    monkeypatch.setenv("FCONV_WGRAD_KERNEL", "dma")
    if kernel in ("ring4", "ring8"):
        monkeypatch.setenv("FCONV_WGRAD_RING", kernel[-1])
    elif kernel == "tk256":
        monkeypatch.setenv("FCONV_WGRAD_TK", "256")
    elif kernel == "groups1":
        monkeypatch.setenv("FCONV_WGRAD_GROUPS", "1")


@pytest.mark.parametrize("kernel", ["default", "halo", "ring4", "ring8", "tk256", "groups1",
                                    "staged"])
@pytest.mark.parametrize("out_fp32", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES)
def test_wgrad_small_shapes(case, dtype, out_fp32, kernel, monkeypatch):
    """Every kernel: the plan's own choice (bf16 3x3 stride 1 with 32-channel
    input slices, 64-channel output blocks and rows of 33-64 pixels: the
    row-halo kernel), the row-halo kernel pinned (two-row steps on narrower
    rows), the
    direct-to-LDS one (where C and K fill 16-byte chunks)
    with its 4- and 8-stage rings (FCONV_WGRAD_RING; the default is 4 for
    bf16, 8 for fp32), bf16 with K > 128 on 256- instead of 128-channel tiles
    (FCONV_WGRAD_TK=256), bf16 64/128-channel tiles with one wave group
    instead of two (FCONV_WGRAD_GROUPS=1), and the register-staged one
    (FCONV_WGRAD_KERNEL=staged)."""
    if dtype == "fp32" and out_fp32:
        pytest.skip("fp32 plans always write fp32")
    _pin(kernel, monkeypatch)
    N, H, W, C, K, R, S, stride, padding = case
    dev = device()
    plan = fc.WgradPlan(N, H, W, C, K, R, S, stride, padding, dtype, out_fp32=out_fp32)
    say("wgrad", case, dtype, "out_fp32" if out_fp32 else "", plan.kernel_name,
        "ws", plan.workspace_bytes)
    # A seed that is the same in every process (str hashes are randomised).
    rng = np.random.default_rng(zlib.crc32(repr((case, dtype)).encode()))
    x = draw(rng, (N, H, W, C), dtype)
    dy = draw(rng, plan.dy_shape, dtype)
    got = run_wgrad(plan, x, dy, dev, fill=7.0)
    ref = oracle.wgrad(x, dy, R, S, stride, padding)
    assert got.shape == ref.shape
    e = float_error(got, ref)
    assert e <= TOL[plan.out_dtype], (case, dtype, e)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_wgrad_empty_batch_gives_zeros(dtype):
    dev = device()
    plan = fc.WgradPlan(0, 8, 8, 16, 32, 3, 3, 1, "SAME", dtype)
    say("wgrad N=0", dtype)
    x = torch.empty((0, 8, 8, 16), dtype=torch.float32, device=dev)
    dy = torch.empty((0, 8, 8, 32), dtype=torch.float32, device=dev)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[plan.out_dtype]
    dw = torch.full(plan.dw_shape, 3.0, dtype=tdt, device=dev)
    # Zero-size tensors have no storage: pass any aligned device address.
    base = torch.empty(16, dtype=torch.uint8, device=dev)
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    st = plan.run_raw(base.data_ptr(), base.data_ptr(), dw, ws)
    assert st == 0
    torch.cuda.synchronize()
    assert bool((dw == 0).all())


def test_wgrad_is_deterministic():
    dev = device()
    L = wl.WGRAD_LAYERS["wgrad_3x3_bf16"]
    inp = wl.make_wgrad_inputs(L, N=4)
    plan = fc.WgradPlan(4, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, "bf16",
                        out_fp32=True)
    say("wgrad determinism", plan.kernel_name, "ws", plan.workspace_bytes)
    a = run_wgrad(plan, inp.x, inp.dy, dev)
    b = run_wgrad(plan, inp.x, inp.dy, dev, fill=1.0)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kernel", ["default", "halo", "ring4", "ring8", "tk256", "groups1",
                                    "staged"])
@pytest.mark.parametrize("name", list(wl.WGRAD_LAYERS))
def test_wgrad_full_workload(name, kernel, monkeypatch):
    """The full benchmark workloads, every element against the oracle."""
    _pin(kernel, monkeypatch)
    dev = device()
    L = wl.WGRAD_LAYERS[name]
    inp = wl.make_wgrad_inputs(L)
    plan = fc.WgradPlan(L.N, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                        out_fp32=True)
    assert plan.dy_shape == (L.N, L.Ho, L.Wo, L.K)
    say("wgrad full", name, plan.kernel_name, "ws", plan.workspace_bytes)
    got = run_wgrad(plan, inp.x, inp.dy, dev)
    ref = oracle.wgrad(inp.x, inp.dy, L.R, L.S, L.stride, L.padding)
    e = float_error(got, ref)
    say("  normwise error", e)
    assert e <= TOL["fp32"], (name, e)


@pytest.mark.parametrize("name", ["wgrad_3x3_bf16", "wgrad_3x3_64_bf16"])
def test_wgrad_graph_replay_matches_eager(name):
    """A captured HIP graph of gradient runs (main kernel and the sum of the
    pixel ranges), replayed several times with eager work and
    synchronisation in between, reproduces the eager dw bit for bit."""
    dev = device()
    L = wl.WGRAD_LAYERS[name]
    inp = wl.make_wgrad_inputs(L, N=4)
    plan = fc.WgradPlan(4, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                        out_fp32=True)
    say("wgrad graph replay", name, plan.kernel_name, "ws", plan.workspace_bytes)
    x, dy = to_dev(inp.x, dev), to_dev(inp.dy, dev)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    dw_eager = torch.empty(plan.dw_shape, dtype=torch.float32, device=dev)
    plan.run(x, dy, dw_eager, ws)
    torch.cuda.synchronize()
    ref = dw_eager.cpu()
    dw = torch.zeros(plan.dw_shape, dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(3):
                assert plan.run_raw(x, dy, dw, ws, stream=s) == 0
    torch.cuda.synchronize()
    for rep in range(4):
        dw.fill_(float(rep + 1))  # eager work between replays
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.cpu(), ref), "replay %d differs" % rep


@pytest.mark.parametrize("shape", [
    (8, 56, 56, 128, 128, 3, 3, 2, "SAME"),   # the strided layer's geometry (pads 0/1)
    (4, 28, 28, 256, 64, 1, 1, 1, "VALID"),   # 1x1: a plain GEMM over the pixels
    (2, 30, 30, 64, 96, 5, 5, 1, "SAME"),     # 5x5, K neither 64 nor a multiple of 128
])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_wgrad_layer_shapes(shape, dtype):
    """Larger layers of other geometries, every element against the oracle."""
    N, H, W, C, K, R, S, stride, padding = shape
    dev = device()
    plan = fc.WgradPlan(N, H, W, C, K, R, S, stride, padding, dtype, out_fp32=True)
    say("wgrad layer", shape, dtype, plan.kernel_name, "ws", plan.workspace_bytes)
    rng = np.random.default_rng(sum(shape[:7]) * 7 + (dtype == "bf16"))
    x = draw(rng, (N, H, W, C), dtype)
    dy = draw(rng, plan.dy_shape, dtype)
    got = run_wgrad(plan, x, dy, dev)
    ref = oracle.wgrad(x, dy, R, S, stride, padding)
    e = float_error(got, ref)
    say("  normwise error", e)
    assert e <= TOL["fp32"], (shape, dtype, e)


@pytest.mark.parametrize("pin", ["default", "halo"])
def test_wgrad_fuzz_row_halo(pin, monkeypatch):
    """Random bf16 3x3 stride-1 layers on the row-halo weight-gradient kernel:
    32-channel input slices (C = 32, 64, 96), 64-channel output blocks,
    padded rows of up to 64 pixels (one-row steps past 32 output columns;
    pinned, FCONV_WGRAD_KERNEL=halo, two-row steps on narrower rows), SAME
    and VALID, images of one output row and up, ranges that cross images."""
    _pin(pin, monkeypatch)
    rng = np.random.default_rng(440 if pin == "default" else 441)
    dev = device()
    count = 16
    say("row-halo wgrad fuzz (%s): %d cases" % (pin, count))
    for i in range(count):
        C = int(rng.choice([32, 64, 96]))
        K = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 4))
        pad = "SAME" if rng.random() < 0.7 else "VALID"
        H = int(rng.integers(3, 12))
        W = int(rng.integers(35, 63)) if pin == "default" else int(rng.integers(3, 63))
        plan = fc.WgradPlan(N, H, W, C, K, 3, 3, 1, pad, "bf16", out_fp32=True)
        where = (i, (N, H, W, C, K, pad), plan.kernel_name)
        if pin == "default":
            assert plan.kernel_name == "wgrad_halo_bf16", where
        x = draw(rng, (N, H, W, C), "bf16")
        dy = draw(rng, plan.dy_shape, "bf16")
        got = run_wgrad(plan, x, dy, dev, fill=7.0)
        ref = oracle.wgrad(x, dy, 3, 3, 1, pad)
        e = float_error(got, ref)
        assert e <= TOL[plan.out_dtype], (where, e)
