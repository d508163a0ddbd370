"""GPU parity at the largest tensors a plan accepts: inputs just under 2^31
bytes (the limit of the kernels' 32-bit buffer offsets), one case per kernel
family (row-halo 3x3, streaming 1x1, the stride-2 row kernel, 128- and 256-pixel
tiled stride 2 int8,
tiled bf16, the full-size VALID GEMM, the resident-filter and general
kernels), and the weight gradient in bf16 and fp32.  The inputs are drawn
on the GPU from a
seeded generator; the oracle cannot run whole layers of this size, so it
computes sampled outputs one by one from their input windows (the first and
last output pixels, the image borders, and random pixels), element by
element against the GPU's.  Guard bytes after y must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import TOL, float_error, make_plan, say

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31 - 1  # bytes: the largest tensor a plan accepts

INT8_OPS = [wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS, wl.OP_RELU]
# (family, dtype, H, W, C, K, R, stride, padding, ops, environment pins)
CASES = [
    ("halo", "int8", 56, 56, 64, 64, 3, 1, "SAME", INT8_OPS, {}),
    ("stream", "int8", 56, 56, 256, 64, 1, 1, "VALID", [wl.OP_SCALE, wl.OP_BIAS], {}),
    ("halo_s2", "int8", 56, 56, 128, 128, 3, 2, "SAME", INT8_OPS, {}),
    ("tile", "int8", 56, 56, 128, 128, 3, 2, "SAME", INT8_OPS, {"FCONV_FORCE_VARIANT": "tile"}),
    ("tile", "int8", 56, 56, 128, 128, 3, 2, "SAME", INT8_OPS,
     {"FCONV_FORCE_VARIANT": "tile", "FCONV_TILE_BM": "256"}),
    ("tile", "bf16", 28, 28, 256, 256, 3, 1, "SAME", [wl.OP_BIAS, wl.OP_BN, wl.OP_RELU], {}),
    ("gemm", "int8", 7, 7, 512, 1024, 7, 1, "VALID", INT8_OPS, {}),
    ("rf", "int8", 56, 56, 64, 64, 3, 1, "SAME", INT8_OPS, {"FCONV_FORCE_VARIANT": "rf"}),
    # C = 8: the general kernel; here y (16 channels) is the tensor at the limit
    ("general", "int8", 56, 56, 8, 16, 3, 1, "SAME", INT8_OPS, {}),
]


def _window(x, n, ho, wo, R, stride, pt, pl):
    """Input window of output pixel (n, ho, wo) as an [R, R, C] host array,
    zeros outside the image."""
    _, H, W, C = x.shape
    h0, w0 = ho * stride - pt, wo * stride - pl
    hs, he = max(h0, 0), min(h0 + R, H)
    ws, we = max(w0, 0), min(w0 + R, W)
    out = torch.zeros((R, R, C), dtype=x.dtype)
    if hs < he and ws < we:
        out[hs - h0:he - h0, ws - w0:we - w0] = x[n, hs:he, ws:we].cpu()
    return out


@pytest.mark.parametrize("case", CASES, ids=["%s-%s%s" % (c[0], c[1], "".join(
    "-" + v for v in c[10].values())) for c in CASES])
def test_largest_accepted_tensors(case, monkeypatch):
    family, dtype, H, W, C, K, R, stride, padding, ops, pins = case
    for k, v in pins.items():
        monkeypatch.setenv(k, v)
    dev = torch.device("cuda:0")
    esize = 1 if dtype == "int8" else 2
    Ho0 = (H - 1) // stride + 1 if padding == "SAME" else (H - R) // stride + 1
    N = LIMIT // (max(H * W * C, Ho0 * Ho0 * K) * esize)
    plan = make_plan(N, H, W, C, K, R, R, stride, padding, dtype, ops)
    assert plan.kernel_name.startswith("conv_" + family), plan.kernel_name
    Ho, Wo = plan.Ho, plan.Wo
    pt, pl = plan.pads[0], plan.pads[2]
    say("max size %s %s: x %d bytes, N=%d, %s" % (family, dtype, N * H * W * C * esize, N,
                                                 plan.kernel_name))
    gen = torch.Generator(device=dev)
    gen.manual_seed(2026)
    rng = np.random.default_rng(31)
    n_out = N * Ho * Wo * K
    guard = 256
    raw = torch.full((n_out * esize + guard,), 0x5A, dtype=torch.uint8, device=dev)
    tdt = torch.int8 if dtype == "int8" else torch.bfloat16
    y = raw[:n_out * esize].view(tdt).view(N, Ho, Wo, K)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    if dtype == "int8":
        x = torch.randint(-128, 128, (N, H, W, C), dtype=torch.int8, device=dev, generator=gen)
        w = wl.draw_int8(rng, (R, R, C, K), -128, 127)
        bias = rng.normal(0, 16, K).astype(np.float32)
        use_side = wl.OP_SIDE in ops
        side = (torch.randint(-128, 128, (N, Ho, Wo, K), dtype=torch.int8, device=dev,
                              generator=gen) if use_side else None)
        cis, sis = np.float32(1.0 / (R * R * C * 64)), np.float32(0.5 if use_side else 0.0)
        relu = wl.OP_RELU in ops
        plan.run(x, torch.from_numpy(w).to(dev), y, ws, bias=torch.from_numpy(bias).to(dev),
                 side=side, conv_input_scale=float(cis), side_input_scale=float(sis))
    else:
        x = torch.randn((N, H, W, C), dtype=torch.bfloat16, device=dev, generator=gen)
        wf = rng.normal(0, 1.0 / np.sqrt(R * R * C), (R, R, C, K)).astype(np.float32)
        w = wl.float_to_bf16_bits(wf)
        bias = rng.normal(0, 0.1, K).astype(np.float32)
        bn = dict(mean=rng.normal(0, .1, K).astype(np.float32),
                  var=rng.uniform(.5, 1.5, K).astype(np.float32),
                  gamma=rng.uniform(.5, 1.5, K).astype(np.float32),
                  beta=rng.normal(0, .1, K).astype(np.float32), eps=1e-5)
        bnd = {k: torch.from_numpy(v).to(dev) for k, v in bn.items() if k != "eps"}
        bnd["eps"] = bn["eps"]
        wd = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16)
        plan.run(x, wd, y, ws, bias=torch.from_numpy(bias).to(dev), bn=bnd)
    torch.cuda.synchronize()
    assert bool((raw[n_out * esize:] == 0x5A).all()), "write past the end of y"

    # Sampled outputs: the first and last pixels, corners of the first and
    # last images, and random pixels.
    pix = [(0, 0, 0), (N - 1, Ho - 1, Wo - 1), (N - 1, 0, Wo - 1), (N - 1, Ho - 1, 0),
           (0, Ho - 1, Wo - 1), (N // 2, Ho // 2, 0)]
    pix += [(int(rng.integers(N)), int(rng.integers(Ho)), int(rng.integers(Wo)))
            for _ in range(90)]
    win = torch.stack([_window(x, n, ho, wo, R, stride, pt, pl) for n, ho, wo in pix])
    got = torch.stack([y[n, ho, wo].cpu() for n, ho, wo in pix])
    if dtype == "int8":
        sd = (np.stack([side[n, ho, wo].cpu().numpy() for n, ho, wo in pix])[:, None, None]
              if side is not None else None)
        ref = oracle.fused_conv_i8(win.numpy(), w, bias, cis, sd, sis, relu, 1, "VALID")
        g = got.numpy()[:, None, None]
        bad = np.count_nonzero(g != ref)
        assert bad == 0, "%d of %d sampled outputs differ" % (bad, ref.size)
    else:
        xw = win.float().numpy()
        ref = oracle.fused_conv_float(xw, wl.bf16_bits_to_float(w), bias, bn, True, 1, "VALID")
        e = float_error(got.float().numpy()[:, None, None], ref)
        assert e <= TOL["bf16"], e
    del x, y, raw, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_weight_gradient_largest_accepted_tensors(dtype):
    """The weight gradient with x and dy just under 2^31 bytes (the 3x3
    64-channel geometry): sampled dw elements against the oracle's weight
    gradient of the one input channel and one gradient channel they involve
    (every pixel of the batch)."""
    dev = torch.device("cuda:0")
    H, W, C, K, R = 56, 56, 64, 64, 3
    esize = 2 if dtype == "bf16" else 4
    N = LIMIT // (H * W * C * esize)
    plan = fc_wgrad_plan(N, H, W, C, K, R, dtype)
    say("max size wgrad %s: x %d bytes, N=%d, %s, %d B workspace" % (
        dtype, N * H * W * C * esize, N, plan.kernel_name, plan.workspace_bytes))
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.randn((N, H, W, C), dtype=tdt, device=dev, generator=gen)
    dy = torch.randn((N, H, W, K), dtype=tdt, device=dev, generator=gen)
    dw = torch.empty(plan.dw_shape, dtype=torch.float32, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    plan.run(x, dy, dw, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    taps = [(0, 0, 0, 0), (R - 1, R - 1, C - 1, K - 1), (1, 1, 0, K - 1)]
    taps += [tuple(int(v) for v in (rng.integers(R), rng.integers(R), rng.integers(C),
                                    rng.integers(K))) for _ in range(9)]
    got, ref = [], []
    for r, s, c, k in taps:
        xc = x[..., c:c + 1].float().cpu().numpy()  # bf16 widens exactly
        dk = dy[..., k:k + 1].float().cpu().numpy()
        ref.append(float(oracle.wgrad(xc, dk, R, R, 1, "SAME")[r, s, 0, 0]))
        got.append(float(dw[r, s, c, k]))
    got, ref = np.array(got), np.array(ref)
    e = float(np.max(np.abs(got - ref))) / float(np.max(np.abs(ref)))
    assert e <= 1e-4, (e, got, ref)
    del x, dy, dw, ws
    torch.cuda.empty_cache()


def fc_wgrad_plan(N, H, W, C, K, R, dtype):
    import convolution_implicit_gemm_nhwc_amd as fc
    return fc.WgradPlan(N, H, W, C, K, R, R, 1, "SAME", dtype, out_fp32=True)
