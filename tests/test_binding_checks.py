"""The Python binding rejects tensors that do not match the plan before it
calls the C ABI (CPU only: plans are host objects, and the checks run before
any device address is taken).  The kernels size every access from the plan,
so a short or mistyped tensor would otherwise be read or written past its
end."""
import pytest
import torch

import convolution_implicit_gemm_nhwc_amd as fc


def _plan(dtype="int8"):
    ops = ("scale", "side", "bias", "relu") if dtype == "int8" else ("bias", "bn", "relu")
    return fc.Plan(2, 6, 5, 16, 24, 3, 3, 1, "SAME", dtype, ops=ops)


def _args(p, **over):
    tdt = {"int8": torch.int8, "bf16": torch.bfloat16, "fp32": torch.float32}[p.dtype]
    d = p.desc
    a = dict(x=torch.zeros(d.N * d.H * d.W * d.C, dtype=tdt),
             w=torch.zeros(d.R * d.S * d.C * d.K, dtype=tdt),
             y=torch.zeros(p.out_shape, dtype=tdt),
             workspace=torch.zeros(p.workspace_bytes, dtype=torch.uint8),
             bias=torch.zeros(d.K, dtype=torch.float32))
    if p.dtype == "int8":
        a["side"] = torch.zeros(p.out_shape, dtype=torch.int8)
    else:
        a["bn"] = {k: torch.zeros(d.K, dtype=torch.float32)
                   for k in ("gamma", "beta", "mean", "var")}
        a["bn"]["eps"] = 1e-5
    a.update(over)
    return a


def test_matching_cpu_tensors_fail_only_on_the_device_check():
    for dtype in ("int8", "bf16", "fp32"):
        p = _plan(dtype)
        with pytest.raises(ValueError, match="GPU"):
            p.make_args(**_args(p))


@pytest.mark.parametrize("name,bad", [
    ("x", torch.zeros(2 * 6 * 5 * 16 - 1, dtype=torch.int8)),
    ("x", torch.zeros(2 * 6 * 5 * 16, dtype=torch.uint8)),
    ("w", torch.zeros(3 * 3 * 16 * 24 - 16, dtype=torch.int8)),
    ("y", torch.zeros(2 * 6 * 5 * 24 - 1, dtype=torch.int8)),
    ("y", torch.zeros(2 * 6 * 5 * 24, dtype=torch.float32)),
    ("bias", torch.zeros(23, dtype=torch.float32)),
    ("bias", torch.zeros(24, dtype=torch.float64)),
    ("side", torch.zeros(2 * 6 * 5 * 23, dtype=torch.int8)),
    ("conv_input_scale", torch.zeros(12, dtype=torch.float32)),
])
def test_short_or_mistyped_int8_tensors_are_rejected(name, bad):
    p = _plan("int8")
    with pytest.raises(ValueError, match=name.split("_")[0]):
        p.make_args(**_args(p, **{name: bad}))


def test_short_batch_norm_vector_is_rejected():
    p = _plan("bf16")
    a = _args(p)
    a["bn"]["var"] = torch.zeros(3, dtype=torch.float32)
    with pytest.raises(ValueError, match="bn var"):
        p.make_args(**a)


def test_bf16_plan_rejects_fp32_input():
    p = _plan("bf16")
    with pytest.raises(ValueError, match="dtype"):
        p.make_args(**_args(p, x=torch.zeros(2 * 6 * 5 * 16, dtype=torch.float32)))


def test_pack_filter_rejects_a_short_filter():
    p = _plan("int8")
    with pytest.raises(ValueError, match="w"):
        p.pack_filter(torch.zeros(10, dtype=torch.int8),
                      torch.zeros(p.workspace_bytes, dtype=torch.uint8))


def test_wgrad_rejects_mismatched_tensors():
    g = fc.WgradPlan(2, 6, 5, 16, 24, 3, 3, 1, "SAME", "bf16", out_fp32=True)
    x = torch.zeros(2 * 6 * 5 * 16, dtype=torch.bfloat16)
    dy = torch.zeros(g.dy_shape, dtype=torch.bfloat16)
    dw = torch.zeros(g.dw_shape, dtype=torch.float32)
    ws = torch.zeros(max(g.workspace_bytes, 16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        g.run_raw(x, dy, dw, ws)
    with pytest.raises(ValueError, match="dw"):
        g.run_raw(x, dy, dw.to(torch.bfloat16), ws)  # out_fp32 plan writes fp32
    with pytest.raises(ValueError, match="dy"):
        g.run_raw(x, dy[:1], dw, ws)
    with pytest.raises(ValueError, match="x"):
        g.run_raw(x.to(torch.float32), dy, dw, ws)
