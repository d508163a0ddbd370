"""fconv_plan_run_no_alloc (the entry point for callers that cannot
allocate) against fconv_plan_run through the C ABI: the same kernels, so
the outputs must be identical bit for bit.  Two calls in a row on one GPU,
the second with a smaller input, so the second reuses the scratch array the
first one filled; then a prepacked call that reuses the filter the previous
call left there; and a plan too large for the array is refused."""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_nhwc_amd as fc
from convolution_implicit_gemm_nhwc_amd import _abi
from gpu_helpers import device, make_plan, say, to_dev
import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(L, N):
    return wl.make_inputs(L, N=N)


def _bits_equal(a, b):
    """Bit-for-bit equality (bf16 / fp32 compared as integers)."""
    iv = {torch.int8: torch.int8, torch.bfloat16: torch.int16, torch.float32: torch.int32}
    return torch.equal(a.view(iv[a.dtype]), b.view(iv[b.dtype]))


def _both(L, N, dev):
    inp = _inputs(L, N)
    plan = make_plan(N, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops)
    tdt = {"int8": torch.int8, "bf16": torch.bfloat16, "fp32": torch.float32}[L.dtype]
    x, w = to_dev(inp.x, dev), to_dev(inp.w, dev)
    bias, side = to_dev(inp.bias, dev), to_dev(inp.side, dev)
    bn = None
    if inp.bn is not None:
        bn = {k: to_dev(np.asarray(inp.bn[k], np.float32), dev)
              for k in ("gamma", "beta", "mean", "var")}
        bn["eps"] = float(inp.bn["eps"])
    kw = dict(bias=bias, side=side, conv_input_scale=L.conv_input_scale,
              side_input_scale=L.side_input_scale, bn=bn)
    ref = torch.empty(plan.out_shape, dtype=tdt, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    plan.run(x, w, ref, ws, **kw)
    got = torch.full(plan.out_shape, 3, dtype=tdt, device=dev)
    plan.run_no_alloc(x, w, got, **kw)
    torch.cuda.synchronize()
    return plan, ref, got, (x, w, kw)


@pytest.mark.parametrize("first,second", [
    (("resnet_3x3_int8", 8), ("resnet_3x3_int8", 3)),
    (("resnet_3x3_bf16_bn", 4), ("resnet_3x3s2_int8", 2)),
    (("resnet_3x3_fp32_bn", 2), ("resnet_1x1_int8", 1)),
])
def test_no_alloc_matches_run_twice(first, second):
    dev = device()
    for name, N in (first, second):
        L = wl.LAYERS[name]
        plan, ref, got, _ = _both(L, N, dev)
        say("no-alloc %s N=%d kernel=%s workspace=%d" % (name, N, plan.kernel_name,
                                                         plan.workspace_bytes))
        assert _bits_equal(got, ref), name


def test_no_alloc_prepacked_reuses_the_last_filter():
    dev = device()
    L = wl.LAYERS["resnet_3x3s2_int8"]
    plan, ref, got, (x, w, kw) = _both(L, 2, dev)
    assert _bits_equal(got, ref)
    again = torch.zeros_like(ref)
    args = plan.make_args(x, None, again, None, workspace_bytes=0, prepacked=True, **kw)
    assert plan.run_no_alloc_args(args) == _abi.FCONV_OK
    torch.cuda.synchronize()
    assert _bits_equal(again, ref)


def test_no_alloc_refuses_a_plan_beyond_the_array():
    # fp32 filter of 3x3x512 -> 512 channels: ~9.4 MB packed, above 4 MiB.
    plan = fc.Plan(1, 4, 4, 512, 512, 3, 3, 1, "SAME", "fp32", ops=("bias",))
    assert plan.workspace_bytes > _abi.FCONV_NO_ALLOC_SCRATCH_BYTES
    dev = device()
    x = torch.zeros((1, 4, 4, 512), dtype=torch.float32, device=dev)
    w = torch.zeros((3, 3, 512, 512), dtype=torch.float32, device=dev)
    y = torch.zeros((1, 4, 4, 512), dtype=torch.float32, device=dev)
    b = torch.zeros(512, dtype=torch.float32, device=dev)
    args = plan.make_args(x, w, y, None, workspace_bytes=0, bias=b)
    assert plan.run_no_alloc_args(args) == _abi.FCONV_ERR_WORKSPACE
