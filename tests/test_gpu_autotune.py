"""Autotuning (fconv_plan_autotune): the chosen configuration is one that can
run the shape, its result stays bit-exact (int8) or within tolerance (float)
against the oracle, and a later plan with the same descriptor starts from the
cached choice until the cache is cleared."""
import numpy as np
import pytest
import torch

import convolution_implicit_gemm_nhwc_amd as fc
import workloads as wl
from gpu_helpers import TOL, device, float_error, from_dev, make_plan, oracle_out, say, to_dev

pytestmark = pytest.mark.gpu

FAMILIES = ("conv_halo_", "conv_stream_", "conv_tile_", "conv_rf_", "conv_general_",
            "conv_halo_s2_")


@pytest.mark.parametrize("name", ["resnet_3x3_int8", "resnet_1x1_int8", "resnet_3x3s2_int8",
                                  "resnet_3x3_bf16_bn"])
def test_autotune_keeps_parity_and_caches(name):
    fc.autotune_cache_clear()
    dev = device()
    L = wl.LAYERS[name]
    inp = wl.make_inputs(L, N=4)
    n = inp.x.shape[0]
    plan = make_plan(n, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops)
    before = plan.kernel_name
    tdt = {"int8": torch.int8, "bf16": torch.bfloat16, "fp32": torch.float32}[L.dtype]
    y = torch.empty(plan.out_shape, dtype=tdt, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    bn = None
    if inp.bn is not None:
        bn = {k: to_dev(np.asarray(inp.bn[k], np.float32), dev) for k in
              ("gamma", "beta", "mean", "var")}
        bn["eps"] = float(inp.bn["eps"])
    us = plan.autotune(to_dev(inp.x, dev), to_dev(inp.w, dev), y, ws, repeats=5,
                       bias=to_dev(inp.bias, dev), side=to_dev(inp.side, dev),
                       conv_input_scale=L.conv_input_scale,
                       side_input_scale=L.side_input_scale, bn=bn)
    torch.cuda.synchronize()
    say("%s: heuristic %s, autotuned %s (%.2f us)" % (name, before, plan.kernel_name, us))
    assert us > 0 and plan.kernel_name.startswith(FAMILIES)
    out = from_dev(y, L.dtype)
    r = oracle_out(L.dtype, inp.x, inp.w, L.stride, L.padding, inp.bias, inp.side,
                   L.conv_input_scale, L.side_input_scale, L.relu, inp.bn,
                   use_bias=wl.OP_BIAS in L.ops)
    if L.dtype == "int8":
        assert np.array_equal(out, r)
    else:
        assert float_error(out, r) <= TOL[L.dtype]
    again = make_plan(n, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops)
    assert again.kernel_name == plan.kernel_name
    fc.autotune_cache_clear()
    fresh = make_plan(n, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype, L.ops)
    assert fresh.kernel_name == before
