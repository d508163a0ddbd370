"""Weight-gradient plan: host-side checks of the C ABI (no GPU needed; the
failing runs return before anything is enqueued, so the fake device
addresses are never dereferenced)."""
import ctypes

import pytest

import convolution_implicit_gemm_nhwc_amd as fc
import oracle
import workloads as wl
from convolution_implicit_gemm_nhwc_amd import _abi


def _desc(**kw):
    d = _abi.FconvDesc()
    base = dict(N=2, H=8, W=8, C=16, K=32, R=3, S=3, stride_h=1, stride_w=1, padding=0,
                dtype=_abi.FCONV_BF16, n_ops=0, flags=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def _create(d):
    h = ctypes.c_void_p()
    st = _abi.lib().fconv_wgrad_plan_create(ctypes.byref(d), ctypes.byref(h))
    if st == 0:
        _abi.lib().fconv_wgrad_plan_destroy(h)
    return st


def test_create_accepts_float_dtypes_only():
    assert _create(_desc(dtype=_abi.FCONV_BF16)) == _abi.FCONV_OK
    assert _create(_desc(dtype=_abi.FCONV_FP32)) == _abi.FCONV_OK
    assert _create(_desc(dtype=_abi.FCONV_INT8)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(dtype=7)) == _abi.FCONV_ERR_UNSUPPORTED


@pytest.mark.parametrize("field,value", [("H", 0), ("W", -1), ("C", 0), ("K", 0), ("R", 0),
                                         ("S", 0), ("stride_h", 0), ("stride_w", -2),
                                         ("N", -1)])
def test_create_rejects_bad_sizes(field, value):
    assert _create(_desc(**{field: value})) == _abi.FCONV_ERR_INVALID_ARG


def test_create_rejects_ops_flags_and_bad_valid():
    assert _create(_desc(n_ops=1)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(flags=2)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(flags=_abi.FCONV_WGRAD_OUT_FP32)) == _abi.FCONV_OK
    assert _create(_desc(padding=1, H=2)) == _abi.FCONV_ERR_INVALID_ARG
    assert _create(_desc(padding=3)) == _abi.FCONV_ERR_UNSUPPORTED
    h = ctypes.c_void_p()
    assert _abi.lib().fconv_wgrad_plan_create(None, ctypes.byref(h)) == _abi.FCONV_ERR_INVALID_ARG
    assert _abi.lib().fconv_wgrad_plan_create(ctypes.byref(_desc()), None) == \
        _abi.FCONV_ERR_INVALID_ARG
    assert _abi.lib().fconv_wgrad_plan_destroy(None) == _abi.FCONV_OK
    assert _abi.lib().fconv_wgrad_plan_kernel_name(None) is None


@pytest.mark.parametrize("shape", [(2, 13, 11, 40, 72, 3, 3, 1, "SAME"),
                                   (3, 10, 10, 24, 136, 3, 3, 2, "SAME"),
                                   (1, 17, 15, 32, 48, 5, 5, 3, "VALID"),
                                   (64, 56, 56, 128, 128, 3, 3, 2, "SAME")])
def test_dims_match_oracle_geometry(shape):
    N, H, W, C, K, R, S, stride, padding = shape
    g = fc.WgradPlan(N, H, W, C, K, R, S, stride, padding, "fp32")
    (sh, sw), (pt, pb, pl, pr) = oracle.resolve((N, H, W, C), (R, S, C, K), stride, padding)
    Ho = (H + pt + pb - R) // sh + 1
    Wo = (W + pl + pr - S) // sw + 1
    assert g.dy_shape == (N, Ho, Wo, K)
    assert g.pads == (pt, pb, pl, pr)
    assert g.dw_shape == (R, S, C, K)


def test_workloads_and_workspace():
    for L in wl.WGRAD_LAYERS.values():
        g = fc.WgradPlan(L.N, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                         out_fp32=True)
        assert g.dy_shape == (L.N, L.Ho, L.Wo, L.K)
        kg_k = L.R * L.S * L.C * L.K
        # partial sums: a whole number of fp32 dW copies (or none)
        assert g.workspace_bytes % (4 * ((kg_k + 3) // 4)) == 0
        want = {"wgrad_3x3_64_bf16": "wgrad_halo_bf16", "wgrad_3x3_bf16": "wgrad_dma2_bf16_128",
                "wgrad_3x3_fp32": "wgrad_dma8_f32_128"}
        assert g.kernel_name == want[L.name], (L.name, g.kernel_name)


def test_run_checks_arguments():
    g = fc.WgradPlan(8, 28, 28, 64, 64, 3, 3, 1, "SAME", "bf16")
    assert g.workspace_bytes > 0
    lib = _abi.lib()
    A = 1 << 40  # fake, 16-byte aligned device addresses, far apart
    x, dy, dw, ws = A, 2 * A, 3 * A, 4 * A
    ok = dict(x=x, dy=dy, dw=dw, ws=ws, n=g.workspace_bytes)

    def run(**kw):
        a = dict(ok, **kw)
        return lib.fconv_wgrad_plan_run(g._h, None, a["x"], a["dy"], a["dw"], a["ws"], a["n"])

    assert lib.fconv_wgrad_plan_run(None, None, x, dy, dw, ws, ok["n"]) == \
        _abi.FCONV_ERR_INVALID_ARG
    assert run(x=None) == _abi.FCONV_ERR_INVALID_ARG
    assert run(dy=None) == _abi.FCONV_ERR_INVALID_ARG
    assert run(dw=None) == _abi.FCONV_ERR_INVALID_ARG
    assert run(ws=None) == _abi.FCONV_ERR_WORKSPACE
    assert run(n=ok["n"] - 1) == _abi.FCONV_ERR_WORKSPACE
    assert run(x=x + 8) == _abi.FCONV_ERR_MISALIGNED
    assert run(dw=dw + 2) == _abi.FCONV_ERR_MISALIGNED
    assert run(ws=ws + 4) == _abi.FCONV_ERR_MISALIGNED
    assert run(dw=x + 64) == _abi.FCONV_ERR_INVALID_ARG   # dw overlaps x
    assert run(ws=dy + 16) == _abi.FCONV_ERR_INVALID_ARG  # workspace overlaps dy


def test_binding_refuses_host_tensors():
    import torch
    g = fc.WgradPlan(1, 4, 4, 8, 8, 3, 3, 1, "SAME", "fp32")
    with pytest.raises(ValueError):
        g(torch.zeros(1, 4, 4, 8), torch.zeros(1, 4, 4, 8))


def test_create_rejects_tensors_of_2gib_or_more():
    # x of 2^31 bytes or more (bf16): buffer offsets are 32-bit.
    assert _create(_desc(N=1024, H=256, W=256, C=32)) == _abi.FCONV_ERR_UNSUPPORTED
    # dy likewise, through K.
    assert _create(_desc(N=1024, H=64, W=64, C=16, K=256)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(N=64, H=64, W=64, C=16, K=256)) == _abi.FCONV_OK


def test_staged_kernel_can_be_pinned(monkeypatch):
    monkeypatch.setenv("FCONV_WGRAD_KERNEL", "staged")
    g = fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "bf16")
    assert g.kernel_name == "wgrad_bf16_128"
    monkeypatch.delenv("FCONV_WGRAD_KERNEL")
    gh = fc.WgradPlan(32, 56, 56, 64, 64, 3, 3, 1, "SAME", "bf16")
    assert gh.kernel_name == "wgrad_halo_bf16"
    # 2 input slices x 1 output block, 128 ranges of 14 output rows: one
    # workgroup per CU, 128 fp32 dW copies in the workspace
    assert gh.workspace_bytes == 128 * 9 * 64 * 64 * 4
    assert fc.WgradPlan(32, 56, 56, 64, 64, 3, 3, 2, "SAME", "bf16").kernel_name != \
        "wgrad_halo_bf16"  # stride 2
    assert fc.WgradPlan(32, 56, 56, 48, 64, 3, 3, 1, "SAME", "bf16").kernel_name != \
        "wgrad_halo_bf16"  # C not a multiple of 32
    assert fc.WgradPlan(4, 8, 70, 32, 64, 3, 3, 1, "SAME", "bf16").kernel_name != \
        "wgrad_halo_bf16"  # padded rows wider than 64 pixels
    g2 = fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "bf16")
    assert g2.kernel_name == "wgrad_dma2_bf16_128"  # rows of 28 pixels
    monkeypatch.setenv("FCONV_WGRAD_KERNEL", "halo")
    assert fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "bf16").kernel_name == \
        "wgrad_halo_bf16"
    monkeypatch.setenv("FCONV_WGRAD_KERNEL", "dma")
    assert fc.WgradPlan(32, 56, 56, 64, 64, 3, 3, 1, "SAME", "bf16").kernel_name == \
        "wgrad_dma2_bf16_64"
    monkeypatch.setenv("FCONV_WGRAD_TK", "256")
    g256 = fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "bf16")
    assert g256.kernel_name == "wgrad_dma_bf16_256"
    # two wave groups on 128-channel tiles: half the ranges of 256-channel tiles
    assert g256.workspace_bytes == 2 * g2.workspace_bytes
    monkeypatch.delenv("FCONV_WGRAD_TK")
    monkeypatch.setenv("FCONV_WGRAD_GROUPS", "1")
    g4 = fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "bf16")
    assert g4.kernel_name == "wgrad_dma_bf16_128"
    # two wave groups per workgroup: half the pixel ranges of one group
    assert g4.workspace_bytes == 2 * g2.workspace_bytes
    monkeypatch.delenv("FCONV_WGRAD_GROUPS")
    assert fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "fp32").kernel_name == \
        "wgrad_dma8_f32_128"
    monkeypatch.setenv("FCONV_WGRAD_RING", "8")
    g = fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "bf16")
    assert g.kernel_name == "wgrad_dma8_bf16_128"
    # the 8-stage ring runs one workgroup per CU: half the pixel ranges
    assert g4.workspace_bytes > g.workspace_bytes
    monkeypatch.setenv("FCONV_WGRAD_RING", "4")
    assert fc.WgradPlan(16, 28, 28, 256, 256, 3, 3, 1, "SAME", "fp32").kernel_name == \
        "wgrad_dma_f32_128"
    monkeypatch.delenv("FCONV_WGRAD_RING")
    g = fc.WgradPlan(2, 7, 6, 3, 5, 3, 3, 1, "SAME", "bf16")
    assert g.kernel_name == "wgrad_bf16_64_elem"
