"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, and every host-side check returns its status without touching a
device (the failing runs below return before anything is enqueued, so the
fake device addresses are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import convolution_implicit_gemm_nhwc_amd as fc
import oracle
import workloads as wl
from convolution_implicit_gemm_nhwc_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fconv.h")

INT8_OPS = ("scale", "side", "bias", "relu")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"FCONV_API\s+[\w\s\*]+?\b(fconv_\w+)\s*\(", text))
    assert declared == set(_abi.EXPORTS)
    lib = ctypes.CDLL(_abi.lib_path())
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    L = _abi.lib()
    for s in range(6):
        assert L.fconv_status_string(s)
    assert L.fconv_status_string(99) == b"unknown status"


def _desc(**kw):
    d = _abi.FconvDesc()
    base = dict(N=1, H=8, W=8, C=8, K=8, R=3, S=3, stride_h=1, stride_w=1, padding=0,
                dtype=0)
    base.update({k: v for k, v in kw.items() if k not in ("ops", "flags")})
    for k, v in base.items():
        setattr(d, k, v)
    ops = kw.get("ops", [1, 2, 3, 5])
    d.n_ops = len(ops)
    for i, o in enumerate(ops[:_abi.FCONV_MAX_OPS]):
        d.ops[i] = o
    d.flags = kw.get("flags", 0)
    return d


def _create(d):
    h = ctypes.c_void_p()
    st = _abi.lib().fconv_plan_create(ctypes.byref(d), ctypes.byref(h))
    if st == 0:
        _abi.lib().fconv_plan_destroy(h)
    return st


@pytest.mark.parametrize("field,value", [("H", 0), ("W", -1), ("C", 0), ("K", 0), ("R", 0),
                                         ("S", 0), ("stride_h", 0), ("stride_w", -2),
                                         ("N", -1)])
def test_create_rejects_bad_sizes(field, value):
    assert _create(_desc(**{field: value})) == _abi.FCONV_ERR_INVALID_ARG


def test_create_valid_filter_larger_than_image():
    assert _create(_desc(H=2, padding=1)) == _abi.FCONV_ERR_INVALID_ARG
    assert _create(_desc(W=2, padding=1)) == _abi.FCONV_ERR_INVALID_ARG
    assert _create(_desc(H=2, padding=0)) == _abi.FCONV_OK  # SAME pads it


@pytest.mark.parametrize("ops,dtype,ok", [
    ([1, 3], 0, True), ([1, 2, 3], 0, True), ([1, 2, 3, 5], 0, True), ([1, 3, 5], 0, True),
    ([3, 1], 0, False), ([1, 2], 0, False), ([3], 0, False), ([1, 3, 4], 0, False),
    ([1, 3, 5, 5], 0, False), ([], 0, False), ([1, 2, 2, 3], 0, False),
    ([], 1, True), ([3, 4, 5], 1, True), ([4, 5], 2, True), ([5], 2, True),
    ([3], 2, True), ([4, 3], 1, False), ([1, 3], 2, False), ([2], 1, False),
    ([5, 3], 2, False), ([9], 1, False),
    ([3, 4, 6], 1, True), ([3, 7], 2, True), ([8], 1, True), ([4, 8], 2, True),
    ([1, 3, 6], 0, False), ([1, 3, 8], 0, False), ([5, 6], 1, False), ([6, 5], 2, False),
    ([7, 3], 1, False), ([6, 7], 2, False)])
def test_operator_sequences(ops, dtype, ok):
    st = _create(_desc(ops=ops, dtype=dtype))
    assert st == (_abi.FCONV_OK if ok else _abi.FCONV_ERR_UNSUPPORTED)


def test_create_rejects_unknown_enums_and_flags():
    assert _create(_desc(dtype=7)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(padding=3)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(flags=2)) == _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(flags=_abi.FCONV_DESC_CUDNN7_ORDER)) == _abi.FCONV_OK
    assert _create(_desc(flags=_abi.FCONV_DESC_CUDNN7_ORDER, dtype=1, ops=[3])) == \
        _abi.FCONV_ERR_UNSUPPORTED
    assert _create(_desc(ops=list(range(9)))) == _abi.FCONV_ERR_INVALID_ARG
    assert _create(_desc(N=2 ** 20, H=2 ** 10, W=2 ** 10, C=4)) == _abi.FCONV_ERR_UNSUPPORTED


def test_null_pointers_are_rejected():
    L = _abi.lib()
    h = ctypes.c_void_p()
    assert L.fconv_plan_create(None, ctypes.byref(h)) == _abi.FCONV_ERR_INVALID_ARG
    assert L.fconv_plan_create(ctypes.byref(_desc()), None) == _abi.FCONV_ERR_INVALID_ARG
    assert L.fconv_plan_output_dims(None, None, None, None) == _abi.FCONV_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert L.fconv_plan_workspace_size(None, ctypes.byref(n)) == _abi.FCONV_ERR_INVALID_ARG
    assert L.fconv_plan_run(None, None, None) == _abi.FCONV_ERR_INVALID_ARG
    assert L.fconv_plan_destroy(None) == _abi.FCONV_OK
    assert L.fconv_plan_kernel_name(None) is None


def test_output_dims_match_oracle_geometry():
    """The plan's size/padding resolution is independent code from the
    oracle's; the two must agree over a grid of shapes."""
    for H in range(1, 30, 3):
        for R in range(1, 7):
            for st in range(1, 4):
                for same in (True, False):
                    if not same and H < R:
                        continue
                    p = fc.Plan(1, H, H + 1, 4, 4, R, R, stride=st,
                                padding="SAME" if same else "VALID")
                    g = oracle.geometry(H, H + 1, R, R, st, st, same)
                    assert (p.Ho, p.Wo) + p.pads == g


def test_workload_plans():
    for L in wl.LAYERS.values():
        ops = [wl.OP_SCALE, wl.OP_SIDE, wl.OP_BIAS, wl.OP_BN, wl.OP_RELU]
        p = fc.Plan(L.N, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                    ops=[o for o in ops if o in L.ops])
        assert (p.Ho, p.Wo) == (L.Ho, L.Wo)
        esize = {"int8": 1, "bf16": 2, "fp32": 4}[L.dtype]
        # the packed filter holds at least the filter and at most whole tiles
        assert L.R * L.S * L.C * L.K * esize <= p.workspace_bytes
        kstep = 64 // esize
        # rows padded by one 16-byte chunk
        Kp = -(-L.K // 64) * 64
        packed = Kp * (-(-(L.R * L.S * L.C) // kstep) * kstep * esize + 16)
        if L.padding == "VALID" and (L.R, L.S) == (L.H, L.W):
            # full-size filter: the split GEMM's partial sums follow the
            # packed filter (256-byte aligned), one [N][Kp] tile per split
            assert p.kernel_name.startswith("conv_gemm_"), p.kernel_name
            part = p.workspace_bytes - (-(-packed // 256) * 256)
            assert part > 0 and part % (L.N * Kp * 4) == 0
        else:
            assert p.workspace_bytes == packed
        assert p.kernel_name
    p = fc.Plan(64, 56, 56, 128, 128, 3, 3, 2, "SAME", "int8", INT8_OPS)
    assert p.pads == (0, 1, 0, 1)


# ----------------------------------------------------------- run arg checks

FAKE = 1 << 40  # never dereferenced: every case below fails validation first


def _plan_and_args():
    p = fc.Plan(2, 8, 8, 16, 16, 3, 3, 1, "SAME", "int8", INT8_OPS)
    ws = p.workspace_bytes
    x, y, side, w, wsp = FAKE, FAKE + 2 ** 20, FAKE + 2 ** 21, FAKE + 2 ** 22, FAKE + 2 ** 23
    bias = FAKE + 2 ** 24
    kw = dict(bias=bias, side=side, conv_input_scale=1.0, side_input_scale=0.5)
    return p, (x, w, y, wsp), kw, ws


def _run(p, x, w, y, wsp, ws_bytes, **kw):
    a = p.make_args(x, w, y, wsp, workspace_bytes=ws_bytes, **kw)
    return p.run_args(a, stream=0)


def test_run_rejects_missing_pointers():
    p, (x, w, y, wsp), kw, ws = _plan_and_args()
    assert _run(p, None, w, y, wsp, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, w, None, wsp, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, None, y, wsp, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, w, y, wsp, ws, **dict(kw, bias=None)) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, w, y, wsp, ws, **dict(kw, side=None)) == _abi.FCONV_ERR_INVALID_ARG


def test_run_rejects_workspace_and_alignment():
    p, (x, w, y, wsp), kw, ws = _plan_and_args()
    assert _run(p, x, w, y, wsp, ws - 1, **kw) == _abi.FCONV_ERR_WORKSPACE
    assert _run(p, x, w, y, None, ws, **kw) == _abi.FCONV_ERR_WORKSPACE
    assert _run(p, x + 8, w, y, wsp, ws, **kw) == _abi.FCONV_ERR_MISALIGNED
    assert _run(p, x, w, y + 4, wsp, ws, **kw) == _abi.FCONV_ERR_MISALIGNED
    assert _run(p, x, w + 1, y, wsp, ws, **kw) == _abi.FCONV_ERR_MISALIGNED
    assert _run(p, x, w, y, wsp + 8, ws, **kw) == _abi.FCONV_ERR_MISALIGNED
    assert _run(p, x, w, y, wsp, ws, **dict(kw, side=kw["side"] + 8)) == _abi.FCONV_ERR_MISALIGNED
    assert _run(p, x, w, y, wsp, ws, **dict(kw, bias=kw["bias"] + 2)) == _abi.FCONV_ERR_MISALIGNED


def test_run_rejects_in_place_and_aliasing():
    p, (x, w, y, wsp), kw, ws = _plan_and_args()
    assert _run(p, x, w, x, wsp, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, w, kw["side"], wsp, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, w, wsp, wsp, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG
    assert _run(p, x, w, y, w, ws, **kw) == _abi.FCONV_ERR_INVALID_ARG  # w into workspace
    a = p.make_args(x, w, y, wsp, workspace_bytes=ws, **kw)
    a.flags = 0x10
    assert p.run_args(a, stream=0) == _abi.FCONV_ERR_UNSUPPORTED


def test_run_bn_requires_all_vectors():
    p = fc.Plan(1, 8, 8, 16, 16, 3, 3, 1, "SAME", "fp32", ("bias", "bn", "relu"))
    bn = dict(gamma=FAKE, beta=FAKE + 64, mean=FAKE + 128, var=None, eps=1e-5)
    st = _run(p, FAKE + 2 ** 20, FAKE + 2 ** 21, FAKE + 2 ** 22, FAKE + 2 ** 23,
              p.workspace_bytes, bias=FAKE + 256, bn=bn)
    assert st == _abi.FCONV_ERR_INVALID_ARG


def test_pack_filter_checks():
    p, (x, w, y, wsp), kw, ws = _plan_and_args()
    L = _abi.lib()
    assert L.fconv_plan_pack_filter(p.handle, None, None, wsp, ws) == _abi.FCONV_ERR_INVALID_ARG
    assert L.fconv_plan_pack_filter(p.handle, None, w, wsp, ws - 1) == _abi.FCONV_ERR_WORKSPACE
    assert L.fconv_plan_pack_filter(p.handle, None, w + 4, wsp, ws) == _abi.FCONV_ERR_MISALIGNED
    assert L.fconv_plan_pack_filter(p.handle, None, w, w, ws) == _abi.FCONV_ERR_INVALID_ARG


def test_python_binding_refuses_host_tensors():
    import torch
    p = fc.Plan(1, 8, 8, 16, 16, 3, 3)
    with pytest.raises(ValueError):
        p.run(torch.zeros(1, 8, 8, 16, dtype=torch.int8), None, None, None)


def test_cudnn7_plans_choose_the_same_kernel_family():
    """Every int8 kernel family implements both epilogue orders, so the flag
    does not change the kernel choice."""
    shapes = [(32, 56, 56, 64, 64, 3, 3, 1), (32, 56, 56, 256, 64, 1, 1, 1),
              (64, 56, 56, 128, 128, 3, 3, 2), (1, 8, 8, 8, 8, 3, 3, 1)]
    for N, H, W, C, K, R, S, st in shapes:
        p8 = fc.Plan(N, H, W, C, K, R, S, st, "SAME", "int8", INT8_OPS)
        p7 = fc.Plan(N, H, W, C, K, R, S, st, "SAME", "int8", INT8_OPS, cudnn7_order=True)
        assert p7.kernel_name == p8.kernel_name


def test_run_checks_per_channel_scales():
    p, (x, w, y, wsp), kw, ws = _plan_and_args()
    a = p.make_args(x, w, y, wsp, workspace_bytes=ws, **kw)
    a.conv_input_scales = FAKE + 2 ** 25 + 2  # not 4-byte aligned
    assert p.run_args(a, stream=0) == _abi.FCONV_ERR_MISALIGNED
    pf = fc.Plan(2, 8, 8, 16, 16, 3, 3, 1, "SAME", "fp32", ["bias"])
    af = pf.make_args(x, w, y, wsp, workspace_bytes=pf.workspace_bytes, bias=kw["bias"])
    af.conv_input_scales = FAKE + 2 ** 25
    assert pf.run_args(af, stream=0) == _abi.FCONV_ERR_UNSUPPORTED


def test_run_checks_activation_arguments():
    x, y, w, wsp, bias = FAKE, FAKE + 2 ** 20, FAKE + 2 ** 22, FAKE + 2 ** 23, FAKE + 2 ** 24
    for op, alpha, beta, ok in [("clamp", 0.5, 0.25, False), ("clamp", float("nan"), 1.0, False),
                                ("clamp", -1.0, float("inf"), False),
                                ("leaky_relu", float("inf"), 0.0, False),
                                ("clipped_relu", float("nan"), 0.0, False)]:
        p = fc.Plan(2, 8, 8, 16, 16, 3, 3, 1, "SAME", "fp32", ["bias", op])
        a = p.make_args(x, w, y, wsp, workspace_bytes=p.workspace_bytes, bias=bias,
                        activ_alpha=alpha, activ_beta=beta)
        assert p.run_args(a, stream=0) == _abi.FCONV_ERR_INVALID_ARG, (op, alpha, beta)


def test_autotune_checks_its_arguments():
    p, (x, w, y, wsp), kw, ws = _plan_and_args()
    L = _abi.lib()
    a = p.make_args(x, w, y, wsp, workspace_bytes=ws, **kw)
    assert L.fconv_plan_autotune(p.handle, None, ctypes.byref(a), 0, None) == \
        _abi.FCONV_ERR_INVALID_ARG
    assert L.fconv_plan_autotune(None, None, ctypes.byref(a), 5, None) == \
        _abi.FCONV_ERR_INVALID_ARG
    b = p.make_args(None, w, y, wsp, workspace_bytes=ws, **kw)
    assert L.fconv_plan_autotune(p.handle, None, ctypes.byref(b), 5, None) == \
        _abi.FCONV_ERR_INVALID_ARG
    fc.autotune_cache_clear()


def test_fconv_log_prints_the_plan_decisions():
    """FCONV_LOG=1: plan creation prints its decisions (kernel family, tiling,
    workspace) on stderr; checked in a child process so the environment
    variable is read fresh."""
    import subprocess
    import sys
    code = ("import convolution_implicit_gemm_nhwc_amd as fc\n"
            "fc.Plan(32, 56, 56, 64, 64, 3, 3, 1, 'SAME', 'int8',"
            " ops=('scale', 'side', 'bias', 'relu'))\n"
            "fc.WgradPlan(2, 9, 7, 16, 24, 3, 3, 1, 'SAME', 'bf16')\n")
    env = dict(os.environ, FCONV_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("fconv:")]
    assert any("kernel=conv_halo_i8" in l and "Ho=56" in l and "pads(t,b,l,r)=1,1,1,1" in l
               for l in lines), r.stderr
    assert any(l.startswith("fconv: wgrad plan") and "kernel=wgrad_" in l for l in lines), r.stderr
    env["FCONV_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert not [l for l in r.stderr.splitlines() if l.startswith("fconv:")]
