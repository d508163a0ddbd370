"""Fused NHWC implicit-GEMM convolution for AMD MI355X (gfx950).

Python binding over the C ABI of ``include/fconv.h`` (``libfconv.so``).  It
only marshals arguments: every step of the convolution and its epilogue runs
in the library's HIP kernels.  Tensors are torch tensors on the GPU (torch
provides device memory and streams) or raw device addresses given as ints.

    plan = Plan(N, H, W, C, K, R, S, stride=1, padding="SAME", dtype="int8",
                ops=("scale", "side", "bias", "relu"))
    y = plan(x, w, bias=b, side=s, conv_input_scale=2**-11, side_input_scale=0.25)

    g = WgradPlan(N, H, W, C, K, R, S, stride=1, padding="SAME", dtype="bf16")
    dw = g(x, dy)          # filter gradient, HWIO
"""
from __future__ import annotations

import ctypes

from . import _abi

__all__ = ["Plan", "WgradPlan", "FconvError", "DTYPES", "OPS"]

DTYPES = {"int8": _abi.FCONV_INT8, "bf16": _abi.FCONV_BF16, "fp32": _abi.FCONV_FP32}
OPS = {"scale": _abi.OP_SCALE, "side": _abi.OP_SIDE, "bias": _abi.OP_BIAS,
       "bn": _abi.OP_BN, "relu": _abi.OP_RELU, "leaky_relu": _abi.OP_LEAKY_RELU,
       "clipped_relu": _abi.OP_CLIPPED_RELU, "clamp": _abi.OP_CLAMP}
PADDINGS = {"SAME": _abi.FCONV_PAD_SAME, "VALID": _abi.FCONV_PAD_VALID}


class FconvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _abi.lib().fconv_status_string(status).decode()
        super().__init__("%s: %s (status %d)" % (what, msg, status))


def _check(status: int, what: str):
    if status != _abi.FCONV_OK:
        raise FconvError(status, what)


def _addr(t):
    """Device address of a torch GPU tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU (got %s)" % t.device)
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


_TORCH_DTYPES = {"int8": ("torch.int8",), "bf16": ("torch.bfloat16",),
                 "fp32": ("torch.float32",)}


def _validate(checks):
    """Checks every (tensor, name, numel, dtypes) against what the plan
    expects: at least `numel` elements of one of `dtypes` (torch dtype
    names).  The kernels size their reads and writes from the plan, not from
    the allocation, so a short or mistyped tensor is rejected here, before
    any device address is taken or the C ABI is called (a longer one is
    safe: only its first `numel` elements are touched).  None is skipped; an
    int is a raw device address, which the caller vouches for."""
    for t, what, numel, dtypes in checks:
        if t is None or isinstance(t, int):
            continue
        if str(t.dtype) not in dtypes:
            raise ValueError("%s: dtype %s, expected %s" % (what, t.dtype, " or ".join(dtypes)))
        if t.numel() < numel:
            raise ValueError("%s: %d elements, the plan needs %d" % (what, t.numel(), numel))


def _nbytes(t, default):
    """Byte size of a workspace tensor (a raw address: `default`)."""
    return t.numel() * t.element_size() if hasattr(t, "numel") else default


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """A resolved fused-conv plan (geometry, dtype, ordered epilogue ops)."""

    def __init__(self, N, H, W, C, K, R, S, stride=1, padding="SAME", dtype="int8",
                 ops=("scale", "bias"), cudnn7_order=False):
        sh, sw = (stride, stride) if isinstance(stride, int) else stride
        d = _abi.FconvDesc()
        d.N, d.H, d.W, d.C, d.K, d.R, d.S = N, H, W, C, K, R, S
        d.stride_h, d.stride_w = sh, sw
        d.padding = PADDINGS[padding.upper()] if isinstance(padding, str) else padding
        d.dtype = DTYPES[dtype] if isinstance(dtype, str) else dtype
        codes = [OPS[o] if isinstance(o, str) else int(o) for o in ops]
        if len(codes) > _abi.FCONV_MAX_OPS:
            raise ValueError("too many ops")
        d.n_ops = len(codes)
        for i, c in enumerate(codes):
            d.ops[i] = c
        d.flags = _abi.FCONV_DESC_CUDNN7_ORDER if cudnn7_order else 0
        self.desc = d
        self.dtype = dtype
        self._h = ctypes.c_void_p()
        _check(_abi.lib().fconv_plan_create(ctypes.byref(d), ctypes.byref(self._h)),
               "fconv_plan_create")
        ho, wo = ctypes.c_int32(), ctypes.c_int32()
        pads = (ctypes.c_int32 * 4)()
        _check(_abi.lib().fconv_plan_output_dims(self._h, ctypes.byref(ho),
                                                 ctypes.byref(wo), pads),
               "fconv_plan_output_dims")
        self.Ho, self.Wo = ho.value, wo.value
        self.pads = tuple(pads)
        nbytes = ctypes.c_size_t()
        _check(_abi.lib().fconv_plan_workspace_size(self._h, ctypes.byref(nbytes)),
               "fconv_plan_workspace_size")
        self.workspace_bytes = nbytes.value
        self.kernel_name = _abi.lib().fconv_plan_kernel_name(self._h).decode()
        self.out_shape = (N, self.Ho, self.Wo, K)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _abi.lib().fconv_plan_destroy(h)
            self._h = ctypes.c_void_p()

    @property
    def handle(self):
        return self._h

    def pack_filter(self, w, workspace, stream=None):
        d = self.desc
        _validate([(w, "w", d.R * d.S * d.C * d.K, _TORCH_DTYPES[self.dtype])])
        _check(_abi.lib().fconv_plan_pack_filter(
            self._h, _stream_handle(stream), _addr(w), _addr(workspace),
            _nbytes(workspace, self.workspace_bytes)),
            "fconv_plan_pack_filter")

    def make_args(self, x, w, y, workspace, bias=None, side=None, conv_input_scale=1.0,
                  side_input_scale=0.0, bn=None, prepacked=False, workspace_bytes=None,
                  activ_alpha=0.0, activ_beta=0.0):
        d = self.desc
        K = d.K
        dt = _TORCH_DTYPES[self.dtype]
        f32 = ("torch.float32",)
        n_out = self.out_shape[0] * self.out_shape[1] * self.out_shape[2] * K
        cis_vec = conv_input_scale if hasattr(conv_input_scale, "data_ptr") else None
        checks = [(x, "x", d.N * d.H * d.W * d.C, dt), (w, "w", d.R * d.S * d.C * K, dt),
                  (y, "y", n_out, dt), (bias, "bias", K, f32),
                  (side, "side", n_out, ("torch.int8",)),
                  (cis_vec, "conv_input_scale", K, f32)]
        if bn is not None:
            checks += [(bn[k], "bn " + k, K, f32) for k in ("gamma", "beta", "mean", "var")]
        _validate(checks)
        a = _abi.FconvArgs()
        a.x, a.w, a.y = _addr(x), _addr(w), _addr(y)
        if workspace_bytes is None:
            workspace_bytes = _nbytes(workspace, self.workspace_bytes)
        a.workspace = _addr(workspace)
        a.workspace_bytes = workspace_bytes
        a.bias, a.side = _addr(bias), _addr(side)
        if cis_vec is not None:
            # One fp32 value per output channel, on the GPU.
            a.conv_input_scales = _addr(cis_vec)
            a.conv_input_scale = 0.0
        else:
            a.conv_input_scale = conv_input_scale
        a.side_input_scale = side_input_scale
        if bn is not None:
            a.bn_gamma, a.bn_beta = _addr(bn["gamma"]), _addr(bn["beta"])
            a.bn_mean, a.bn_var = _addr(bn["mean"]), _addr(bn["var"])
            a.bn_eps = bn["eps"]
        a.flags = _abi.FCONV_RUN_FILTER_PREPACKED if prepacked else 0
        a.activ_alpha, a.activ_beta = activ_alpha, activ_beta
        return a

    def run_args(self, args, stream=None) -> int:
        """Enqueue with a prepared FconvArgs; returns the raw status."""
        return _abi.lib().fconv_plan_run(self._h, _stream_handle(stream), ctypes.byref(args))

    def run_no_alloc_args(self, args, stream=None) -> int:
        """fconv_plan_run_no_alloc with a prepared FconvArgs (its workspace
        fields are ignored); returns the raw status."""
        return _abi.lib().fconv_plan_run_no_alloc(self._h, _stream_handle(stream),
                                                  ctypes.byref(args))

    def run_no_alloc(self, x, w, y, stream=None, **kw):
        """Run with the library's own device scratch instead of a workspace
        (fconv_plan_run_no_alloc): nothing is allocated per call."""
        _check(self.run_no_alloc_args(self.make_args(x, w, y, None, workspace_bytes=0, **kw),
                                      stream), "fconv_plan_run_no_alloc")
        return y

    def autotune(self, x, w, y, workspace, repeats=20, stream=None, **kw):
        """Time every kernel configuration for this shape on these buffers and
        keep the fastest (see fconv_plan_autotune); returns its microseconds
        per launch.  y holds the chosen configuration's result."""
        best = ctypes.c_float()
        _check(_abi.lib().fconv_plan_autotune(self._h, _stream_handle(stream),
                                              ctypes.byref(self.make_args(x, w, y, workspace,
                                                                          **kw)),
                                              int(repeats), ctypes.byref(best)),
               "fconv_plan_autotune")
        self.kernel_name = _abi.lib().fconv_plan_kernel_name(self._h).decode()
        return best.value

    def run(self, x, w, y, workspace, stream=None, **kw):
        _check(self.run_args(self.make_args(x, w, y, workspace, **kw), stream),
               "fconv_plan_run")
        return y

    def __call__(self, x, w, stream=None, **kw):
        """Allocate y and the workspace with torch, run, return y."""
        import torch
        tdt = {"int8": torch.int8, "bf16": torch.bfloat16, "fp32": torch.float32}[self.dtype]
        y = torch.empty(self.out_shape, dtype=tdt, device=x.device)
        ws = torch.empty(max(self.workspace_bytes, 16), dtype=torch.uint8, device=x.device)
        return self.run(x, w, y, ws, stream=stream, **kw)


class WgradPlan:
    """Weight gradient of the convolution with this geometry (see
    fconv_wgrad_plan_create): dw[r,s,c,k] = sum over n, ho, wo of the input
    under tap (r, s) times dy[n,ho,wo,k].  dtype "bf16" or "fp32"; a bf16
    plan writes dw in bf16, or in fp32 with out_fp32=True."""

    def __init__(self, N, H, W, C, K, R, S, stride=1, padding="SAME", dtype="bf16",
                 out_fp32=False):
        sh, sw = (stride, stride) if isinstance(stride, int) else stride
        d = _abi.FconvDesc()
        d.N, d.H, d.W, d.C, d.K, d.R, d.S = N, H, W, C, K, R, S
        d.stride_h, d.stride_w = sh, sw
        d.padding = PADDINGS[padding.upper()] if isinstance(padding, str) else padding
        d.dtype = DTYPES[dtype] if isinstance(dtype, str) else dtype
        d.n_ops = 0
        d.flags = _abi.FCONV_WGRAD_OUT_FP32 if out_fp32 else 0
        self.desc = d
        self.dtype = dtype
        self.out_dtype = "fp32" if (out_fp32 or dtype == "fp32") else dtype
        self._h = ctypes.c_void_p()
        _check(_abi.lib().fconv_wgrad_plan_create(ctypes.byref(d), ctypes.byref(self._h)),
               "fconv_wgrad_plan_create")
        ho, wo = ctypes.c_int32(), ctypes.c_int32()
        pads = (ctypes.c_int32 * 4)()
        _check(_abi.lib().fconv_wgrad_plan_output_dims(self._h, ctypes.byref(ho),
                                                       ctypes.byref(wo), pads),
               "fconv_wgrad_plan_output_dims")
        self.Ho, self.Wo = ho.value, wo.value
        self.pads = tuple(pads)
        nbytes = ctypes.c_size_t()
        _check(_abi.lib().fconv_wgrad_plan_workspace_size(self._h, ctypes.byref(nbytes)),
               "fconv_wgrad_plan_workspace_size")
        self.workspace_bytes = nbytes.value
        self.kernel_name = _abi.lib().fconv_wgrad_plan_kernel_name(self._h).decode()
        self.dy_shape = (N, self.Ho, self.Wo, K)
        self.dw_shape = (R, S, C, K)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _abi.lib().fconv_wgrad_plan_destroy(h)
            self._h = ctypes.c_void_p()

    def run_raw(self, x, dy, dw, workspace, workspace_bytes=None, stream=None) -> int:
        """Enqueue; returns the raw status (no exception)."""
        if workspace_bytes is None:
            workspace_bytes = _nbytes(workspace, self.workspace_bytes)
        d = self.desc
        dt = _TORCH_DTYPES[self.dtype]
        _validate([(x, "x", d.N * d.H * d.W * d.C, dt),
                   (dy, "dy", d.N * self.Ho * self.Wo * d.K, dt),
                   (dw, "dw", d.R * d.S * d.C * d.K, _TORCH_DTYPES[self.out_dtype])])
        ptrs = (_addr(x), _addr(dy), _addr(dw), _addr(workspace))
        return _abi.lib().fconv_wgrad_plan_run(self._h, _stream_handle(stream), *ptrs,
                                               workspace_bytes)

    def run(self, x, dy, dw, workspace, stream=None):
        _check(self.run_raw(x, dy, dw, workspace, stream=stream), "fconv_wgrad_plan_run")
        return dw

    def __call__(self, x, dy, stream=None):
        """Allocate dw and the workspace with torch, run, return dw."""
        import torch
        tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[self.out_dtype]
        dw = torch.empty(self.dw_shape, dtype=tdt, device=x.device)
        ws = torch.empty(max(self.workspace_bytes, 16), dtype=torch.uint8, device=x.device)
        return self.run(x, dy, dw, ws, stream=stream)


def autotune_cache_clear():
    """Forget every autotuned configuration of this process."""
    _abi.lib().fconv_autotune_cache_clear()
