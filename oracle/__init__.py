"""CPU oracle for the fused NHWC convolution (numpy front end over oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the library under
``convolution_implicit_gemm_nhwc_amd`` never does, and shares no code with it.

Every function here is argument marshalling around ``oracle.c``; the
arithmetic lives there and is documented there, with the passages of the
pages it follows:

* geometry: TensorFlow conv_ops_fused_int8.cc, LaunchFusedConv2DOpGpuInt8Helper
  (SAME padding total and its split) and conv_grad_filter_ops.cc, Im2col (the
  output-size expression);
* contraction: direct seven-loop form and the Im2col patch-matrix form;
* int8 epilogue: conv_ops_fused_int8.cc, BiasActivationOutputKernel (cuDNN 8
  order: scale, side-input FMA, bias, round half to even, clip, cast);
* float epilogue: MIOpen "Using the fusion API" (operators apply in creation
  order; conv -> bias -> batch-norm inference -> activation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# FCONV_ORACLE_LIBRARY (environment): load another build of oracle.c (e.g. one
# built under sanitizers) instead of liboracle.so.
_LOAD_PATH = os.environ.get("FCONV_ORACLE_LIBRARY") or _LIB_PATH

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-shared", "-fPIC", "-Wall"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _bind(lib):
    """Declare the C signatures on a loaded oracle library; returns it."""
    p = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_geometry.argtypes = [i, i, i, i, i, i, i, p]
    lib.oracle_output_hw.argtypes = [p, p]
    for name in ("oracle_conv_i8_direct", "oracle_conv_i8_im2col",
                 "oracle_conv_f32_direct", "oracle_conv_bf16_direct"):
        getattr(lib, name).argtypes = [p, p, p, p]
        getattr(lib, name).restype = i
    lib.oracle_epilogue_i8.argtypes = [p, ctypes.c_long, i, ctypes.c_float, p,
                                       ctypes.c_float, p, i, p]
    lib.oracle_epilogue_i8.restype = None
    lib.oracle_epilogue_i8_ex.argtypes = [p, ctypes.c_long, i, ctypes.c_float, p, p,
                                          ctypes.c_float, p, i, i, p]
    lib.oracle_epilogue_i8_ex.restype = None
    lib.oracle_epilogue_float.argtypes = [p, ctypes.c_long, i, p, p, p, p, p,
                                          ctypes.c_float, i, p]
    lib.oracle_epilogue_float.restype = None
    lib.oracle_epilogue_float_ex.argtypes = [p, ctypes.c_long, i, p, p, p, p, p,
                                             ctypes.c_float, i, ctypes.c_float,
                                             ctypes.c_float, p]
    lib.oracle_epilogue_float_ex.restype = None
    lib.oracle_wgrad_direct.argtypes = [p, p, p, p]
    lib.oracle_wgrad_direct.restype = i
    lib.oracle_num_threads.restype = i
    lib.oracle_set_num_threads.argtypes = [i]
    lib.oracle_set_num_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LOAD_PATH))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def geometry(H, W, R, S, stride_h, stride_w, same):
    """(Ho, Wo, pad_top, pad_bottom, pad_left, pad_right) for SAME or VALID."""
    out = np.zeros(6, dtype=np.int32)
    rc = _load().oracle_geometry(H, W, R, S, stride_h, stride_w, int(bool(same)),
                                 _ptr(out))
    if rc != 0:
        raise OracleError("invalid geometry (rc=%d)" % rc)
    return tuple(int(v) for v in out)


def _shape_block(x, w, stride, pads):
    N, H, W, C = x.shape
    R, S, Cw, K = w.shape
    if Cw != C:
        raise OracleError("filter depth %d != input depth %d" % (Cw, C))
    sh, sw = stride
    pt, pb, pl, pr = pads
    d = np.array([N, H, W, C, K, R, S, sh, sw, pt, pb, pl, pr], dtype=np.int32)
    hw = np.zeros(2, dtype=np.int32)
    if _load().oracle_output_hw(_ptr(d), _ptr(hw)) != 0:
        raise OracleError("invalid shape block")
    return d, (N, int(hw[0]), int(hw[1]), K)


def resolve(x_shape, w_shape, stride, padding):
    """Stride pair and explicit pads from 'SAME' / 'VALID' or explicit pads."""
    if isinstance(stride, int):
        stride = (stride, stride)
    if isinstance(padding, str):
        g = geometry(x_shape[1], x_shape[2], w_shape[0], w_shape[1], stride[0],
                     stride[1], padding.upper() == "SAME")
        pads = g[2:]
    else:
        pads = tuple(padding)
    return tuple(stride), pads


def conv_acc(x, w, stride=1, padding="SAME", form="direct"):
    """Raw accumulator of the convolution.

    int8 x/w -> int32 (exact); float32 -> float64; bf16 given as uint16 bit
    patterns -> float64.  form = "direct" or "im2col" (int8 only).
    """
    stride, pads = resolve(x.shape, w.shape, stride, padding)
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    d, oshape = _shape_block(x, w, stride, pads)
    lib = _load()
    if x.dtype == np.int8 and w.dtype == np.int8:
        acc = np.empty(oshape, dtype=np.int32)
        fn = lib.oracle_conv_i8_im2col if form == "im2col" else lib.oracle_conv_i8_direct
    elif form != "direct":
        raise OracleError("im2col form is int8 only")
    elif x.dtype == np.float32 and w.dtype == np.float32:
        acc = np.empty(oshape, dtype=np.float64)
        fn = lib.oracle_conv_f32_direct
    elif x.dtype == np.uint16 and w.dtype == np.uint16:
        acc = np.empty(oshape, dtype=np.float64)
        fn = lib.oracle_conv_bf16_direct
    else:
        raise OracleError("unsupported dtypes %s/%s" % (x.dtype, w.dtype))
    rc = fn(_ptr(x), _ptr(w), _ptr(d), _ptr(acc))
    if rc != 0:
        raise OracleError("conv failed (rc=%d)" % rc)
    return acc


def _as_f64(a):
    """float64 copy of float32 data or of bf16 given as uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def wgrad(x, dy, R, S, stride=1, padding="SAME"):
    """Filter gradient dW [R][S][C][K] (float64) of the convolution with
    input x (NHWC) and output gradient dy (N, Ho, Wo, K); x and dy float32 or
    bf16 bit patterns (uint16)."""
    x64 = _as_f64(x)
    dy64 = _as_f64(dy)
    K = dy64.shape[-1]
    w_shape = (R, S, x64.shape[-1], K)
    stride, pads = resolve(x64.shape, w_shape, stride, padding)
    d, oshape = _shape_block(x64, np.empty(w_shape), stride, pads)
    if tuple(dy64.shape) != oshape:
        raise OracleError("dy shape %s != output shape %s" % (dy64.shape, oshape))
    dw = np.empty(w_shape, dtype=np.float64)
    rc = _load().oracle_wgrad_direct(_ptr(x64), _ptr(dy64), _ptr(d), _ptr(dw))
    if rc != 0:
        raise OracleError("wgrad failed (rc=%d)" % rc)
    return dw


def epilogue_i8(acc, conv_input_scale, bias, side=None, side_input_scale=0.0,
                relu=False, order=8):
    """int8 fused epilogue over an NHWC int32 accumulator; returns int8 NHWC.

    conv_input_scale: a scalar, or one fp32 value per output channel.
    order: 8 (cuDNN 8 order: scale, side, bias) or 7 (cuDNN 7 order:
    fmaf(acc, scale, bias), then side).
    """
    if order not in (7, 8):
        raise OracleError("order must be 7 or 8")
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    K = acc.shape[-1]
    M = acc.size // K
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    if side is not None:
        side = np.ascontiguousarray(side, dtype=np.int8)
        if side.shape != acc.shape:
            raise OracleError("side input must have the output's shape")
    scales = None
    if np.ndim(conv_input_scale) > 0:
        scales = np.ascontiguousarray(conv_input_scale, dtype=np.float32).reshape(-1)
        if scales.size != K:
            raise OracleError("a conv_input_scale vector needs one value per output channel")
        conv_input_scale = 0.0
    y = np.empty(acc.shape, dtype=np.int8)
    _load().oracle_epilogue_i8_ex(_ptr(acc), M, K, float(conv_input_scale), _ptr(scales),
                                  _ptr(side), float(side_input_scale), _ptr(bias),
                                  int(bool(relu)), int(order), _ptr(y))
    return y


ACTIVATIONS = {None: 0, "relu": 1, "leaky_relu": 2, "clipped_relu": 3, "clamp": 4}


def epilogue_float(acc, bias=None, bn=None, relu=False, act=None, alpha=0.0, beta=0.0):
    """bias -> batch-norm inference -> activation in double.

    bn = dict(gamma=, beta=, mean=, var=, eps=) or None.  The activation is
    `act` (None, "relu", "leaky_relu", "clipped_relu", "clamp") with its
    arguments alpha and beta; relu=True is act="relu".
    """
    if relu:
        act = act or "relu"
    if act not in ACTIVATIONS:
        raise OracleError("unknown activation %r" % (act,))
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    K = acc.shape[-1]
    M = acc.size // K
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    bias = f32(bias)
    if bn is not None:
        g, b, mu, var = (f32(bn[k]) for k in ("gamma", "beta", "mean", "var"))
        eps = float(bn["eps"])
    else:
        g = b = mu = var = None
        eps = 0.0
    y = np.empty(acc.shape, dtype=np.float64)
    _load().oracle_epilogue_float_ex(_ptr(acc), M, K, _ptr(bias), _ptr(g), _ptr(b),
                                     _ptr(mu), _ptr(var), eps, ACTIVATIONS[act], float(alpha),
                                     float(beta), _ptr(y))
    return y


def fused_conv_i8(x, w, bias, conv_input_scale, side=None, side_input_scale=0.0,
                  relu=False, stride=1, padding="SAME", form="direct", order=8):
    acc = conv_acc(x, w, stride, padding, form)
    return epilogue_i8(acc, conv_input_scale, bias, side, side_input_scale, relu, order)


def fused_conv_float(x, w, bias=None, bn=None, relu=False, stride=1,
                     padding="SAME", act=None, alpha=0.0, beta=0.0):
    acc = conv_acc(x, w, stride, padding)
    return epilogue_float(acc, bias, bn, relu, act, alpha, beta)


def num_threads():
    return int(_load().oracle_num_threads())


def set_num_threads(n: int):
    """Threads of the oracle's OpenMP loops from now on (for baseline timing)."""
    _load().oracle_set_num_threads(int(n))
