"""ctypes declarations of the C ABI in include/fconv.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

# FCONV_LIBRARY (environment) loads another build of the same library
# instead, e.g. one with the host code built under address and
# undefined-behaviour sanitizers.
_LIB_PATH = os.environ.get("FCONV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfconv.so")

FCONV_OK = 0
FCONV_ERR_INVALID_ARG = 1
FCONV_ERR_UNSUPPORTED = 2
FCONV_ERR_WORKSPACE = 3
FCONV_ERR_MISALIGNED = 4
FCONV_ERR_DEVICE = 5

FCONV_INT8, FCONV_BF16, FCONV_FP32 = 0, 1, 2
FCONV_PAD_SAME, FCONV_PAD_VALID = 0, 1
OP_SCALE, OP_SIDE, OP_BIAS, OP_BN, OP_RELU = 1, 2, 3, 4, 5
OP_LEAKY_RELU, OP_CLIPPED_RELU, OP_CLAMP = 6, 7, 8
FCONV_MAX_OPS = 8
FCONV_RUN_FILTER_PREPACKED = 1
FCONV_DESC_CUDNN7_ORDER = 1
FCONV_WGRAD_OUT_FP32 = 1
FCONV_NO_ALLOC_SCRATCH_BYTES = 4 << 20

# Every symbol include/fconv.h declares.
EXPORTS = ("fconv_plan_create", "fconv_plan_output_dims", "fconv_plan_workspace_size",
           "fconv_plan_pack_filter", "fconv_plan_run", "fconv_plan_destroy",
           "fconv_plan_kernel_name", "fconv_status_string", "fconv_plan_autotune",
           "fconv_autotune_cache_clear", "fconv_wgrad_plan_create",
           "fconv_wgrad_plan_output_dims", "fconv_wgrad_plan_workspace_size",
           "fconv_wgrad_plan_run", "fconv_wgrad_plan_kernel_name",
           "fconv_wgrad_plan_destroy", "fconv_plan_run_no_alloc")


class FconvDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("N", "H", "W", "C", "K", "R", "S", "stride_h", "stride_w", "padding",
                 "dtype", "n_ops")] + [("ops", ctypes.c_int32 * FCONV_MAX_OPS),
                                       ("flags", ctypes.c_uint32)]


class FconvArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("side", ctypes.c_void_p), ("conv_input_scale", ctypes.c_float),
                ("side_input_scale", ctypes.c_float), ("bn_gamma", ctypes.c_void_p),
                ("bn_beta", ctypes.c_void_p), ("bn_mean", ctypes.c_void_p),
                ("bn_var", ctypes.c_void_p), ("bn_eps", ctypes.c_float),
                ("y", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32),
                ("conv_input_scales", ctypes.c_void_p), ("activ_alpha", ctypes.c_float),
                ("activ_beta", ctypes.c_float)]


class LibraryMissing(RuntimeError):
    pass


_lib = None


def lib():
    """The loaded libfconv.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise LibraryMissing(
                "libfconv.so is not built (run python -m "
                "convolution_implicit_gemm_nhwc_amd.build); no fallback exists")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        st = ctypes.c_int
        L.fconv_plan_create.argtypes = [ctypes.POINTER(FconvDesc), ctypes.POINTER(P)]
        L.fconv_plan_create.restype = st
        L.fconv_plan_output_dims.argtypes = [P, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_int32)]
        L.fconv_plan_output_dims.restype = st
        L.fconv_plan_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.fconv_plan_workspace_size.restype = st
        L.fconv_plan_pack_filter.argtypes = [P, P, P, P, ctypes.c_size_t]
        L.fconv_plan_pack_filter.restype = st
        L.fconv_plan_run.argtypes = [P, P, ctypes.POINTER(FconvArgs)]
        L.fconv_plan_run.restype = st
        L.fconv_plan_run_no_alloc.argtypes = [P, P, ctypes.POINTER(FconvArgs)]
        L.fconv_plan_run_no_alloc.restype = st
        L.fconv_plan_destroy.argtypes = [P]
        L.fconv_plan_destroy.restype = st
        L.fconv_plan_kernel_name.argtypes = [P]
        L.fconv_plan_kernel_name.restype = ctypes.c_char_p
        L.fconv_plan_autotune.argtypes = [P, P, ctypes.POINTER(FconvArgs), ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_float)]
        L.fconv_plan_autotune.restype = st
        L.fconv_autotune_cache_clear.argtypes = []
        L.fconv_autotune_cache_clear.restype = None
        L.fconv_wgrad_plan_create.argtypes = [ctypes.POINTER(FconvDesc), ctypes.POINTER(P)]
        L.fconv_wgrad_plan_create.restype = st
        L.fconv_wgrad_plan_output_dims.argtypes = [P, ctypes.POINTER(ctypes.c_int32),
                                                   ctypes.POINTER(ctypes.c_int32),
                                                   ctypes.POINTER(ctypes.c_int32)]
        L.fconv_wgrad_plan_output_dims.restype = st
        L.fconv_wgrad_plan_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.fconv_wgrad_plan_workspace_size.restype = st
        L.fconv_wgrad_plan_run.argtypes = [P, P, P, P, P, P, ctypes.c_size_t]
        L.fconv_wgrad_plan_run.restype = st
        L.fconv_wgrad_plan_kernel_name.argtypes = [P]
        L.fconv_wgrad_plan_kernel_name.restype = ctypes.c_char_p
        L.fconv_wgrad_plan_destroy.argtypes = [P]
        L.fconv_wgrad_plan_destroy.restype = st
        L.fconv_status_string.argtypes = [st]
        L.fconv_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def lib_path() -> str:
    return _LIB_PATH
