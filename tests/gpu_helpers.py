"""Shared helpers of the GPU tests: run the HIP path through the C ABI on
torch device buffers, and compute the oracle's answer for the same inputs."""
import sys

import numpy as np
import torch

import convolution_implicit_gemm_nhwc_amd as fc
import oracle
import workloads as wl

OPNAMES = {wl.OP_SCALE: "scale", wl.OP_SIDE: "side", wl.OP_BIAS: "bias", wl.OP_BN: "bn",
           wl.OP_RELU: "relu"}

# Tolerances on e = max|y - r| / max|r| (normwise; ReLU zeros make element-wise
# ratios meaningless): fp32 1e-5, bf16 2e-2, both against the float64 oracle.
TOL = {"fp32": 1e-5, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


def to_dev(a, dev):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def from_dev(t, dtype):
    if dtype == "bf16":
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return wl.bf16_bits_to_float(bits).astype(np.float64)
    return t.cpu().numpy()


def make_plan(N, H, W, C, K, R, S, stride, padding, dtype, ops, cudnn7_order=False):
    return fc.Plan(N, H, W, C, K, R, S, stride, padding, dtype,
                   ops=[OPNAMES[o] if isinstance(o, int) else o for o in ops],
                   cudnn7_order=cudnn7_order)


def run_gpu(plan, dtype, x, w, bias=None, side=None, cis=1.0, sis=0.0, bn=None,
            prepacked_ws=None, guard=0, dev=None, activ=(0.0, 0.0), raw_bits=False):
    """Run the plan on device copies of numpy inputs; returns (y, guards_ok)
    (y as bf16 bit patterns, uint16, for a bf16 plan with raw_bits)."""
    dev = dev or device()
    tdt = {"int8": torch.int8, "bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    esize = {"int8": 1, "bf16": 2, "fp32": 4}[dtype]
    n_out = int(np.prod(plan.out_shape))
    # y inside a guarded byte buffer: `guard` bytes of 0x5A on both sides.
    g = (guard + 15) // 16 * 16
    raw = torch.full((2 * g + n_out * esize + 16,), 0x5A, dtype=torch.uint8, device=dev)
    y = raw[g:g + n_out * esize].view(tdt).view(plan.out_shape)
    xd, wd = to_dev(x, dev), to_dev(w, dev)
    bd, sd = to_dev(bias, dev), to_dev(side, dev)
    bnd = None
    if bn is not None:
        bnd = {k: to_dev(np.asarray(bn[k], np.float32), dev) for k in ("gamma", "beta", "mean",
                                                                     "var")}
        bnd["eps"] = float(bn["eps"])
    if prepacked_ws is not None:
        ws = prepacked_ws
    else:
        ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    # cis: a scalar, or a numpy fp32 vector of one scale per output channel
    cis_arg = to_dev(np.asarray(cis, np.float32), dev) if np.ndim(cis) > 0 else float(cis)
    plan.run(xd, wd, y, ws, bias=bd, side=sd, conv_input_scale=cis_arg,
             side_input_scale=float(sis), bn=bnd, prepacked=prepacked_ws is not None,
             activ_alpha=float(activ[0]), activ_beta=float(activ[1]))
    torch.cuda.synchronize()
    if raw_bits and dtype == "bf16":
        out = y.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        out = from_dev(y, dtype)
    guards_ok = True
    if g:
        rb = raw.cpu().numpy()
        guards_ok = bool((rb[:g] == 0x5A).all() and (rb[g + n_out * esize:] == 0x5A).all())
    return out, guards_ok


def oracle_out(dtype, x, w, stride, padding, bias=None, side=None, cis=1.0, sis=0.0,
               relu=False, bn=None, use_bias=True, order=8):
    if dtype == "int8":
        c = np.asarray(cis, np.float32) if np.ndim(cis) > 0 else np.float32(cis)
        return oracle.fused_conv_i8(x, w, bias, c, side, np.float32(sis), relu,
                                    stride, padding, order=order)
    return oracle.fused_conv_float(x, w, bias if use_bias else None, bn, relu, stride, padding)


def float_error(y, r):
    den = float(np.max(np.abs(r)))
    return float(np.max(np.abs(y - r))) / (den if den > 0 else 1.0)
