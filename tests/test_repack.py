"""The filter repack (fconv_plan_pack_filter) against a numpy packing of the
same layout, byte for byte: rows of the packed filter are output channels,
each row the reduction (r, s, c) contiguous in the HWIO order the filter
arrives in (the [R*S*C, K] view of TensorFlow conv_ops_fused_int8.cc's GEMM
special cases, transposed), zero-padded to whole 64-byte k-steps and followed
by a 16-byte zero pad; K is padded to whole 64-row blocks with zero rows, and
inside each 64-row block row 16j + a holds output channel 16(a/4) + 4j + a%4
(so that an MFMA lane's outputs are 16 consecutive channels)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import device, make_plan, say, to_dev

pytestmark = pytest.mark.gpu

ESIZE = {"int8": 1, "bf16": 2, "fp32": 4}


def packed_reference(w, dtype):
    """numpy packing of an HWIO filter (int8, bf16 bits as uint16, fp32)."""
    R, S, C, K = w.shape
    es = ESIZE[dtype]
    kg = R * S * C
    kstep = 64 // es
    kgp = -(-kg // kstep) * kstep
    kp = -(-K // 64) * 64
    row_bytes = kgp * es + 16
    out = np.zeros((kp, row_bytes), np.uint8)
    wk = np.ascontiguousarray(w.reshape(kg, K))  # [(r, s, c)][k]
    for p in range(kp):
        blk, rr = divmod(p, 64)
        j, a = divmod(rr, 16)
        ch = 64 * blk + 16 * (a // 4) + 4 * j + a % 4
        if ch < K:
            out[p, :kg * es] = np.ascontiguousarray(wk[:, ch]).view(np.uint8)
    return out.reshape(-1)


@pytest.mark.parametrize("dtype", ["int8", "bf16", "fp32"])
@pytest.mark.parametrize("R,C,K", [(3, 64, 64), (3, 128, 200), (1, 24, 40), (5, 7, 13),
                                   (7, 64, 130), (2, 256, 64)])
def test_packed_filter_is_byte_exact(R, C, K, dtype):
    rng = np.random.default_rng(R * 1000 + C * 10 + K)
    if dtype == "int8":
        w = wl.draw_int8(rng, (R, R, C, K), -128, 127)
    else:
        w = rng.normal(0, 1, (R, R, C, K)).astype(np.float32)
        if dtype == "bf16":
            w = wl.float_to_bf16_bits(w)
    plan = make_plan(2, 9, 9, C, K, R, R, 1, "SAME", dtype,
                     [wl.OP_SCALE, wl.OP_BIAS] if dtype == "int8" else [wl.OP_BIAS])
    ref = packed_reference(w, dtype)
    dev = device()
    say("repack %s R=%d C=%d K=%d: %d packed bytes" % (dtype, R, C, K, ref.size))
    assert plan.workspace_bytes == ref.size
    ws = torch.full((plan.workspace_bytes,), 0xA5, dtype=torch.uint8, device=dev)
    plan.pack_filter(to_dev(w, dev), ws)
    torch.cuda.synchronize()
    got = ws.cpu().numpy()
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, "%d bytes differ, first at %d" % (bad.size, bad[0])
