"""Element counts beyond 2^31 and 2^32 per rank (64-bit offsets everywhere).

Ring AllReduce of 2 ranks x (2^32 + 37) int8 elements and RHD AllReduce of
3 ranks x (2^31 + 5) fp16 elements (non-power-of-two merge and restore),
checked bit for bit against the windowed oracle around every segment
boundary, the 2^31 / 2^32 element marks and the ends, and with all ranks
identical on the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
import synth
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("algo,P,L,dtype", [("ring", 2, (1 << 32) + 37, "int8"),
                                            ("rhd", 3, (1 << 31) + 5, "fp16")])
def test_beyond_32_bit_counts(algo, P, L, dtype):
    def gen(rank, first, n):
        if dtype == "int8":
            return synth.generate("int8", n, synth.UNIFORM_INT, -128, 127, stream=40, rank=rank, first=first)
        return synth.generate("fp16", n, synth.NORMAL, 1.0, stream=41, rank=rank, first=first)

    say(f"case large algo={algo} P={P} L={L} dtype={dtype}: upload")
    dev = []
    for r in range(P):
        x = gen(r, 0, L)
        dev.append(to_dev(x, dtype))
        del x
    with hc.Comm(P, algo) as c:
        say("case large: allreduce")
        c.allreduce(dev, dtype, "sum")
        torch.cuda.synchronize()
    iv = torch.int8 if dtype == "int8" else torch.int16
    assert all(torch.equal(d.view(iv), dev[0].view(iv)) for d in dev[1:])
    parts = P if algo == "ring" else 1 << (P.bit_length() - 1)
    q = -(-L // parts)
    marks = sorted({k * q for k in range(parts + 1)} | {1 << 31, 1 << 32, L})
    for m in marks:
        w0, w1 = max(0, m - 64), min(L, m + 64)
        if w0 >= w1:
            continue
        xs = [gen(r, w0, w1 - w0) for r in range(P)]
        want = [x.copy() for x in xs]
        oracle.run("allreduce", algo, want, dtype, "sum", L=L, w0=w0)
        for r in range(P):
            refops.assert_same(dtype, to_host(dev[r][w0:w1], dtype), want[r], f"window [{w0},{w1}) rank {r}")
    del dev
    torch.cuda.empty_cache()
