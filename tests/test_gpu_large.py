"""Element counts beyond 2^31 and 2^32 per rank (64-bit offsets everywhere).

Ring AllReduce of 2 ranks x (2^32 + 37) int8 elements and RHD AllReduce of
3 ranks x (2^31 + 5) fp16 elements (non-power-of-two merge and restore):
every rank's whole buffer checked bit for bit against the oracle's replay
(run as windows on the host's cores), and all ranks identical on the GPU.
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
    xs, dev = [], []
    for r in range(P):
        xs.append(gen(r, 0, L))
        dev.append(to_dev(xs[-1], dtype))
    with hc.Comm(P, algo) as c:
        say("case large: allreduce")
        c.allreduce(dev, dtype, "sum")
        torch.cuda.synchronize()
    iv = torch.int8 if dtype == "int8" else torch.int16
    assert all(torch.equal(d.view(iv), dev[0].view(iv)) for d in dev[1:])
    say("case large: oracle replay")
    oracle.run_parallel("allreduce", algo, xs, dtype, "sum")  # in place: xs now holds the expected result
    ui = np.uint8 if dtype == "int8" else np.uint16
    for r in range(P):
        say(f"case large: compare rank {r}")
        got = to_host(dev[r], dtype)
        if not np.array_equal(got.view(ui), xs[r].view(ui)):
            refops.assert_same(dtype, got, xs[r], f"{algo} rank {r}")
        del got
    del dev, xs
    torch.cuda.empty_cache()
