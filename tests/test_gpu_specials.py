"""IEEE special values through every launch form, bit for bit against the oracle.

The inputs mix ordinary values with signed zeros, infinities, quiet and
signalling NaNs, the least and greatest subnormals and the largest finite
values of each float type, so sums overflow to infinity, inf - inf and
0 * inf give NaN, subnormal sums round, and max / min see every ordering
case of the element ops (-0 below +0, any NaN giving the canonical quiet
NaN).  Sum / prod NaNs are compared as a class, max / min bit for bit.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
import synth
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

SPECIALS = {  # bit patterns
    "fp32": [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7FA00000, 0xFFC00001,
             0x00000001, 0x807FFFFF, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x3F800000],
    "fp16": [0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0x7D00, 0xFE01, 0x0001, 0x83FF, 0x03FF, 0x0400,
             0x7BFF, 0xFBFF, 0x3C00],
    "bf16": [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7FA0, 0xFFC1, 0x0001, 0x807F, 0x007F, 0x0080,
             0x7F7F, 0xFF7F, 0x3F80],
}
BITS = {"fp32": np.uint32, "fp16": np.uint16, "bf16": np.uint16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def special_inputs(dtype, op, P, L, seed):
    """Normal values with about one element in five replaced by a special."""
    rng = np.random.default_rng(seed)
    xs = []
    for r in range(P):
        x = synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=72, rank=r)
        if op == "prod":
            x = refops.from_f32(dtype, (1.0 + 0.05 * refops.to_f64(dtype, x)).astype(np.float32))
        bits = np.ascontiguousarray(x).view(BITS[dtype]).copy()
        pick = rng.random(L) < 0.2
        bits[pick] = rng.choice(np.array(SPECIALS[dtype], dtype=BITS[dtype]), size=int(pick.sum()))
        xs.append(bits.view(refops.STORAGE[dtype]))
    return xs


@pytest.mark.parametrize("mode", ["steps", "fused", "columns", "lds", "regs", "flow"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("algo,P", [("ring", 5), ("rhd", 5), ("flat", 4)])
def test_specials(algo, P, dtype, mode):
    L = 3 * 1024 + 37
    with hc.Comm(P, algo) as comm:
        comm.set_exec_mode(mode)
        assert comm.exec_choice("allreduce", L, dtype) == mode
        for op in ("sum", "prod", "max", "min"):
            seed = zlib.crc32(f"specials/{algo}/{dtype}/{op}".encode())
            say(f"case specials {mode} algo={algo} P={P} dtype={dtype} op={op} L={L}")
            xs = special_inputs(dtype, op, P, L, seed)
            dev = [to_dev(x, dtype) for x in xs]
            comm.allreduce(dev, dtype, op)
            torch.cuda.synchronize()
            want = [x.copy() for x in xs]
            oracle.run("allreduce", algo, want, dtype, op)
            for r in range(P):
                got = to_host(dev[r], dtype)
                refops.assert_same(dtype, got, want[r], f"specials {mode} {algo} {dtype} {op} rank {r}")
                if op in ("max", "min"):
                    assert np.array_equal(got.view(np.uint8), want[r].view(np.uint8))
