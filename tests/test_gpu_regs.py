"""GPU parity of the register form (HBMC_EXEC_REGS) against the oracle, bit for bit.

The register form evaluates each element's expression, derived on the host
from the schedule, in registers.  Cases span ring (a left fold rotated per
segment), RHD (pairwise trees, with merged pairs when P is not a power of
two) and Flat; all dtypes and ops; lengths whose segment edges cut 16-byte
positions (element-wise lanes), lengths below one vector, and rank buffers
at every 16-byte phase (head and tail elements).
"""
import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
from gpu_util import strided_buffers, to_dev, to_host
from test_gpu_parity import make_inputs, say

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16", "int32", "int8"]
OPS = ["sum", "prod", "max", "min"]


def run_regs(algo, P, L, dtype, op, seed, offsets=None, coll="allreduce", S=0, M=0, root=0):
    xs = make_inputs(dtype, op, P, L, seed)
    if offsets is None:
        dev = [to_dev(x, dtype) for x in xs]
    else:
        dev, _keep = strided_buffers(xs, dtype, offsets)
    with hc.Comm(P, algo, S, M) as c:
        c.set_exec_mode("regs")
        form = c.exec_choice(coll, L, dtype, root=root)
        say(f"case regs {algo} {coll} P={P} L={L} {dtype} {op} offsets={offsets} -> {form}")
        if coll == "broadcast":
            c.broadcast(dev, dtype, root=root)
        elif coll == "reduce":
            c.reduce(dev, dtype, op, root=root)
        else:
            getattr(c, coll)(dev, dtype, op)
        torch.cuda.synchronize()
    want = [x.copy() for x in xs]
    kw = dict(S=S, M=M) if algo == "pipeline" else (dict(M=M) if algo == "tree" else {})
    oracle.run(coll, algo, want, dtype, op, root=root, **kw)
    for r in range(P):
        got = to_host(dev[r], dtype)
        refops.assert_same(dtype, got, want[r], f"regs {algo} P={P} L={L} {dtype} {op} rank {r}")
        if op in ("max", "min") and dtype in refops.FLOATS:
            assert np.array_equal(got.view(np.uint8), want[r].view(np.uint8))
    return form


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("algo,P", [("ring", 8), ("ring", 3), ("ring", 16), ("rhd", 8), ("rhd", 5),
                                    ("rhd", 6), ("rhd", 16), ("flat", 7)])
def test_regs_parity(algo, P, dtype):
    forms = set()
    for i, op in enumerate(OPS):
        for L in (1, 7, 1001, 3 * 4096 + 5, 40_000 + 3):
            forms.add(run_regs(algo, P, L, dtype, op, seed=1000 * i + L))
    assert forms == {"regs"}


@pytest.mark.parametrize("algo,P,coll", [("ring", 8, "allreduce"), ("rhd", 5, "allreduce"),
                                         ("ring", 6, "reduce_scatter"), ("ring", 7, "all_gather"),
                                         ("rhd", 6, "all_gather"), ("rhd", 8, "reduce_scatter")])
def test_regs_phases(algo, P, coll):
    """Rank buffers at one shared 16-byte phase other than 0: the head and
    tail elements go element by element (fold and tree; prefix and copy)."""
    for dtype in ("fp16", "int8", "fp32"):
        e = np.dtype(refops.STORAGE[dtype]).itemsize
        for ph in range(0, 16 // e):
            assert run_regs(algo, P, 2000 + ph, dtype, "sum", seed=ph, offsets=[ph] * P, coll=coll) == "regs"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("algo,P,coll,S,M", [("ring", 8, "reduce_scatter", 0, 0), ("ring", 3, "reduce_scatter", 0, 0),
                                             ("ring", 16, "reduce_scatter", 0, 0), ("ring", 8, "all_gather", 0, 0),
                                             ("ring", 5, "all_gather", 0, 0), ("rhd", 8, "all_gather", 0, 0),
                                             ("rhd", 6, "all_gather", 0, 0), ("rhd", 5, "broadcast", 0, 0),
                                             ("pipeline", 8, "all_gather", 2, 4), ("tree", 5, "allreduce", 0, 2),
                                             ("tree", 3, "allreduce", 0, 2), ("rhd", 17, "allreduce", 0, 0),
                                             ("rhd", 4, "reduce_scatter", 0, 0), ("rhd", 8, "reduce_scatter", 0, 0),
                                             ("rhd", 16, "reduce_scatter", 0, 0), ("rhd", 8, "reduce", 0, 0),
                                             ("rhd", 16, "reduce", 0, 0), ("rhd", 4, "reduce", 0, 0)])
def test_regs_other_collectives(algo, P, coll, S, M, dtype):
    """Copies (all-gather, broadcast), prefixes of one fold (the ring's
    reduce-scatter, whose other segments keep the schedule's partials), nodes
    of one tree (RHD's reduce-scatter and Reduce: every rank keeps its input or
    holds the subtree it last kept) and a small tree AllReduce whose nesting
    is a fold: every rank's whole buffer against the oracle."""
    forms = set()
    for i, op in enumerate(OPS if coll in ("reduce_scatter", "allreduce", "reduce") else ["sum"]):
        for L in (7, 1001, 3 * 4096 + 5, 40_000 + 3):
            forms.add(run_regs(algo, P, L, dtype, op, seed=77 * i + L, coll=coll, S=S, M=M, root=P - 2))
    assert forms == {"regs"}
