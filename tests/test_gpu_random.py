"""Seeded random cases, bit for bit against the oracle.

Each case draws a communicator (ring, RHD, pipeline, Flat, tree,
hierarchical, up to 64 ranks), a collective it supports, a dtype, an op, a
ragged length, a launch form, a column length and the buffers' 16-byte
phases (aligned, one common offset, or offsets that differ by rank), so
combinations that the targeted tests take one at a time meet here: batches
next to element edges, lanes owning several positions, empty segments,
fallbacks from a forced form that a call cannot take.  A forced form the call
is not eligible for falls back to another form; the result must not change.
Every rank's buffer is compared (Reduce: the root's, the only one it
defines).
"""
import sys

import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
from gpu_util import strided_buffers, to_dev, to_host
from test_gpu_parity import make_inputs

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16", "int32", "int8"]
OPS = ["sum", "prod", "max", "min"]
MODES = ["auto", "steps", "fused", "columns", "lds", "regs", "flow"]
CASES_PER_BATCH = 60


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(rng):
    algo = str(rng.choice(["ring", "rhd", "pipeline", "flat", "tree", "hier"]))
    kw = {}
    if algo in ("pipeline", "hier"):
        S, M = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        P = S * M
        loop = int(rng.choice([0, 1024, 4096, 65536]))
        args = (P, algo, S, M, loop)
        kw = dict(S=S, M=M, loop_bytes=loop) if algo == "pipeline" else dict(S=S, M=M)
    elif algo == "tree":
        K = int(rng.integers(2, 5))
        P = int(rng.integers(2, 33))
        args = (P, "tree", 0, K)
        kw = dict(M=K)
    else:
        P = int(rng.integers(2, 65))
        args = (P, algo)
    colls = {"ring": ["allreduce", "reduce_scatter", "all_gather"],
             "rhd": ["allreduce", "reduce_scatter", "all_gather", "reduce", "broadcast"],
             "pipeline": ["allreduce", "reduce_scatter", "all_gather"]}.get(algo, ["allreduce"])
    coll = str(rng.choice(colls))
    size_class = int(rng.integers(0, 3))
    L = int(rng.integers(0, 64)) if size_class == 0 else (
        int(rng.integers(64, 5000)) if size_class == 1 else int(rng.integers(5000, 120_000)))
    return dict(algo=algo, P=P, args=args, kw=kw, coll=coll, dtype=str(rng.choice(DTYPES)),
                op=str(rng.choice(OPS)), L=L, mode=str(rng.choice(MODES)),
                column=int(rng.choice([0, 16, 256, 1024, 8192])),
                phase=str(rng.choice(["aligned", "same", "different"])), root=int(rng.integers(0, P)),
                seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("batch", range(10))
def test_random_cases(batch):
    rng = np.random.default_rng(9000 + batch)
    for i in range(CASES_PER_BATCH):
        c = draw(rng)
        say(f"case batch={batch} i={i} " + " ".join(f"{k}={v}" for k, v in c.items() if k not in ("args", "kw")))
        P, L, dtype, op, coll = c["P"], c["L"], c["dtype"], c["op"], c["coll"]
        xs = make_inputs(dtype, op, P, L, c["seed"])
        esz = np.dtype(refops.STORAGE[dtype]).itemsize
        if c["phase"] == "aligned" or L == 0:
            dev, keep = [to_dev(x, dtype) for x in xs], None
        else:
            step = max(1, 16 // esz)
            offs = [1 % step] * P if c["phase"] == "same" else [r % step for r in range(P)]
            dev, keep = strided_buffers(xs, dtype, offs)
        with hc.Comm(*c["args"]) as comm:
            comm.set_exec_mode(c["mode"])
            comm.set_columns(1 << 40 if c["column"] else 64 << 20, c["column"])
            if coll == "reduce":
                comm.reduce(dev, dtype, op, root=c["root"])
            elif coll == "broadcast":
                comm.broadcast(dev, dtype, root=c["root"])
            else:
                getattr(comm, coll)(dev, dtype, op)
            torch.cuda.synchronize()
        want = [x.copy() for x in xs]
        oracle.run(coll, c["algo"], want, dtype, op, root=c["root"], **c["kw"])
        for r in ([c["root"]] if coll == "reduce" else range(P)):
            refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"batch {batch} case {i} rank {r}")
            if op in ("max", "min") and dtype in refops.FLOATS:
                assert np.array_equal(to_host(dev[r], dtype).view(np.uint8), want[r].view(np.uint8))
        del dev, keep


def test_random_large_cases():
    """Larger seeded cases (1-3 MiB of every rank per segment or block): ring,
    RHD and pipeline AllReduce / reduce-scatter / all-gather, one launch per
    step or AUTO, aligned buffers or one shared 16-byte phase; copy steps of
    items of 1 MiB or more take 4 KiB tiles here.  Whole buffers compared."""
    rng = np.random.default_rng(777)
    for i in range(12):
        algo = str(rng.choice(["ring", "rhd", "pipeline"]))
        if algo == "pipeline":
            S, M = int(rng.integers(2, 5)), int(rng.choice([2, 4]))
            P, args, kw = S * M, (S * M, "pipeline", S, M, 0), dict(S=S, M=M, loop_bytes=0)
        else:
            P = int(rng.integers(2, 17))
            args, kw = (P, algo), {}
        coll = str(rng.choice(["allreduce", "reduce_scatter", "all_gather"]))
        if algo == "rhd" and coll != "allreduce" and P & (P - 1):
            coll = "allreduce"
        dtype = str(rng.choice(DTYPES))
        op = str(rng.choice(["sum", "max", "min"]))
        e = np.dtype(refops.STORAGE[dtype]).itemsize
        L = int(rng.integers(P * (1 << 20) // e // 2, P * (3 << 20) // e)) + int(rng.integers(0, 64))
        mode = str(rng.choice(["auto", "steps"]))
        phase = str(rng.choice(["aligned", "same"]))
        say(f"case large {i}: {algo} P={P} {coll} {dtype} {op} L={L} mode={mode} phase={phase}")
        xs = make_inputs(dtype, op, P, L, 1000 + i)
        if phase == "aligned":
            dev, keep = [to_dev(x, dtype) for x in xs], None
        else:
            dev, keep = strided_buffers(xs, dtype, [1 % max(1, 16 // e)] * P)
        with hc.Comm(*args) as comm:
            comm.set_exec_mode(mode)
            getattr(comm, coll)(dev, dtype, op)
            torch.cuda.synchronize()
        want = [x.copy() for x in xs]
        oracle.run_parallel(coll, algo, want, dtype, op, **kw)
        for r in range(P):
            refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"large case {i} rank {r}")
        del dev, keep
