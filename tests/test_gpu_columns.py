"""The column kernels (one launch per call; one wave, or with the columns
resident in LDS one workgroup, runs each column of elements through every
step) against the CPU oracle, bit for bit.

Columns far narrower than the items (down to one 16-byte vector) make every
item span many columns and every column cross item and segment boundaries;
sizes leave ragged tails and empty segments; the buffers share a non-zero
16-byte phase in some cases; the automatic column length is used too.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
from gpu_util import strided_buffers, to_dev, to_host
from test_gpu_parity import OPS, make_inputs

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16", "int32", "int8"]
MODES = ["columns", "lds"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [  # (algo, P, comm args, oracle keywords, collectives)
    ("ring", 5, (5, "ring"), {}, ["allreduce", "reduce_scatter", "all_gather"]),
    ("ring", 8, (8, "ring"), {}, ["allreduce"]),
    ("rhd", 8, (8, "rhd"), {}, ["allreduce", "reduce_scatter", "all_gather", "reduce", "broadcast"]),
    ("rhd", 7, (7, "rhd"), {}, ["allreduce", "reduce_scatter", "all_gather", "reduce", "broadcast"]),
    ("pipeline", 8, (8, "pipeline", 2, 4, 4096), dict(S=2, M=4, loop_bytes=4096),
     ["allreduce", "reduce_scatter", "all_gather"]),
    ("flat", 6, (6, "flat"), {}, ["allreduce"]),
    ("tree", 11, (11, "tree", 0, 3), dict(M=3), ["allreduce"]),
    ("hier", 6, (6, "hier", 3, 2), dict(S=3, M=2), ["allreduce"]),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}{c[1]}" for c in CASES])
def test_columns_parity(case, dtype, mode):
    algo, P, args, kw, colls = case
    rng = np.random.default_rng(zlib.crc32(f"columns/{algo}/{P}/{dtype}".encode()))
    with hc.Comm(*args) as comm:
        comm.set_exec_mode(mode)
        for coll in colls:
            op = str(rng.choice(OPS))
            L = int(rng.choice([7, 1000, 3 * 4096 + 5, 40_003]))
            chunk = int(rng.choice([0, 16, 48, 1024, 4096]))
            comm.set_columns(1 << 40, chunk)
            root = int(rng.integers(0, P))
            say(f"case {mode} algo={algo} P={P} coll={coll} dtype={dtype} op={op} L={L} chunk={chunk} root={root}")
            assert comm.exec_choice(coll, L, dtype, root=root) == mode
            xs = make_inputs(dtype, op, P, L, seed=L + P)
            if rng.random() < 0.5:
                dev = [to_dev(x, dtype) for x in xs]
            else:
                ph = int(rng.integers(1, 4))
                dev, _keep = strided_buffers(xs, dtype, [ph] * P)
            if coll == "reduce":
                comm.reduce(dev, dtype, op, root=root)
            elif coll == "broadcast":
                comm.broadcast(dev, dtype, root=root)
            else:
                getattr(comm, coll)(dev, dtype, op)
            torch.cuda.synchronize()
            want = [x.copy() for x in xs]
            oracle.run(coll, algo, want, dtype, op, root=root, **kw)
            for r in ([root] if coll == "reduce" else range(P)):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"{mode} {algo} {coll} rank {r}")


@pytest.mark.parametrize("mode", MODES)
def test_columns_step_ranges_and_repeats(mode):
    """Sub-ranges of steps, repeated launches of one plan, column lengths
    changed between calls and per-step calls interleaved on one communicator."""
    P, L, dtype = 6, 30_001, "int32"
    xs = make_inputs(dtype, "sum", P, L, seed=9)
    with hc.Comm(P, "ring") as comm:
        comm.set_columns(1 << 40, 512)
        comm.set_exec_mode(mode)
        n = comm.plan_info("allreduce", L, dtype)["nsteps"]
        dev = [to_dev(x, dtype) for x in xs]
        want = [x.copy() for x in xs]
        for a, b in ((0, 1), (1, 4), (4, n)):
            say(f"case {mode} steps [{a},{b})")
            comm.run_steps("allreduce", dev, a, b, dtype, "sum")
            oracle.run("allreduce", "ring", want, dtype, "sum", first_step=a, last_step=b)
            torch.cuda.synchronize()
            for r in range(P):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"steps [{a},{b}) rank {r}")
        for rep in range(6):
            say(f"case {mode} repeat {rep}")
            if rep % 2:
                comm.set_columns(0)
            else:
                comm.set_columns(1 << 40, 512 if rep < 4 else 2048)
            comm.allreduce(dev, dtype, "sum")
            oracle.run("allreduce", "ring", want, dtype, "sum")
            torch.cuda.synchronize()
            for r in range(P):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"repeat {rep} rank {r}")


@pytest.mark.parametrize("mode", MODES)
def test_columns_out_of_place_and_graph(mode):
    P, L, dtype = 5, 9999, "bf16"
    xs = make_inputs(dtype, "max", P, L, seed=4)
    with hc.Comm(P, "rhd") as comm:
        comm.set_columns(1 << 40, 1024)
        comm.set_exec_mode(mode)
        send = [to_dev(x, dtype) for x in xs]
        recv = [torch.empty_like(t) for t in send]
        comm.out_of_place("allreduce", send, recv, dtype, "max")
        torch.cuda.synchronize()
        want = [x.copy() for x in xs]
        oracle.run("allreduce", "rhd", want, dtype, "max")
        for r in range(P):
            refops.assert_same(dtype, to_host(recv[r], dtype), want[r], f"oop rank {r}")
            refops.assert_same(dtype, to_host(send[r], dtype), xs[r], f"send untouched rank {r}")
        # graph node of the same call, replayed with eager work between replays
        gb = [to_dev(x, dtype) for x in xs]
        with hc.Graph() as g:
            g.add(comm, "allreduce", gb, dtype, "max")
            g.build()
            for rep in range(3):
                for t, x in zip(gb, xs):
                    t.copy_(to_dev(x, dtype))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                for r in range(P):
                    refops.assert_same(dtype, to_host(gb[r], dtype), want[r], f"graph replay {rep} rank {r}")


@pytest.mark.parametrize("mode", MODES + ["auto"])
@pytest.mark.parametrize("algo", ["ring", "rhd", "flat"])
def test_max_ranks(algo, mode):
    """64 ranks, the most a communicator takes: chunk records whose rank lists
    run past 16 entries (Flat folds 64 sources into one destination and
    copies one source to 63), empty segments (L < P) and ragged tails."""
    P = 64
    with hc.Comm(P, algo) as comm:
        comm.set_exec_mode(mode)
        for L, dtype, op in ((40, "int32", "sum"), (1000, "bf16", "max"), (6000 + 5, "fp16", "sum")):
            say(f"case {mode} max ranks algo={algo} L={L} dtype={dtype} op={op} "
                f"form={comm.exec_choice('allreduce', L, dtype)}")
            xs = make_inputs(dtype, op, P, L, seed=L)
            dev = [to_dev(x, dtype) for x in xs]
            comm.allreduce(dev, dtype, op)
            torch.cuda.synchronize()
            want = [x.copy() for x in xs]
            oracle.run("allreduce", algo, want, dtype, op)
            for r in range(P):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"{mode} {algo} P=64 rank {r}")


@pytest.mark.parametrize("algo,P,dtype,L", [("ring", 8, "fp32", 8 << 20), ("rhd", 5, "bf16", 32 << 20)])
def test_lds_past_the_default_limit(algo, P, dtype, L):
    """With the column limit raised, the LDS form runs calls of 256-320 MiB in
    all (hundreds of thousands of columns); its result equals one launch per
    step bit for bit (that form is pinned to the oracle at full size)."""
    xs = make_inputs(dtype, "sum", P, L, seed=5)
    with hc.Comm(P, algo) as comm:
        comm.set_columns(1 << 40, 0)
        comm.set_exec_mode("lds")
        say(f"case lds large algo={algo} P={P} dtype={dtype} L={L} form={comm.exec_choice('allreduce', L, dtype)}")
        assert comm.exec_choice("allreduce", L, dtype) == "lds"
        a = [to_dev(x, dtype) for x in xs]
        comm.allreduce(a, dtype, "sum")
        comm.set_exec_mode("steps")
        b = [to_dev(x, dtype) for x in xs]
        comm.allreduce(b, dtype, "sum")
        torch.cuda.synchronize()
        for r in range(P):
            assert torch.equal(a[r].view(torch.int16 if dtype == "bf16" else torch.int32),
                               b[r].view(torch.int16 if dtype == "bf16" else torch.int32)), f"rank {r}"


COMPOSED = [  # trailing copy steps: ring 15, RHD 16 ranks 4, 17 ranks 5 (with the restore), pipeline 5
    ("ring", 16, (16, "ring"), {}),
    ("rhd", 16, (16, "rhd"), {}),
    ("rhd", 17, (17, "rhd"), {}),
    ("pipeline", 20, (20, "pipeline", 5, 4, 4096), dict(S=5, M=4, loop_bytes=4096)),
]


@pytest.mark.parametrize("case", COMPOSED, ids=[f"{c[0]}{c[1]}" for c in COMPOSED])
def test_lds_composed_stores(case):
    """LDS form, whole calls: columns whose chunk lists end in copies over three
    or more steps store the copies' results directly instead of running them.
    Columns inside one segment, across two and across many (which keep their
    copies), ragged lengths, buffers on a shared non-zero 16-byte phase;
    AllReduce, stand-alone AllGather and ReduceScatter."""
    algo, P, args, kw = case
    dtypes = ["fp32", "bf16", "int8", "fp16"]
    with hc.Comm(*args) as comm:
        comm.set_exec_mode("lds")
        i = 0
        for coll in ("allreduce", "all_gather", "reduce_scatter"):
            for chunk in (16, 48, 1024):
                for L in (16 * 97 + 5, 40_003):
                    for ph in (0, 1):
                        dtype, op = dtypes[i % len(dtypes)], OPS[i % len(OPS)]
                        i += 1
                        comm.set_columns(1 << 40, chunk)
                        say(f"case composed algo={algo} P={P} coll={coll} chunk={chunk} L={L} phase={ph} "
                            f"dtype={dtype} op={op}")
                        assert comm.exec_choice(coll, L, dtype) == "lds"
                        xs = make_inputs(dtype, op, P, L, seed=L + chunk + ph)
                        if ph:
                            esz = np.dtype(refops.STORAGE[dtype]).itemsize
                            dev, _keep = strided_buffers(xs, dtype, [max(1, 4 // esz)] * P)
                        else:
                            dev = [to_dev(x, dtype) for x in xs]
                        getattr(comm, coll)(dev, dtype, op)
                        torch.cuda.synchronize()
                        want = [x.copy() for x in xs]
                        oracle.run(coll, algo, want, dtype, op, **kw)
                        for r in range(P):
                            refops.assert_same(dtype, to_host(dev[r], dtype), want[r],
                                               f"composed {algo} {coll} chunk={chunk} L={L} rank {r}")
