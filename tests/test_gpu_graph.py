"""Graph mode on the GPU: each replay equals the eager calls bit for bit.

A graph is built once and replayed several times; between replays the test
does its own eager work (restoring the inputs) and synchronises, and every
replay is compared with the eager result of the same sequence.
"""
import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import refops
import synth
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def inputs(P, L, dtype="bf16", seed=0):
    return [synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=80, rank=r) for r in range(P)]


def eager(seq, dtype):
    """seq: list of (comm, coll, bufs) run eagerly; returns host copies of all buffers."""
    for comm, coll, bufs in seq:
        getattr(comm, coll)(bufs, dtype, "sum")
    torch.cuda.synchronize()


@pytest.mark.parametrize("algo,P", [("ring", 8), ("rhd", 5), ("rhd", 8)])
def test_graph_single_allreduce_replays(algo, P):
    L, dtype = 3 * 4096 + 5, "bf16"
    xs = inputs(P, L, dtype)
    with hc.Comm(P, algo) as comm:
        ref = [to_dev(x, dtype) for x in xs]
        eager([(comm, "allreduce", ref)], dtype)
        want = [to_host(t, dtype) for t in ref]
        bufs = [to_dev(x, dtype) for x in xs]
        with hc.Graph() as g:
            g.add(comm, "allreduce", bufs, dtype, "sum")
            g.build()
            for rep in range(4):
                for b, x in zip(bufs, xs):  # eager work between replays
                    b.copy_(to_dev(x, dtype))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                for r in range(P):
                    refops.assert_same(dtype, to_host(bufs[r], dtype), want[r], f"replay {rep} rank {r}")


def test_graph_pipeline_many_items():
    """A 4 x 8 pipeline with 8 KiB loops, one launch per step: over 1000 items per
    step, so the fold and fan-out launches reserve LDS to cap the workgroups a
    compute unit holds; as graph nodes they replay bit for bit like the eager
    calls, which match the oracle."""
    import oracle
    S, M, loop = 4, 8, 8192
    P, L, dtype = S * M, 128 * 1024 + 5, "bf16"
    xs = inputs(P, L, dtype, seed=7)
    with hc.Comm(P, "pipeline", S, M, loop) as comm:
        comm.set_exec_mode("steps")
        assert comm.step_info("allreduce", L, dtype, 0)["nitems"] >= 64
        ref = [to_dev(x, dtype) for x in xs]
        eager([(comm, "allreduce", ref)], dtype)
        want = [to_host(t, dtype) for t in ref]
        expect = [x.copy() for x in xs]
        oracle.run("allreduce", "pipeline", expect, dtype, "sum", S=S, M=M, loop_bytes=loop)
        for r in range(P):
            refops.assert_same(dtype, want[r], expect[r], f"eager rank {r}")
        bufs = [to_dev(x, dtype) for x in xs]
        with hc.Graph() as g:
            g.add(comm, "allreduce", bufs, dtype, "sum")
            g.build()
            for rep in range(3):
                for b, x in zip(bufs, xs):
                    b.copy_(to_dev(x, dtype))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                for r in range(P):
                    refops.assert_same(dtype, to_host(bufs[r], dtype), want[r], f"replay {rep} rank {r}")


def test_graph_independent_and_dependent_nodes():
    """Two AllReduces on disjoint buffer sets (may overlap in time), then a
    reduce-scatter + all-gather on the first set (depends on the first node)."""
    P, L, dtype = 8, 50_001, "bf16"
    xa, xb = inputs(P, L, dtype, seed=1), inputs(P, L, dtype, seed=2)
    with hc.Comm(P, "ring") as ring, hc.Comm(P, "rhd") as rhd:
        ra = [to_dev(x, dtype) for x in xa]
        rb = [to_dev(x, dtype) for x in xb]
        eager([(ring, "allreduce", ra), (rhd, "allreduce", rb), (ring, "reduce_scatter", ra),
               (ring, "all_gather", ra)], dtype)
        want_a = [to_host(t, dtype) for t in ra]
        want_b = [to_host(t, dtype) for t in rb]
        ga = [to_dev(x, dtype) for x in xa]
        gb = [to_dev(x, dtype) for x in xb]
        with hc.Graph() as g:
            g.add(ring, "allreduce", ga, dtype, "sum")
            g.add(rhd, "allreduce", gb, dtype, "sum")
            g.add(ring, "reduce_scatter", ga, dtype, "sum")
            g.add(ring, "all_gather", ga, dtype, "sum")
            g.build()
            for rep in range(3):
                for b, x in zip(ga, xa):
                    b.copy_(to_dev(x, dtype))
                for b, x in zip(gb, xb):
                    b.copy_(to_dev(x, dtype))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                for r in range(P):
                    refops.assert_same(dtype, to_host(ga[r], dtype), want_a[r], f"replay {rep} set a rank {r}")
                    refops.assert_same(dtype, to_host(gb[r], dtype), want_b[r], f"replay {rep} set b rank {r}")


def test_graph_on_a_side_stream():
    P, L, dtype = 4, 10_000, "fp32"
    xs = [synth.generate(dtype, L, synth.NORMAL, 1.0, stream=81, rank=r) for r in range(P)]
    with hc.Comm(P, "ring") as comm:
        ref = [to_dev(x, dtype) for x in xs]
        eager([(comm, "allreduce", ref)], dtype)
        want = [to_host(t, dtype) for t in ref]
        bufs = [to_dev(x, dtype) for x in xs]
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        with hc.Graph() as g:
            g.add(comm, "allreduce", bufs, dtype, "sum")
            g.build()
            g.launch(stream=s)
            s.synchronize()
        for r in range(P):
            assert np.array_equal(to_host(bufs[r], dtype).view(np.uint32), want[r].view(np.uint32))


@pytest.mark.parametrize("form", ["lds", "columns"])
def test_graph_survives_a_column_length_change(form):
    """A graph built in a one-launch form keeps the device tables of its column
    length: after the communicator's column length changes and an eager call
    builds the tables of the new length, replays of the old graph still match
    the oracle bit for bit, and so do eager calls at the new length."""
    import oracle
    P, L, dtype = 8, 40_000 + 3, "bf16"
    xs = inputs(P, L, dtype, seed=11)
    expect = [x.copy() for x in xs]
    oracle.run("allreduce", "ring", expect, dtype, "sum")
    with hc.Comm(P, "ring") as comm:
        comm.set_exec_mode(form)
        comm.set_columns(64 << 20, 4096)
        assert comm.exec_choice("allreduce", L, dtype) == form
        bufs = [to_dev(x, dtype) for x in xs]
        with hc.Graph() as g:
            g.add(comm, "allreduce", bufs, dtype, "sum")
            g.build()
            g.launch()
            torch.cuda.synchronize()
            for r in range(P):
                refops.assert_same(dtype, to_host(bufs[r], dtype), expect[r], f"first replay rank {r}")
            # a new column length: the next eager call builds new tables
            comm.set_columns(64 << 20, 1024)
            other = [to_dev(x, dtype) for x in xs]
            comm.allreduce(other, dtype, "sum")
            torch.cuda.synchronize()
            for r in range(P):
                refops.assert_same(dtype, to_host(other[r], dtype), expect[r], f"new length rank {r}")
            for rep in range(3):
                for b, x in zip(bufs, xs):
                    b.copy_(to_dev(x, dtype))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                for r in range(P):
                    refops.assert_same(dtype, to_host(bufs[r], dtype), expect[r], f"replay {rep} rank {r}")
