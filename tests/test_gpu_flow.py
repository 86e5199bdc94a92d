"""GPU parity of the flow form (HBMC_EXEC_FLOW) against the oracle, bit for bit.

The flow kernel runs every step of a call in one launch, tiles handed out in
step order and each tile waiting on its column's counter.  Cases: the
schedules and collectives (ring, RHD with and without a power of two,
pipeline, Flat, tree, hierarchical; AllReduce, reduce-scatter, all-gather,
Reduce, Broadcast), every dtype and op, tiles from 16 bytes (many tiles per
item, ragged tails) to 16 KiB, one or several tiles per ticket, rank buffers
at a shared 16-byte phase other than 0, calls repeated back to back (the counters reset by the kernel itself),
graphs that replay it, a 16-rank ring of 16 MiB per rank compared whole, step
ranges run one launch each, and the give-up path forced from the host.
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
SCHEDS = [  # (comm args, oracle keywords, collectives)
    ((8, "ring"), {}, ["allreduce", "reduce_scatter", "all_gather"]),
    ((3, "ring"), {}, ["allreduce"]),
    ((8, "rhd"), {}, ["allreduce", "reduce_scatter", "all_gather"]),
    ((6, "rhd"), {}, ["allreduce", "reduce", "broadcast"]),
    ((8, "pipeline", 2, 4, 4096), dict(S=2, M=4, loop_bytes=4096), ["allreduce", "reduce_scatter", "all_gather"]),
    ((7, "flat"), {}, ["allreduce"]),
    ((9, "tree", 0, 3), dict(M=3), ["allreduce"]),
    ((6, "hier", 3, 2), dict(S=3, M=2), ["allreduce"]),
]


def _check(got_dev, want, dtype, what):
    for r, w in enumerate(want):
        got = to_host(got_dev[r], dtype)
        refops.assert_same(dtype, got, w, f"{what} rank {r}")
        if dtype in refops.FLOATS:
            assert np.array_equal(got.view(np.uint8), w.view(np.uint8)), f"{what} rank {r}: bits"


def run_flow(args, kw, coll, L, dtype, op, seed, tile, offsets=None, repeat=1, per_ticket=1):
    P = args[0]
    root = 1 % P
    xs = make_inputs(dtype, op, P, L, seed)
    if offsets is None:
        dev = [to_dev(x, dtype) for x in xs]
    else:
        dev, _keep = strided_buffers(xs, dtype, offsets)
    with hc.Comm(*args) as c:
        c.set_exec_mode("flow")
        c.set_flow(tile, tiles_per_ticket=per_ticket)
        form = c.exec_choice(coll, L, dtype, root=root)
        say(f"case flow {args} {coll} L={L} {dtype} {op} tile={tile} per_ticket={per_ticket} offsets={offsets} "
            f"repeat={repeat} -> {form}")
        for _ in range(repeat):
            if coll == "broadcast":
                c.broadcast(dev, dtype, root=root)
            elif coll == "reduce":
                c.reduce(dev, dtype, op, root=root)
            else:
                getattr(c, coll)(dev, dtype, op)
        torch.cuda.synchronize()
        assert c.flow_timeouts() == 0
    want = [x.copy() for x in xs]
    for _ in range(repeat):
        oracle.run(coll, args[1], want, dtype, op, root=root, **kw)
    _check(dev, want, dtype, f"flow {args} {coll} L={L} {dtype} {op} tile={tile}")
    return form


@pytest.mark.parametrize("sched", SCHEDS, ids=[f"{s[0][1]}-P{s[0][0]}" for s in SCHEDS])
@pytest.mark.parametrize("dtype", DTYPES)
def test_flow_parity(sched, dtype):
    args, kw, colls = sched
    forms = set()
    for i, coll in enumerate(colls):
        for j, op in enumerate(OPS if coll not in ("all_gather", "broadcast") else ["sum"]):
            for L, tile, per in ((1001, 16, 1), (3 * 4096 + 5, 1024, 5), (40_000 + 3, 16 << 10, 1),
                                 (40_000 + 3, 256, 16)):
                forms.add(run_flow(args, kw, coll, L, dtype, op, seed=100 * i + 10 * j + L, tile=tile,
                                   per_ticket=per))
    assert forms == {"flow"}


def test_flow_phases_and_repeats():
    """A shared 16-byte phase other than 0 (head and tail elements one by one
    per chunk), and calls back to back whose counters the kernel resets."""
    for dtype in ("fp16", "int8", "fp32"):
        e = np.dtype(refops.STORAGE[dtype]).itemsize
        for ph in range(1, 16 // e, 3):
            assert run_flow((8, "ring"), {}, "allreduce", 5000 + ph, dtype, "sum", seed=ph, tile=64,
                            offsets=[ph] * 8) == "flow"
    assert run_flow((5, "rhd"), {}, "allreduce", 20_001, "int32", "max", seed=3, tile=256, repeat=12) == "flow"
    assert run_flow((8, "ring"), {}, "reduce_scatter", 9_999, "bf16", "sum", seed=4, tile=128, repeat=5) == "flow"


def test_flow_ring_16_ranks_16MiB():
    """The mid-size band the flow form is for: 16 ranks x 16 MiB fp16, whole buffers."""
    P, L, dtype = 16, 8 << 20, "fp16"
    for algo in ("ring", "rhd"):
        for per in (1, 16):
            assert run_flow((P, algo), {}, "allreduce", L, dtype, "sum", seed=16, tile=16 << 10,
                            per_ticket=per) == "flow"


@pytest.mark.parametrize("sched", [SCHEDS[0], SCHEDS[2], SCHEDS[3], SCHEDS[4], SCHEDS[7]],
                         ids=["ring-P8", "rhd-P8", "rhd-P6", "pipeline-P8", "hier-P6"])
def test_flow_step_ranges(sched):
    """hbmc_run_steps ranges in the flow form: the steps cut into three
    ranges, each run as one flow launch (a range of one step takes the step
    kernel), every rank's whole buffer compared with the oracle's replay of
    the same steps after each range; then the same ranges again, repeated."""
    args, kw, colls = sched
    P, dtype, op, L = args[0], "bf16", "sum", 3 * 4096 + 77
    xs = make_inputs(dtype, op, P, L, seed=P + 40)
    dev = [to_dev(x, dtype) for x in xs]
    want = [x.copy() for x in xs]
    with hc.Comm(*args) as c:
        c.set_exec_mode("flow")
        c.set_flow(512)
        n = c.plan_info("allreduce", L, dtype)["nsteps"]
        cuts = sorted({0, 1, n // 2, n})
        for rep in range(2):
            for a, b in zip(cuts, cuts[1:]):
                form = c.exec_choice("allreduce", L, dtype, first=a, last=b)
                say(f"case flow steps [{a}, {b}) of {n} {args} rep {rep} -> {form}")
                assert form == ("flow" if b - a > 1 else "steps")
                c.run_steps("allreduce", dev, a, b, dtype, op)
                torch.cuda.synchronize()
                oracle.run("allreduce", args[1], want, dtype, op, first_step=a, last_step=b, **kw)
                _check(dev, want, dtype, f"flow {args} steps [{a}, {b}) rep {rep}")
        assert c.flow_timeouts() == 0


def test_flow_graph_replays():
    """Two flow AllReduces of one plan on disjoint buffers in a graph (the
    graph orders them, since they share the plan's counters), replayed with
    eager work between replays."""
    P, L, dtype = 8, 30_001, "int32"
    xs = make_inputs(dtype, "max", P, L, 11)
    ys = make_inputs(dtype, "max", P, L, 12)
    a = [to_dev(x, dtype) for x in xs]
    b = [to_dev(y, dtype) for y in ys]
    want_a = [x.copy() for x in xs]
    want_b = [y.copy() for y in ys]
    oracle.run("allreduce", "ring", want_a, dtype, "max")
    oracle.run("allreduce", "ring", want_b, dtype, "max")
    with hc.Comm(P, "ring") as c:
        c.set_exec_mode("flow")
        c.set_flow(512)
        with hc.Graph() as g:
            g.add(c, "allreduce", a, dtype, "max")
            g.add(c, "allreduce", b, dtype, "max")
            g.build()
            for rep in range(4):
                say(f"case flow graph replay {rep}")
                g.launch()
                torch.cuda.synchronize()
                _check(a, want_a, dtype, f"graph a replay {rep}")
                _check(b, want_b, dtype, f"graph b replay {rep}")
                torch.cuda.synchronize()
        assert c.flow_timeouts() == 0


def test_flow_gives_up_when_forced_and_recovers():
    """Every wait made unreachable from the host: each tile with an earlier
    tile gives up after the 50 us bound, the launch ends normally and counts
    timeouts; the next calls, with reachable waits, are exact, also after the
    tile length changed (the counts of the earlier tables are still read)."""
    P, L, dtype = 8, 50_000, "fp32"
    xs = make_inputs(dtype, "sum", P, L, 21)
    want = [x.copy() for x in xs]
    oracle.run("allreduce", "ring", want, dtype, "sum")
    with hc.Comm(P, "ring") as c:
        c.set_exec_mode("flow")
        c.set_flow(1024, wait_us=50, unreachable=True)
        dev = [to_dev(x, dtype) for x in xs]
        say("case flow give-up forced")
        c.allreduce(dev, dtype, "sum")
        torch.cuda.synchronize()
        assert c.flow_timeouts() >= 1
        assert c.flow_timeouts() == 0  # read and cleared
        for tile in (1024, 2048):
            if tile == 2048:  # a give-up under the old length, then a new length
                c.set_flow(1024, wait_us=50, unreachable=True)
                dev = [to_dev(x, dtype) for x in xs]
                c.allreduce(dev, dtype, "sum")
                torch.cuda.synchronize()
            c.set_flow(tile)
            dev = [to_dev(x, dtype) for x in xs]
            say(f"case flow after give-up, tile {tile}")
            c.allreduce(dev, dtype, "sum")
            torch.cuda.synchronize()
            _check(dev, want, dtype, f"flow after give-up, tile {tile}")
            n = c.flow_timeouts()
            assert (n >= 1) if tile == 2048 else (n == 0)
        assert c.flow_timeouts() == 0
