"""GPU parity: the C-ABI library on gfx950 against the CPU oracle, bit for bit.

Every case uploads seeded inputs, runs one collective through the C ABI, and
compares every rank's buffer with the oracle's replay of the same schedule
(NaNs of sum / prod compared as a class; max / min NaNs bit-exactly).
Sizes span several 4096-element tiles with ragged tails, segments shorter
than one vector, empty segments (L < P) and L = 0.
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
from gpu_util import strided_buffers, to_dev, to_host

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16", "int32", "int8"]
OPS = ["sum", "prod", "max", "min"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_inputs(dtype, op, P, L, seed):
    if dtype in ("int32", "int8"):
        lo, hi = (-(2 ** 20), 2 ** 20) if dtype == "int32" else (-128, 127)
        if op == "prod":
            lo, hi = -3, 3
        return [synth.generate(dtype, L, synth.UNIFORM_INT, lo, hi, seed=seed, stream=70, rank=r)
                for r in range(P)]
    xs = [synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=71, rank=r) for r in range(P)]
    if op == "prod":
        xs = [refops.from_f32(dtype, (1.0 + 0.05 * refops.to_f64(dtype, x)).astype(np.float32)) for x in xs]
    return xs


def comm_for(algo, P, loop_bytes=0):
    if algo == "pipeline":
        # prefer two or more servers with several ranks each
        shapes = [(P // M, M) for M in (8, 4, 3, 2) if P % M == 0]
        S, M = next((sm for sm in shapes if sm[0] >= 2), shapes[0] if shapes else (P, 1))
        return hc.Comm(P, "pipeline", S, M, loop_bytes), S, M
    return hc.Comm(P, algo), 1, 1


def check_case(algo, coll, dtype, op, P, L, seed, loop_bytes=0, exec_mode="auto"):
    say(f"case algo={algo} coll={coll} dtype={dtype} op={op} P={P} L={L} seed={seed} exec={exec_mode}")
    comm, S, M = comm_for(algo, P, loop_bytes)
    with comm:
        comm.set_exec_mode(exec_mode)
        xs = make_inputs(dtype, op, P, L, seed)
        dev = [to_dev(x, dtype) for x in xs]
        getattr(comm, coll)(dev, dtype, op)
        torch.cuda.synchronize()
        want = [x.copy() for x in xs]
        oracle.run(coll, algo, want, dtype, op, S=S, M=M, loop_bytes=loop_bytes)
        for r in range(P):
            got = to_host(dev[r], dtype)
            refops.assert_same(dtype, got, want[r], f"{algo} {coll} {dtype} {op} P={P} L={L} rank {r}")
            if op in ("max", "min") and dtype in refops.FLOATS:
                assert np.array_equal(got.view(np.uint8), want[r].view(np.uint8))


LS = [0, 1, 5, 1000, 3 * 4096 + 7, 50_001]


@pytest.mark.parametrize("exec_mode", ["steps", "auto"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather"])
@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
def test_parity(algo, coll, dtype, exec_mode):
    """Every case once with one launch per step and once with the launch form
    the communicator picks by default (single workgroup, column kernel or
    steps, by size)."""
    rng = np.random.default_rng(zlib.crc32(f"{algo}/{coll}/{dtype}".encode()))
    Ps = [2, 3, 5, 8] if not (algo == "rhd" and coll != "allreduce") else [2, 4, 5, 6, 8]
    for op in OPS:
        for P in Ps:
            L = int(rng.choice(LS))
            check_case(algo, coll, dtype, op, P, L, seed=int(rng.integers(1 << 30)),
                       loop_bytes=(8192 if algo == "pipeline" else 0), exec_mode=exec_mode)


VARIANT_COMMS = [("flat", P, (P, "flat"), {}) for P in (2, 5, 8, 16)] + \
    [("tree", P, (P, "tree", 0, K), dict(M=K)) for P, K in ((7, 2), (13, 3), (16, 4), (32, 2))] + \
    [("hier", S * M, (S * M, "hier", S, M), dict(S=S, M=M)) for S, M in ((2, 4), (4, 8), (3, 2), (4, 1))]


@pytest.mark.parametrize("dtype", DTYPES)
def test_parity_variants(dtype):
    """Flat, tree and hierarchical AllReduce against the oracle, every op."""
    rng = np.random.default_rng(zlib.crc32(dtype.encode()))
    for algo, P, args, kw in VARIANT_COMMS:
        with hc.Comm(*args) as comm:
            for op in OPS:
                L = int(rng.choice(LS))
                say(f"case variant algo={algo} {kw} dtype={dtype} op={op} P={P} L={L}")
                xs = make_inputs(dtype, op, P, L, seed=L + P)
                dev = [to_dev(x, dtype) for x in xs]
                comm.allreduce(dev, dtype, op)
                torch.cuda.synchronize()
                want = [x.copy() for x in xs]
                oracle.run("allreduce", algo, want, dtype, op, **kw)
                for r in range(P):
                    refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"{algo} {kw} rank {r}")


@pytest.mark.parametrize("P,S,M", [(8, 0, 0), (6, 0, 0), (8, 2, 4)])
def test_parity_auto(P, S, M):
    """An AUTO communicator runs the schedule it reports, bit for bit."""
    dtype = "bf16"
    with hc.Comm(P, "auto", S, M) as comm:
        for coll in ("allreduce", "reduce_scatter", "all_gather", "reduce", "broadcast"):
            for L in (100, 3 * 4096 + 1, 200_003):
                algo = comm.auto_choice(coll, L, dtype, root=1)
                say(f"case auto P={P} coll={coll} L={L} -> {algo}")
                xs = make_inputs(dtype, "sum", P, L, seed=L)
                dev = [to_dev(x, dtype) for x in xs]
                if coll in ("reduce", "broadcast"):
                    getattr(comm, coll)(dev, dtype, **({"op": "sum"} if coll == "reduce" else {}), root=1)
                else:
                    getattr(comm, coll)(dev, dtype, "sum")
                torch.cuda.synchronize()
                want = [x.copy() for x in xs]
                kw = dict(S=S, M=M) if algo in ("pipeline", "hier") else (dict(M=2) if algo == "tree" else {})
                oracle.run(coll, algo, want, dtype, "sum", root=1, **kw)
                ranks = [1] if coll == "reduce" else range(P)
                for r in ranks:
                    if coll == "reduce_scatter":
                        b, e = refops.seg_bounds(L, P, r) if algo != "pipeline" else (0, 0)
                        refops.assert_same(dtype, to_host(dev[r], dtype)[b:e], want[r][b:e], f"{coll} rank {r}")
                    else:
                        refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"{coll} {algo} rank {r}")


@pytest.mark.parametrize("P", [4, 5, 8, 6])
def test_parity_auto_rules(P):
    """An AUTO_RULES communicator (the pages' defaults: Flat below 64 KiB per
    rank for AllReduce, RHD for a power-of-two rank count, the ring otherwise)
    runs the schedule its rules pick, bit for bit, on both sides of 64 KiB."""
    pow2 = (P & (P - 1)) == 0
    for dtype, op in (("fp16", "sum"), ("int32", "max")):
        e = 2 if dtype == "fp16" else 4
        with hc.Comm(P, "auto_rules") as comm:
            for coll in ("allreduce", "reduce_scatter", "all_gather"):
                for L in ((64 << 10) // e - 1, (64 << 10) // e, 100_003):
                    algo = comm.auto_choice(coll, L, dtype)
                    expect = "flat" if coll == "allreduce" and L * e < (64 << 10) else ("rhd" if pow2 else "ring")
                    assert algo == expect, (coll, L, algo)
                    say(f"case auto_rules P={P} {coll} {dtype} {op} L={L} -> {algo}")
                    xs = make_inputs(dtype, op, P, L, seed=L + P)
                    dev = [to_dev(x, dtype) for x in xs]
                    getattr(comm, coll)(dev, dtype, op)
                    torch.cuda.synchronize()
                    want = [x.copy() for x in xs]
                    oracle.run(coll, algo, want, dtype, op)
                    for r in range(P):
                        got = to_host(dev[r], dtype)
                        if coll == "reduce_scatter":
                            b, e2 = refops.seg_bounds(L, P, r)
                            refops.assert_same(dtype, got[b:e2], want[r][b:e2], f"rules {coll} rank {r}")
                        else:
                            refops.assert_same(dtype, got, want[r], f"rules {coll} {algo} rank {r}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("coll", ["reduce", "broadcast"])
def test_parity_rooted(coll, dtype):
    """RHD Reduce / Broadcast from every root (the root's buffer for Reduce,
    every buffer for Broadcast, bit for bit against the oracle)."""
    for P in (2, 3, 5, 6, 8, 13):
        L = 4096 * 2 + 37 * P
        with hc.Comm(P, "rhd") as comm:
            for root in range(P):
                op = "max" if dtype in ("int8",) else "sum"
                say(f"case rooted coll={coll} dtype={dtype} op={op} P={P} root={root} L={L}")
                xs = make_inputs(dtype, op, P, L, seed=root)
                dev = [to_dev(x, dtype) for x in xs]
                if coll == "reduce":
                    comm.reduce(dev, dtype, op, root=root)
                else:
                    comm.broadcast(dev, dtype, root=root)
                torch.cuda.synchronize()
                want = [x.copy() for x in xs]
                oracle.run(coll, "rhd", want, dtype, op, root=root)
                for r in ([root] if coll == "reduce" else range(P)):
                    refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"{coll} P={P} root={root} r={r}")


@pytest.mark.parametrize("exec_mode", ["steps", "auto"])
@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline", "flat"])
def test_parity_many_ranks(algo, exec_mode):
    """Up to 64 ranks: item rank lists that run past the first 32-bit word of
    rank numbers (the pipeline's 9 sources, Flat's 64 sources and 63
    destinations), through one launch per step and through AUTO's form."""
    for P in (13, 16, 32, 64):
        if algo == "pipeline" and P == 13:
            continue
        for dtype, op in (("fp32", "sum"), ("bf16", "sum"), ("int8", "max")):
            check_case(algo, "allreduce", dtype, op, P, 20_000 + P, seed=P, loop_bytes=16384,
                       exec_mode=exec_mode)


def test_parity_items_past_grid_y():
    """A step of more than 65536 items (the pipeline with 1 KiB loops): the
    step kernels take the item from grid.y, past the device's reported
    maxGridSize[1] of 65536, which the runtime launches in full."""
    P, L = 32, (1 << 20) + 3
    with hc.Comm(P, "pipeline", 4, 8, 1024) as comm:
        assert comm.step_info("allreduce", L, "bf16", 0)["nitems"] > 65536
    check_case("pipeline", "allreduce", "bf16", "sum", P, L, seed=11, loop_bytes=1024, exec_mode="steps")


@pytest.mark.parametrize("dtype", DTYPES)
def test_parity_wide_copy_tiles(dtype):
    """Copy steps whose items reach 1 MiB and that write at most 32 MiB move
    4 KiB tiles: ring and RHD AllReduce and all-gather with items just below,
    at and above 1 MiB, ragged item ends, and all rank buffers at a shared
    nonzero 16-byte phase (head and tail elements beside the wide body)."""
    e = np.dtype(refops.STORAGE[dtype]).itemsize
    for algo, P in (("ring", 4), ("rhd", 8)):
        for L in ((P << 20) // e - 64, (P << 20) // e, (P << 20) // e + 7, (3 * P << 20) // e + 33):
            for coll in ("allreduce", "all_gather"):
                check_case(algo, coll, dtype, "max", P, L, seed=L % 97, exec_mode="steps")
    P, L = 4, (4 << 20) // e + 5
    offs = [max(1, 16 // e - 1)] * P if e < 16 else [0] * P
    say(f"case wide copy tiles, shared phase {offs[0] * e} bytes, dtype={dtype} P={P} L={L}")
    xs = make_inputs(dtype, "sum", P, L, seed=29)
    views, backing = strided_buffers(xs, dtype, offs)
    with hc.Comm(P, "ring") as comm:
        comm.set_exec_mode("steps")
        comm.allreduce(views, dtype, "sum")
        torch.cuda.synchronize()
    want = [x.copy() for x in xs]
    oracle.run("allreduce", "ring", want, dtype, "sum")
    for r in range(P):
        refops.assert_same(dtype, to_host(views[r], dtype), want[r], f"rank {r}")
    mask = torch.ones_like(backing, dtype=torch.bool)
    for v in views:
        off = (v.data_ptr() - backing.data_ptr()) // e
        mask[off:off + L] = False
    assert int((backing[mask] != 0).sum()) == 0


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
def test_parity_small_and_empty_segments(algo):
    for P in (3, 5, 8, 16):
        for L in range(0, P + 3):
            check_case(algo, "allreduce", "fp16", "sum", P, L, seed=L)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("phases", ["same_nonzero", "different"])
def test_unaligned_buffers(dtype, phases):
    """Buffers at odd element offsets: a shared 16-byte phase takes the vector
    kernel with head/tail elements, differing phases the element-wise kernel."""
    esz = np.dtype(refops.STORAGE[dtype]).itemsize
    for algo in ("ring", "rhd"):
        P, L = 5, 3 * 4096 + 11
        say(f"case unaligned {phases} algo={algo} dtype={dtype} P={P} L={L}")
        xs = make_inputs(dtype, "sum", P, L, seed=3)
        if phases == "same_nonzero":
            offs = [max(1, 4 // esz) if esz < 16 else 0] * P
        else:
            offs = [r % max(2, 16 // esz) for r in range(P)]
        views, backing = strided_buffers(xs, dtype, offs)
        with hc.Comm(P, algo) as comm:
            comm.allreduce(views, dtype, "sum")
            torch.cuda.synchronize()
        want = [x.copy() for x in xs]
        oracle.run("allreduce", algo, want, dtype, "sum")
        for r in range(P):
            refops.assert_same(dtype, to_host(views[r], dtype), want[r], f"rank {r}")
        # nothing outside the rank ranges was written
        mask = torch.ones_like(backing, dtype=torch.bool)
        for v in views:
            off = (v.data_ptr() - backing.data_ptr()) // esz
            mask[off:off + L] = False
        assert int((backing[mask] != 0).sum()) == 0


@pytest.mark.parametrize("phase", ["aligned", "same_nonzero"])
def test_step_item_sources(phase):
    """One launch per step, around the size limit of the kernel-argument item
    form (steps of at most 16 items; larger ones read the device item table):
    ring with 15, 16 and 17 ranks, RHD with 16 and 17, Flat's single 8-source
    fold and the 2 x 2 pipeline, over buffers on one 16-byte phase, zero or
    not (head and tail elements then come before and after the vectors)."""
    cases = [("ring", 15), ("ring", 16), ("ring", 17), ("rhd", 16), ("rhd", 17), ("flat", 8), ("pipeline", 4)]
    for algo, P in cases:
        for dtype, op in (("fp32", "sum"), ("fp16", "max"), ("bf16", "prod"), ("int8", "sum")):
            esz = np.dtype(refops.STORAGE[dtype]).itemsize
            L = 16 * 1024 + 3 * P + 5
            say(f"case item sources {phase} algo={algo} P={P} dtype={dtype} op={op} L={L}")
            xs = make_inputs(dtype, op, P, L, seed=P)
            offs = [0 if phase == "aligned" else max(1, 4 // esz)] * P
            views, backing = strided_buffers(xs, dtype, offs)
            comm, S, M = comm_for(algo, P)
            with comm:
                comm.set_exec_mode("steps")
                comm.allreduce(views, dtype, op)
                torch.cuda.synchronize()
            want = [x.copy() for x in xs]
            oracle.run("allreduce", algo, want, dtype, op, S=S, M=M)
            for r in range(P):
                refops.assert_same(dtype, to_host(views[r], dtype), want[r], f"{algo} P={P} {dtype} {op} rank {r}")
            mask = torch.ones_like(backing, dtype=torch.bool)
            for v in views:
                off = (v.data_ptr() - backing.data_ptr()) // esz
                mask[off:off + L] = False
            assert int((backing[mask] != 0).sum()) == 0


@pytest.mark.parametrize("algo,coll,P", [("ring", "allreduce", 8), ("rhd", "allreduce", 5),
                                         ("rhd", "allreduce", 8), ("rhd", "reduce_scatter", 8),
                                         ("rhd", "reduce_scatter", 6), ("rhd", "all_gather", 7),
                                         ("pipeline", "allreduce", 8), ("ring", "all_gather", 6)])
def test_step_by_step(algo, coll, P):
    """Every rank's whole buffer after every step equals the oracle's replay state."""
    dtype, L = "bf16", 4 * 4096 + 13
    comm, S, M = comm_for(algo, P, loop_bytes=4096)
    with comm:
        xs = make_inputs(dtype, "sum", P, L, seed=11)
        dev = [to_dev(x, dtype) for x in xs]
        nsteps = comm.plan_info(coll, L, dtype)["nsteps"]
        assert nsteps == oracle.num_steps(coll, algo, P, S, M)
        want = [x.copy() for x in xs]
        for s in range(nsteps):
            say(f"case step-by-step algo={algo} coll={coll} P={P} step={s}")
            comm.run_steps(coll, dev, s, s + 1, dtype, "sum")
            torch.cuda.synchronize()
            oracle.run(coll, algo, want, dtype, "sum", S=S, M=M, loop_bytes=4096, first_step=s,
                       last_step=s + 1)
            for r in range(P):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"after step {s}, rank {r}")


def test_single_rank_and_zero_count_leave_buffers_alone():
    x = synth.generate("fp32", 1000, synth.NORMAL, 1.0, seed=1)
    t = to_dev(x, "fp32")
    with hc.Comm(1, "ring") as c:
        c.allreduce([t], "fp32", "sum")
    with hc.Comm(4, "ring") as c:
        bufs = [to_dev(x, "fp32") for _ in range(4)]
        c.allreduce(bufs, "fp32", "sum", count=0)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(t, "fp32"), x)
    assert all(np.array_equal(to_host(b, "fp32"), x) for b in bufs)


def test_non_default_stream():
    P, L = 8, 100_000
    xs = make_inputs("fp32", "sum", P, L, seed=5)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dev = [to_dev(x, "fp32") for x in xs]
        with hc.Comm(P, "ring") as c:
            c.allreduce(dev, "fp32", "sum")
            s.synchronize()
    want = [x.copy() for x in xs]
    oracle.run("allreduce", "ring", want, "fp32", "sum")
    for r in range(P):
        refops.assert_same("fp32", to_host(dev[r], "fp32"), want[r])


@pytest.mark.parametrize("algo,P", [("ring", 5), ("rhd", 6), ("pipeline", 8), ("flat", 4), ("rhd", 1),
                                    ("ring", 17), ("ring", 34)])
def test_out_of_place(algo, P):
    """recv holds what the in-place call would leave; send is untouched; ranks
    with send == recv run in place in the same call.  The copies go 32 ranks
    per launch, a launch of at most 16 with its items in the kernel arguments:
    17 ranks (rank 0 in place) copy 16 in one launch, 34 ranks copy 32, then 1."""
    dtype = "fp16"
    colls = ["allreduce", "reduce_scatter", "all_gather"] if algo != "flat" else ["allreduce"]
    if algo == "rhd":
        colls += ["reduce", "broadcast"]
    with comm_for(algo, P, 8192)[0] as comm:
        S, M = comm.S or 1, comm.M or 1
        for coll in colls:
            for L in (1000, 3 * 4096 + 3):
                say(f"case oop algo={algo} P={P} coll={coll} L={L}")
                xs = make_inputs(dtype, "sum", P, L, seed=L)
                send = [to_dev(x, dtype) for x in xs]
                recv = [torch.full_like(t, 7.0) for t in send]
                recv[0] = send[0]  # rank 0 in place
                comm.out_of_place(coll, send, recv, dtype, "sum", root=min(1, P - 1))
                torch.cuda.synchronize()
                want = [x.copy() for x in xs]
                oracle.run(coll, algo, want, dtype, "sum", S=S, M=M, loop_bytes=8192, root=min(1, P - 1))
                for r in range(P):
                    got = to_host(recv[r], dtype)
                    if coll == "reduce" and r != min(1, P - 1):
                        continue
                    if coll == "reduce_scatter":
                        if algo == "pipeline":
                            continue  # owned blocks are per loop; the full-buffer check below covers them
                        b, e = refops.seg_bounds(L, P, r)
                        refops.assert_same(dtype, got[b:e], want[r][b:e], f"{coll} rank {r}")
                    else:
                        refops.assert_same(dtype, got, want[r], f"{coll} rank {r}")
                    if r > 0:
                        assert np.array_equal(to_host(send[r], dtype).view(np.uint16), xs[r].view(np.uint16))


@pytest.mark.parametrize("dtype", DTYPES)
def test_parity_fused_single_workgroup(dtype):
    """Whole schedules run as one single-workgroup launch give the oracle's bits."""
    rng = np.random.default_rng(zlib.crc32(("fused" + dtype).encode()))
    cases = [("ring", 5, (5, "ring"), {}), ("rhd", 8, (8, "rhd"), {}), ("rhd", 6, (6, "rhd"), {}),
             ("pipeline", 8, (8, "pipeline", 2, 4, 4096), dict(S=2, M=4, loop_bytes=4096)),
             ("flat", 7, (7, "flat"), {}), ("tree", 13, (13, "tree", 0, 3), dict(M=3)),
             ("hier", 6, (6, "hier", 3, 2), dict(S=3, M=2))]
    for algo, P, args, kw in cases:
        with hc.Comm(*args) as comm:
            comm.set_fused_limit(1 << 40)
            comm.set_exec_mode("fused")
            colls = ["allreduce"] if algo in ("flat", "tree", "hier") else ["allreduce", "reduce_scatter", "all_gather"]
            if algo == "rhd":
                colls += ["reduce", "broadcast"]
            for coll in colls:
                op = str(rng.choice(OPS))
                L = int(rng.choice([1, 5, 1000, 3 * 4096 + 7]))
                say(f"case fused algo={algo} coll={coll} dtype={dtype} op={op} P={P} L={L}")
                xs = make_inputs(dtype, op, P, L, seed=L + P)
                dev = [to_dev(x, dtype) for x in xs]
                if coll == "reduce":
                    comm.reduce(dev, dtype, op, root=P - 1)
                elif coll == "broadcast":
                    comm.broadcast(dev, dtype, root=P - 1)
                else:
                    getattr(comm, coll)(dev, dtype, op)
                torch.cuda.synchronize()
                want = [x.copy() for x in xs]
                oracle.run(coll, algo, want, dtype, op, root=P - 1, **kw)
                for r in ([P - 1] if coll == "reduce" else range(P)):
                    refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"fused {algo} {coll} rank {r}")


def test_fused_step_ranges_and_graph():
    """run_steps over sub-ranges and graph nodes also take the single-workgroup path."""
    P, L, dtype = 8, 5000, "bf16"
    xs = make_inputs(dtype, "sum", P, L, seed=3)
    with hc.Comm(P, "ring") as comm:
        comm.set_fused_limit(1 << 40)
        comm.set_exec_mode("fused")
        n = comm.plan_info("allreduce", L, dtype)["nsteps"]
        dev = [to_dev(x, dtype) for x in xs]
        want = [x.copy() for x in xs]
        for a, b in ((0, 3), (3, 4), (4, n)):
            comm.run_steps("allreduce", dev, a, b, dtype, "sum")
            torch.cuda.synchronize()
            oracle.run("allreduce", "ring", want, dtype, "sum", first_step=a, last_step=b)
            for r in range(P):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"steps [{a},{b}) rank {r}")
        gb = [to_dev(x, dtype) for x in xs]
        with hc.Graph() as g:
            g.add(comm, "allreduce", gb, dtype, "sum")
            g.build()
            for rep in range(3):
                for t, x in zip(gb, xs):
                    t.copy_(to_dev(x, dtype))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                for r in range(P):
                    refops.assert_same(dtype, to_host(gb[r], dtype), want[r], f"graph replay {rep} rank {r}")
