"""Host checks of the column kernel's chunk tables (no GPU).

The library cuts every work item into chunks at multiples of a column length
and gives each chunk the earlier chunks it must follow.  Here the tables are checked for shape
(chunks tile each item in order, are cut at multiples of the chunk length,
and wait only on chunks of earlier steps over the same elements) and by outcome: the chunks are executed in orders
that respect ONLY the dependencies — random ones, and the order that always
runs the ready chunk of largest index (as far from step order as the
dependencies allow) — with numpy element ops, and every such order must
give bit for bit the oracle's step-by-step result.  The same adversarial
order with the dependencies dropped must fail, so the check has teeth.
Finally the kernel's own order -- each column on its own, its chunks in
ascending index, the columns one after another (any interleaving of
independent columns is equivalent) -- must give the oracle's result too.
"""
import numpy as np
import pytest

import allreduce_reduction_amd as hc
import oracle
import refops
import synth

MODES = {"copy", "fold", "recv_fold"}


def _exec_chunk(bufs, dtype, op, it, b, e):
    src = [bufs[r][b:e] for r in it["src"]]
    if it["mode"] == "copy":
        v = src[0].copy()
    elif it["mode"] == "fold":
        v = src[0].copy()
        for x in src[1:]:
            v = refops.combine(dtype, op, v, x)
    else:
        acc = src[1].copy()
        for x in src[2:]:
            acc = refops.combine(dtype, op, acc, x)
        v = refops.combine(dtype, op, src[0], acc)
    for r in it["dst"]:
        bufs[r][b:e] = v


def _run_order(xs, dtype, op, items, chunks, order):
    bufs = [x.copy() for x in xs]
    for c in order:
        ch = chunks[c]
        _exec_chunk(bufs, dtype, op, items[ch["item"]], ch["begin"], ch["begin"] + ch["count"])
    return bufs


def _orders(chunks, rng, n_random, use_deps=True):
    n = len(chunks)
    succ = [[] for _ in range(n)]
    indeg = [0] * n
    if use_deps:
        for c, ch in enumerate(chunks):
            for d in ch["deps"]:
                succ[d].append(c)
                indeg[c] += 1
    outs = []
    for k in range(n_random + 1):
        deg = list(indeg)
        ready = [c for c in range(n) if deg[c] == 0]
        order = []
        while ready:
            if k == 0:
                c = max(ready)
            else:
                c = ready[int(rng.integers(0, len(ready)))]
            ready.remove(c)
            order.append(c)
            for s in succ[c]:
                deg[s] -= 1
                if deg[s] == 0:
                    ready.append(s)
        assert len(order) == n, "dependency cycle"
        outs.append(order)
    return outs


def _inputs(dtype, P, L, seed):
    return [synth.generate(dtype, L, synth.UNIFORM_INT, -1000, 1000, seed=seed, stream=90, rank=r)
            for r in range(P)]


CASES = [  # (comm args, oracle keywords, collective, P, L, chunk bytes)
    ((4, "ring"), {}, "allreduce", 4, 103, 64),
    ((5, "ring"), {}, "reduce_scatter", 5, 77, 16),
    ((5, "ring"), {}, "all_gather", 5, 77, 32),
    ((2, "ring"), {}, "allreduce", 2, 40, 16),
    ((8, "rhd"), {}, "allreduce", 8, 200, 64),
    ((6, "rhd"), {}, "allreduce", 6, 131, 48),
    ((6, "rhd"), {}, "reduce_scatter", 6, 131, 32),
    ((7, "rhd"), {}, "all_gather", 7, 90, 16),
    ((5, "rhd"), {}, "reduce", 5, 64, 32),
    ((5, "rhd"), {}, "broadcast", 5, 64, 16),
    ((8, "pipeline", 2, 4, 256), dict(S=2, M=4, loop_bytes=256), "allreduce", 8, 150, 32),
    ((6, "pipeline", 3, 2, 0), dict(S=3, M=2), "reduce_scatter", 6, 61, 16),
    ((6, "flat"), {}, "allreduce", 6, 50, 16),
    ((9, "tree", 0, 3), dict(M=3), "allreduce", 9, 45, 16),
    ((6, "hier", 3, 2), dict(S=3, M=2), "allreduce", 6, 70, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0][1]}-{c[2]}-P{c[3]}" for c in CASES])
def test_chunks_tile_items_and_wait_on_earlier_steps(case):
    args, kw, coll, P, L, chunk = case
    dtype = "int32"
    with hc.Comm(*args) as comm:
        items = comm.plan_items(coll, L, dtype, root=1 % P)
        chunks = comm.plan_chunks(coll, L, dtype, chunk, root=1 % P)
    ce = max(16, chunk // 16 * 16) // 4
    by_item = {}
    for c, ch in enumerate(chunks):
        by_item.setdefault(ch["item"], []).append(ch)
        assert 0 < ch["count"] <= ce
        assert ch["step"] == items[ch["item"]]["step"]
        assert ch["deps"] == sorted(set(ch["deps"]))
        for d in ch["deps"]:
            assert chunks[d]["step"] < ch["step"]
            # a chunk waits only on chunks over the same column of elements
            assert chunks[d]["begin"] // ce == ch["begin"] // ce
        # cut at multiples of the chunk length
        assert ch["begin"] // ce == (ch["begin"] + ch["count"] - 1) // ce
        if c:
            prev = chunks[c - 1]
            assert (prev["step"], prev["item"]) <= (ch["step"], ch["item"])
    assert sorted(by_item) == list(range(len(items)))
    for i, cs in by_item.items():
        pos = items[i]["begin"]
        for ch in cs:
            assert ch["begin"] == pos
            pos += ch["count"]
        assert pos == items[i]["begin"] + items[i]["count"]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0][1]}-{c[2]}-P{c[3]}" for c in CASES])
def test_dependency_orders_give_the_oracle_result(case):
    args, kw, coll, P, L, chunk = case
    dtype, op = "int32", "sum"
    root = 1 % P
    rng = np.random.default_rng(L * 31 + P)
    xs = _inputs(dtype, P, L, seed=P)
    want = [x.copy() for x in xs]
    oracle.run(coll, args[1], want, dtype, op, root=root, **kw)
    with hc.Comm(*args) as comm:
        items = comm.plan_items(coll, L, dtype, root=root)
        chunks = comm.plan_chunks(coll, L, dtype, chunk, root=root)
    for order in _orders(chunks, rng, n_random=6):
        got = _run_order(xs, dtype, op, items, chunks, order)
        for r in range(P):
            assert np.array_equal(got[r], want[r]), f"rank {r}"


@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[10]], ids=["ring", "rhd", "pipeline"])
def test_dropping_dependencies_breaks_the_result(case):
    args, kw, coll, P, L, chunk = case
    dtype, op = "int32", "sum"
    xs = _inputs(dtype, P, L, seed=P)
    want = [x.copy() for x in xs]
    oracle.run(coll, args[1], want, dtype, op, **kw)
    with hc.Comm(*args) as comm:
        items = comm.plan_items(coll, L, dtype)
        chunks = comm.plan_chunks(coll, L, dtype, chunk)
    order = _orders(chunks, np.random.default_rng(0), 0, use_deps=False)[0]
    got = _run_order(xs, dtype, op, items, chunks, order)
    assert any(not np.array_equal(got[r], want[r]) for r in range(P))


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0][1]}-{c[2]}-P{c[3]}" for c in CASES])
def test_column_by_column_order_gives_the_oracle_result(case):
    args, kw, coll, P, L, chunk = case
    dtype, op = "int32", "sum"
    root = 1 % P
    xs = _inputs(dtype, P, L, seed=P + 1)
    want = [x.copy() for x in xs]
    oracle.run(coll, args[1], want, dtype, op, root=root, **kw)
    with hc.Comm(*args) as comm:
        items = comm.plan_items(coll, L, dtype, root=root)
        chunks = comm.plan_chunks(coll, L, dtype, chunk, root=root)
    ce = max(16, chunk // 16 * 16) // 4
    cols = {}
    for c, ch in enumerate(chunks):
        cols.setdefault(ch["begin"] // ce, []).append(c)
    for rev in (False, True):
        order = [c for g in sorted(cols, reverse=rev) for c in cols[g]]
        got = _run_order(xs, dtype, op, items, chunks, order)
        for r in range(P):
            assert np.array_equal(got[r], want[r]), f"rank {r}"


def test_chunk_argument_checks():
    with hc.Comm(4, "ring") as comm:
        for bad in (0, 15, (1 << 31) + 1):
            with pytest.raises(hc.HbmcError):
                comm.plan_chunks("allreduce", 100, "fp32", bad)
        with pytest.raises(hc.HbmcError):
            comm.set_columns(1 << 20, 8)
        with pytest.raises(hc.HbmcError):
            comm.set_columns(1 << 20, (1 << 31) + 16)
        comm.set_columns(1 << 20, 1024)
        comm.set_columns(1 << 20)
        comm.set_columns(0)
        assert len(comm.plan_chunks("allreduce", 0, "fp32", 64)) == 0
