"""Host checks of the flow kernel's tables and of its protocol (no GPU).

The flow kernel runs all steps of a call in one launch: items are cut into
tiles (one step's work on one column of elements), tiles are handed out step
after step by an atomic ticket, and a workgroup that takes the seq-th tile of
a column waits until the column's counter reads seq, runs the tile and sets
the counter to seq + 1.  Here:

- the tables are checked for shape: tiles in ticket order (step after step,
  columns ascending), seq numbering, chunks inside their tile's column and
  step, every item covered exactly once;
- the protocol is modelled on the CPU, action by action, exactly as each
  workgroup executes it (initial ticket; per tile: take the next ticket, wait
  on the column counter with a bound, read every operand, write every result,
  publish; at the end the exit count and the last workgroup's reset), with a
  random scheduler over the resident workgroups and a limit on how many are
  resident at once (the hardware starts a workgroup when a slot frees).  Reads
  and writes of a tile are separate actions, so any race shows.  Every run
  must end (no deadlock for any interleaving or residency), leave the
  counters reset, and give bit for bit the oracle's result;
- with the wait removed, the same model must give a wrong result (the check
  has teeth);
- with every wait made unreachable (the host-forced give-up test), every run
  must still end, count timeouts and reset the counters.
"""
import numpy as np
import pytest

import allreduce_reduction_amd as hc
import oracle
import refops
import synth

CASES = [  # (comm args, oracle keywords, collective, P, L, tile bytes)
    ((4, "ring"), {}, "allreduce", 4, 103, 64),
    ((5, "ring"), {}, "reduce_scatter", 5, 77, 16),
    ((5, "ring"), {}, "all_gather", 5, 77, 32),
    ((16, "ring"), {}, "allreduce", 16, 301, 64),
    ((8, "rhd"), {}, "allreduce", 8, 200, 64),
    ((6, "rhd"), {}, "allreduce", 6, 131, 48),
    ((6, "rhd"), {}, "reduce_scatter", 6, 131, 32),
    ((7, "rhd"), {}, "all_gather", 7, 90, 16),
    ((5, "rhd"), {}, "reduce", 5, 64, 32),
    ((5, "rhd"), {}, "broadcast", 5, 64, 16),
    ((8, "pipeline", 2, 4, 256), dict(S=2, M=4, loop_bytes=256), "allreduce", 8, 150, 32),
    ((6, "flat"), {}, "allreduce", 6, 50, 16),
    ((9, "tree", 0, 3), dict(M=3), "allreduce", 9, 45, 16),
    ((6, "hier", 3, 2), dict(S=3, M=2), "allreduce", 6, 70, 16),
]
IDS = [f"{c[0][1]}-{c[2]}-P{c[3]}" for c in CASES]


def _inputs(dtype, P, L, seed):
    return [synth.generate(dtype, L, synth.UNIFORM_INT, -1000, 1000, seed=seed, stream=91, rank=r)
            for r in range(P)]


def _tables(case, dtype="int32"):
    args, kw, coll, P, L, tile = case
    root = 1 % P
    with hc.Comm(*args) as comm:
        items = comm.plan_items(coll, L, dtype, root=root)
        tiles, chunks = comm.plan_flow(coll, L, dtype, tile, root=root)
    return items, tiles, chunks, max(16, tile // 16 * 16) // np.dtype(refops.STORAGE[dtype]).itemsize


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_tiles_follow_ticket_order_and_cover_every_item(case):
    items, tiles, chunks, ce = _tables(case)
    seen = {}
    prev = (-1, -1)
    covered = {}
    for t in tiles:
        key = (t["step"], t["col"])
        assert key > prev, "step after step, columns ascending"
        prev = key
        assert t["seq"] == seen.get(t["col"], 0)
        seen[t["col"]] = t["seq"] + 1
        assert len(t["chunks"]) > 0
        for c in t["chunks"]:
            ch = chunks[c]
            it = items[ch["item"]]
            assert it["step"] == t["step"]
            assert 0 < ch["count"] <= ce
            assert ch["begin"] // ce == t["col"] == (ch["begin"] + ch["count"] - 1) // ce
            covered.setdefault(ch["item"], []).append((ch["begin"], ch["count"]))
    # the chunks partition every item, in order, and appear once each
    assert [c for t in tiles for c in t["chunks"]] == list(range(len(chunks)))
    assert sorted(covered) == [i for i, it in enumerate(items) if it["count"] > 0]
    for i, parts in covered.items():
        pos = items[i]["begin"]
        for b, n in sorted(parts):
            assert b == pos
            pos += n
        assert pos == items[i]["begin"] + items[i]["count"]


def _combine(dtype, op, mode, vals):
    if mode == "copy":
        return vals[0].copy()
    if mode == "fold":
        v = vals[0].copy()
        for x in vals[1:]:
            v = refops.combine(dtype, op, v, x)
        return v
    acc = vals[1].copy()
    for x in vals[2:]:
        acc = refops.combine(dtype, op, acc, x)
    return refops.combine(dtype, op, vals[0], acc)


def simulate(xs, dtype, op, items, tiles, chunks, ncols, *, groups, resident, rng, wait=True,
             unreachable=False, bound=200_000, batch=1):
    """Run the flow kernel's protocol on the CPU; returns (buffers, timeouts, ctrl, progress)."""
    bufs = [x.copy() for x in xs]
    ntiles = len(tiles)
    ctrl = dict(next=0, done=0, abort=0)
    timeouts = [0]
    progress = [0] * ncols

    def take():
        t = ctrl["next"]
        ctrl["next"] += batch
        return t

    def workgroup():
        # one action per yield; the scheduler interleaves workgroups between them
        cur = take()
        yield
        while cur < ntiles:
            nxt = take()
            yield
            for t in range(cur, min(cur + batch, ntiles)):
                yield from run_tile(tiles[t])
            cur = nxt
            yield
        ctrl["done"] += 1
        if ctrl["done"] == groups:
            for g in range(ncols):
                progress[g] = 0
            ctrl.update(next=0, abort=0, done=0)

    def run_tile(tile):
        ok = True
        if tile["seq"] > 0 and wait:
            target = 1 << 32 if unreachable else tile["seq"]
            spins = 0
            while progress[tile["col"]] != target:
                if ctrl["abort"]:
                    ok = False
                    break
                spins += 1
                if spins > bound:
                    timeouts[0] += 1
                    ctrl["abort"] = 1
                    ok = False
                    break
                yield
        yield
        if ok:
            # every operand of every chunk read, then (later) every result written
            results = []
            for c in tile["chunks"]:
                ch = chunks[c]
                it = items[ch["item"]]
                b, e = ch["begin"], ch["begin"] + ch["count"]
                results.append((it, b, e, _combine(dtype, op, it["mode"], [bufs[r][b:e].copy() for r in it["src"]])))
            yield
            for it, b, e, v in results:
                for r in it["dst"]:
                    bufs[r][b:e] = v
            yield
            progress[tile["col"]] = tile["seq"] + 1
        yield

    pending = list(range(groups))
    active = []
    steps = 0
    while pending or active:
        while pending and len(active) < resident:
            pending.pop(0)
            active.append(workgroup())
        k = int(rng.integers(0, len(active)))
        try:
            next(active[k])
        except StopIteration:
            active.pop(k)
        steps += 1
        assert steps < 50_000_000, "the protocol did not end"
    return bufs, timeouts[0], ctrl, progress


def _want(case, xs, dtype, op):
    args, kw, coll, P, L, tile = case
    want = [x.copy() for x in xs]
    oracle.run(coll, args[1], want, dtype, op, root=1 % P, **kw)
    return want


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_protocol_ends_and_gives_the_oracle_result(case):
    args, kw, coll, P, L, tile = case
    dtype, op = "int32", "sum"
    items, tiles, chunks, ce = _tables(case)
    ncols = (L + ce - 1) // ce
    xs = _inputs(dtype, P, L, seed=P)
    want = _want(case, xs, dtype, op)
    rng = np.random.default_rng(L * 7 + P)
    for groups, resident, batch in ((1, 1, 1), (3, 1, 2), (5, 2, 1), (8, 8, 3), (len(tiles) + 3, 4, 1),
                                    (len(tiles) + 3, len(tiles) + 3, 1), (9, 9, 4), (4, 2, 16)):
        got, tmo, ctrl, progress = simulate(xs, dtype, op, items, tiles, chunks, ncols, groups=groups,
                                            resident=resident, rng=rng, batch=batch)
        assert tmo == 0
        assert ctrl == dict(next=0, done=0, abort=0) and not any(progress)
        for r in range(P):
            assert np.array_equal(got[r], want[r]), f"rank {r}, {groups} workgroups, {resident} resident"


@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[10]], ids=["ring", "rhd", "pipeline"])
def test_protocol_without_the_wait_breaks_the_result(case):
    args, kw, coll, P, L, tile = case
    dtype, op = "int32", "sum"
    items, tiles, chunks, ce = _tables(case)
    ncols = (L + ce - 1) // ce
    xs = _inputs(dtype, P, L, seed=P)
    want = _want(case, xs, dtype, op)
    rng = np.random.default_rng(5)
    wrong = 0
    for _ in range(4):
        got, _, _, _ = simulate(xs, dtype, op, items, tiles, chunks, ncols, groups=len(tiles), resident=len(tiles),
                                rng=rng, wait=False)
        wrong += any(not np.array_equal(got[r], want[r]) for r in range(P))
    assert wrong > 0


@pytest.mark.parametrize("case", [CASES[0], CASES[5]], ids=["ring", "rhd"])
def test_unreachable_waits_give_up_and_reset(case):
    args, kw, coll, P, L, tile = case
    dtype, op = "int32", "sum"
    items, tiles, chunks, ce = _tables(case)
    ncols = (L + ce - 1) // ce
    xs = _inputs(dtype, P, L, seed=P)
    rng = np.random.default_rng(9)
    for groups, resident, batch in ((1, 1, 1), (6, 3, 2), (len(tiles), len(tiles), 1), (5, 5, 7)):
        got, tmo, ctrl, progress = simulate(xs, dtype, op, items, tiles, chunks, ncols, groups=groups,
                                            resident=resident, rng=rng, unreachable=True, bound=50, batch=batch)
        assert tmo >= 1
        assert ctrl == dict(next=0, done=0, abort=0) and not any(progress)


def test_flow_argument_checks():
    with hc.Comm(4, "ring") as comm:
        for bad in (0, 15, (1 << 31) + 1):
            with pytest.raises(hc.HbmcError):
                comm.plan_flow("allreduce", 100, "fp32", bad)
        for kw in (dict(tile_bytes=8), dict(wgs_per_cu=0), dict(wgs_per_cu=65), dict(wait_us=0),
                   dict(tiles_per_ticket=0), dict(tiles_per_ticket=4097)):
            with pytest.raises(hc.HbmcError):
                comm.set_flow(**kw)
        comm.set_flow(64 << 10, 4, 1000)
        # forced flow: calls and step ranges of two or more busy steps on one
        # 16-byte phase
        comm.set_exec_mode("flow")
        assert comm.exec_choice("allreduce", 1000, "fp32") == "flow"
        assert comm.exec_choice("allreduce", 1000, "fp32", first=0, last=3) == "flow"
        assert comm.exec_choice("allreduce", 1000, "fp32", first=2, last=3) == "steps"  # one step
        for first, last in ((-1, 2), (2, 1), (0, 7)):
            with pytest.raises(hc.HbmcError):
                comm.plan_flow("allreduce", 1000, "fp32", 64, first=first, last=last)
        assert comm.exec_bytes("allreduce", 1000, "fp32", "flow") == comm.exec_bytes("allreduce", 1000, "fp32", "steps")
    with hc.Comm(2, "ring") as comm:
        comm.set_exec_mode("flow")
        assert comm.exec_choice("reduce_scatter", 1000, "fp32") == "steps"  # one step
    with hc.Comm(40, "flat") as comm:  # a fold of 40 sources: beyond the records
        comm.set_exec_mode("flow")
        assert comm.exec_choice("allreduce", 1000, "fp32") == "steps"
        with pytest.raises(hc.HbmcError):
            comm.plan_flow("allreduce", 1000, "fp32", 64)
    # AUTO never picks the flow form
    with hc.Comm(16, "ring") as comm:
        assert comm.exec_choice("allreduce", 8 << 20, "fp16") == "steps"


RANGE_CASES = [(CASES[3], 5, 19), (CASES[4], 1, 5), (CASES[5], 0, 4), (CASES[10], 1, 4), (CASES[13], 1, 3)]
RANGE_IDS = [f"{c[0][1]}-P{c[3]}-steps{a}-{b}" for c, a, b in RANGE_CASES]


def _range_tables(case, first, last, dtype="int32"):
    args, kw, coll, P, L, tile = case
    with hc.Comm(*args) as comm:
        n = comm.plan_info(coll, L, dtype, root=1 % P)["nsteps"]
        assert 0 <= first < last <= n
        return comm.plan_flow(coll, L, dtype, tile, root=1 % P, first=first, last=last)


@pytest.mark.parametrize("case,first,last", RANGE_CASES, ids=RANGE_IDS)
def test_range_tables_are_the_whole_tables_steps_renumbered(case, first, last):
    """A step range's table holds the whole call's tiles of those steps, in
    the same order and with the same chunks, each column's seq counted from 0
    within the range."""
    items, tiles, chunks, ce = _tables(case)
    rt, rc = _range_tables(case, first, last)
    sel = [t for t in tiles if first <= t["step"] < last]
    assert len(rt) == len(sel)
    seen = {}
    for a, b in zip(rt, sel):
        assert (a["col"], a["step"]) == (b["col"], b["step"])
        assert a["seq"] == seen.get(a["col"], 0)
        seen[a["col"]] = a["seq"] + 1
        assert [rc[i] for i in a["chunks"]] == [chunks[i] for i in b["chunks"]]


@pytest.mark.parametrize("case,first,last", RANGE_CASES, ids=RANGE_IDS)
def test_range_protocol_gives_the_oracle_step_range(case, first, last):
    """The protocol model over a range's table, from the state the oracle
    reaches after steps [0, first), ends with the oracle's state after steps
    [0, last), for several residencies."""
    args, kw, coll, P, L, tile = case
    dtype, op = "int32", "sum"
    items, _, _, ce = _tables(case)
    rt, rc = _range_tables(case, first, last)
    ncols = (L + ce - 1) // ce
    xs = _inputs(dtype, P, L, seed=P + first)
    start = [x.copy() for x in xs]
    oracle.run(coll, args[1], start, dtype, op, root=1 % P, first_step=0, last_step=first, **kw)
    want = [x.copy() for x in start]
    oracle.run(coll, args[1], want, dtype, op, root=1 % P, first_step=first, last_step=last, **kw)
    rng = np.random.default_rng(first * 31 + last)
    for groups, resident, batch in ((1, 1, 1), (5, 2, 2), (len(rt) + 2, len(rt) + 2, 1), (6, 6, 3)):
        got, tmo, ctrl, progress = simulate(start, dtype, op, items, rt, rc, ncols, groups=groups, resident=resident,
                                            rng=rng, batch=batch)
        assert tmo == 0
        assert ctrl == dict(next=0, done=0, abort=0) and not any(progress)
        for r in range(P):
            assert np.array_equal(got[r], want[r]), f"rank {r}, {groups} workgroups, {resident} resident"
