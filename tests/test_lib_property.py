"""Property test: for random (algorithm, collective, P, L, root, server
shape, loop size), the library's step tables, executed on the CPU with
numpy / torch element ops, equal the oracle's replay bit for bit (int32 sums
and bf16 sums), and every step is free of read/write overlaps between items
(executing its items one after another gives the same result)."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import allreduce_reduction_amd as hc
import oracle
import refops
import synth
from test_lib_host import simulate

ALGOS = ["ring", "rhd", "pipeline", "flat", "tree", "hier"]
COLLS = ["allreduce", "reduce_scatter", "all_gather", "reduce", "broadcast"]


@st.composite
def case(draw):
    algo = draw(st.sampled_from(ALGOS))
    coll = draw(st.sampled_from(COLLS))
    P = draw(st.integers(1, 20))
    L = draw(st.integers(0, 300))
    root = draw(st.integers(0, P - 1))
    divs = [m for m in range(1, P + 1) if P % m == 0]
    M = draw(st.sampled_from(divs))
    K = draw(st.integers(2, 5))
    loop = draw(st.sampled_from([0, 16, 40, 100])) * 4
    dtype = draw(st.sampled_from(["int32", "bf16"]))
    return algo, coll, P, L, root, M, K, loop, dtype


def supported(algo, coll):
    if coll in ("reduce", "broadcast"):
        return algo == "rhd"
    if algo in ("flat", "tree", "hier"):
        return coll == "allreduce"
    return True


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(case())
def test_library_tables_equal_oracle(c):
    algo, coll, P, L, root, M, K, loop, dtype = c
    S = P // M
    if algo in ("pipeline", "hier"):
        comm = hc.Comm(P, algo, S, M, loop)
        kw = dict(S=S, M=M, loop_bytes=loop)
    elif algo == "tree":
        comm = hc.Comm(P, "tree", 0, K)
        kw = dict(M=K)
    else:
        comm = hc.Comm(P, algo)
        kw = {}
    with comm:
        if not supported(algo, coll):
            try:
                comm.plan_info(coll, L, dtype, root=root)
            except hc.HbmcError as e:
                assert e.code == 2
                return
            assert P == 1 and False, "unsupported collective accepted"
        info = comm.plan_info(coll, L, dtype, root=root)
        assert info["nsteps"] == oracle.num_steps(coll, algo, P, kw.get("S", 1), kw.get("M", 1))
        items = comm.plan_items(coll, L, dtype, root=root)
        if dtype == "int32":
            xs = [synth.generate("int32", L, synth.UNIFORM_INT, -1000, 1000, seed=L, stream=50, rank=r)
                  for r in range(P)]
        else:
            xs = [synth.generate("bf16", L, synth.NORMAL, 1.0, seed=L, stream=51, rank=r) for r in range(P)]
        got = simulate(items, info["nsteps"], xs, dtype, "sum")
        seq = simulate(items, info["nsteps"], xs, dtype, "sum", sequential=True)
        want = [x.copy() for x in xs]
        oracle.run(coll, algo, want, dtype, "sum", root=root, **kw)
        for r in range(P):
            refops.assert_same(dtype, got[r], want[r], f"{c} rank {r}")
            refops.assert_same(dtype, seq[r], want[r], f"{c} rank {r} (sequential)")
