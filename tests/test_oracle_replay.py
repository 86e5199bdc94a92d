"""Pins of the oracle's schedule replays against the definition and closed orders.

- value: brute-force direct reduction (numpy, independent of the oracle):
  exact for integer types (wrapped), for max/min in every type, and for
  integer-valued binary32 data; otherwise within the per-element bound of a
  (P-1)-addition sum and the norm-wise bounds (1e-5 for fp32,
  2^-7 (P-1) for fp16/bf16).
- order: the closed-order evaluators of ``closed_order`` agree bit-exactly.
- invariants: all ranks equal; ring == RHD == pipeline for integers;
  ring AllReduce == all-gather after reduce-scatter; P = 2 ring == RHD;
  pipeline(S, 1) == ring(S); pipeline(1, M) == left fold; P = 1 identity;
  windowed and step-range replays agree with the full replay.
"""
import numpy as np
import pytest

import closed_order as co
import oracle
import refops
import synth

DTYPES = ["fp32", "fp16", "bf16", "int32", "int8"]
OPS = ["sum", "prod", "max", "min"]


def inputs(dtype, P, L, seed=0, dist=None):
    """Random inputs; prod uses values near 1 so products stay finite."""
    if dtype in ("int32", "int8"):
        lo, hi = (-(2 ** 20), 2 ** 20) if dtype == "int32" else (-128, 127)
        return [synth.generate(dtype, L, synth.UNIFORM_INT, lo, hi, seed=seed, stream=90, rank=r)
                for r in range(P)]
    return [synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=91, rank=r) for r in range(P)]


def prod_inputs(dtype, P, L, seed=0):
    xs = inputs(dtype, P, L, seed)
    if dtype in refops.FLOATS:
        out = []
        for x in xs:
            f = 1.0 + 0.05 * refops.to_f64(dtype, x)
            out.append(refops.from_f32(dtype, f.astype(np.float32)))
        return out
    return xs


def replay(coll, algo, xs, dtype, op, **kw):
    bufs = [x.copy() for x in xs]
    oracle.run(coll, algo, bufs, dtype, op, **kw)
    return bufs


def brute(dtype, op, xs):
    if dtype in refops.INTS:
        X = np.stack([x.astype(np.int64) for x in xs])
        if op == "sum":
            acc = X.sum(axis=0)
        elif op == "prod":
            acc = X[0].copy()
            for x in X[1:]:
                acc = acc * x
        elif op == "max":
            acc = X.max(axis=0)
        else:
            acc = X.min(axis=0)
        return acc.astype(refops.STORAGE[dtype])  # wraps to the element width
    return None


ALGOS = [("ring", {}), ("rhd", {}), ("pipeline", None)]
PS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 17]
LS = [0, 1, 3, 7, 64, 257]


def pipe_shape(P):
    for M in (4, 3, 2):
        if P % M == 0 and P // M >= 1:
            return P // M, M
    return P, 1


def algo_kwargs(algo, P):
    if algo == "pipeline":
        S, M = pipe_shape(P)
        return dict(S=S, M=M)
    return {}


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
@pytest.mark.parametrize("dtype", ["int32", "int8"])
@pytest.mark.parametrize("op", OPS)
def test_integer_allreduce_exact(algo, dtype, op):
    for P in PS:
        for L in LS:
            xs = prod_inputs(dtype, P, L, seed=P * 1000 + L) if op == "prod" else inputs(dtype, P, L, seed=P * 1000 + L)
            out = replay("allreduce", algo, xs, dtype, op, **algo_kwargs(algo, P))
            want = brute(dtype, op, xs)
            for r in range(P):
                assert np.array_equal(out[r], want), (P, L, r)
            # the C definition agrees with numpy's
            if L:
                assert np.array_equal(oracle.direct(dtype, op, xs).astype(refops.STORAGE[dtype]), want)


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("op", ["max", "min"])
def test_float_maxmin_exact(algo, dtype, op):
    for P in (2, 3, 5, 8, 12):
        L = 301
        xs = inputs(dtype, P, L, seed=P)
        # plant signed zeros, infinities and NaNs
        for r, x in enumerate(xs):
            f = refops.to_f64(dtype, x).astype(np.float32)
            f[r::29] = 0.0
            f[(r + 3)::31] = -0.0
            f[(r * 7) % 97] = np.inf
            if r == 1:
                f[200] = np.nan
            xs[r] = refops.from_f32(dtype, f)
        out = replay("allreduce", algo, xs, dtype, op, **algo_kwargs(algo, P))
        want = co.left_fold(dtype, op, xs)  # max/min are associative and commutative
        for r in range(P):
            refops.assert_same(dtype, out[r], want, f"{algo} P={P} r={r}")
            bits_o = out[r].view(np.uint32 if dtype == "fp32" else np.uint16)
            bits_w = want.view(np.uint32 if dtype == "fp32" else np.uint16)
            assert np.array_equal(bits_o, bits_w)


def test_integer_valued_fp32_is_exact():
    """Integers in [-8, 8] over 4 ranks: every partial is an integer below 2^24."""
    P, L = 4, 4096
    xs = synth.rank_inputs("ring_p4_fp32_int", P, L)
    out = replay("allreduce", "ring", xs, "fp32", "sum")
    want = np.stack([x.astype(np.int64) for x in xs]).sum(axis=0).astype(np.float32)
    for r in range(P):
        assert np.array_equal(out[r], want)


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_float_sum_within_bound(algo, dtype):
    for P in (2, 3, 5, 8, 16):
        L = 1000
        xs = inputs(dtype, P, L, seed=P + 5)
        out = replay("allreduce", algo, xs, dtype, "sum", **algo_kwargs(algo, P))
        ok = refops.sum_bound_ok(dtype, out[0], xs)
        assert ok.all(), (P, int((~ok).sum()))
        exact = np.stack([refops.to_f64(dtype, x) for x in xs]).sum(axis=0)
        rel = np.linalg.norm(refops.to_f64(dtype, out[0]) - exact) / np.linalg.norm(exact)
        assert rel <= (1e-5 if dtype == "fp32" else 2.0 ** -7 * (P - 1))
        # the C definition is the same binary64 sum up to binary64 rounding order
        d = oracle.direct(dtype, "sum", xs)
        assert np.allclose(d, exact, rtol=1e-12, atol=1e-300)


ORDER_CASES = [(P, L) for P in (2, 3, 4, 5, 6, 7, 8, 9, 13, 16) for L in (1, 5, 33, 250)]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_ring_order(dtype, op):
    for P, L in ORDER_CASES:
        xs = prod_inputs(dtype, P, L, seed=P) if op == "prod" else inputs(dtype, P, L, seed=P)
        out = replay("allreduce", "ring", xs, dtype, op)
        want = co.ring_allreduce(dtype, op, xs)
        for r in range(P):
            refops.assert_same(dtype, out[r], want, f"ring P={P} L={L} r={r}")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_rhd_order(dtype, op):
    for P, L in ORDER_CASES:
        xs = prod_inputs(dtype, P, L, seed=P) if op == "prod" else inputs(dtype, P, L, seed=P)
        out = replay("allreduce", "rhd", xs, dtype, op)
        want = co.rhd_allreduce(dtype, op, xs)
        for r in range(P):
            refops.assert_same(dtype, out[r], want, f"rhd P={P} L={L} r={r}")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_pipeline_order(dtype):
    for S, M in ((4, 8), (3, 2), (2, 4), (1, 4), (4, 1), (2, 3), (3, 3)):
        P = S * M
        for L, loop in ((250, 0), (999, 64 * refops.np.dtype(refops.STORAGE[dtype]).itemsize), (40, 8)):
            xs = inputs(dtype, P, L, seed=L + P)
            esz = np.dtype(refops.STORAGE[dtype]).itemsize
            out = replay("allreduce", "pipeline", xs, dtype, "sum", S=S, M=M, loop_bytes=loop)
            loop_elems = (loop // esz) if loop else (32 << 20) // esz
            want = co.pipeline_allreduce(dtype, "sum", xs, S, M, loop_elems)
            for r in range(P):
                refops.assert_same(dtype, out[r], want, f"pipe {S}x{M} L={L} r={r}")


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_rhd_reduce_scatter_order_and_ownership(dtype):
    for P in (2, 4, 8, 16):
        for L in (P, 3 * P + 1, 200):
            xs = inputs(dtype, P, L, seed=P * 3 + L)
            out = replay("reduce_scatter", "rhd", xs, dtype, "sum")
            want = co.rhd_reduce_scatter_value(dtype, "sum", xs)
            for v in range(P):
                b, e = refops.seg_bounds(L, P, v)
                refops.assert_same(dtype, out[v][b:e], want[b:e], f"rhd rs P={P} v={v}")


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
def test_reduce_scatter_ownership_and_all_gather(algo):
    dtype = "int32"
    for P in (2, 4, 6, 8, 12, 16):
        if algo == "rhd" and P & (P - 1):
            continue
        kw = algo_kwargs(algo, P)
        for L in (P - 1, P, 5 * P + 3, 401):
            xs = inputs(dtype, P, L, seed=L)
            want = brute(dtype, "sum", xs)
            rs = replay("reduce_scatter", algo, xs, dtype, "sum", **kw)
            owner = {}
            if algo == "pipeline":
                # blocks of each loop: block g of the loop owned by rank g (one loop here)
                for g in range(P):
                    owner[g] = refops.seg_bounds(L, P, g)
            else:
                for g in range(P):
                    owner[g] = refops.seg_bounds(L, P, g)
            for g, (b, e) in owner.items():
                assert np.array_equal(rs[g][b:e], want[b:e]), (algo, P, L, g)
            # all-gather from "rank g holds segment g" gives everyone everything
            ag_in = [np.zeros(L, np.int32) for _ in range(P)]
            for g, (b, e) in owner.items():
                ag_in[g][b:e] = want[b:e]
            ag = replay("all_gather", algo, ag_in, dtype, "sum", **kw)
            for r in range(P):
                assert np.array_equal(ag[r], want), (algo, P, L, r)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_ring_allreduce_is_all_gather_after_reduce_scatter(dtype):
    for P in (3, 5, 8):
        xs = inputs(dtype, P, 301, seed=P)
        ar = replay("allreduce", "ring", xs, dtype, "sum")
        rs = replay("reduce_scatter", "ring", xs, dtype, "sum")
        ag = replay("all_gather", "ring", rs, dtype, "sum")
        for r in range(P):
            refops.assert_same(dtype, ar[r], ag[r])


@pytest.mark.parametrize("dtype", DTYPES)
def test_two_ranks_ring_equals_rhd(dtype):
    for op in OPS:
        xs = prod_inputs(dtype, 2, 257) if op == "prod" else inputs(dtype, 2, 257)
        a = replay("allreduce", "ring", xs, dtype, op)
        b = replay("allreduce", "rhd", xs, dtype, op)
        refops.assert_same(dtype, a[0], b[0], op)
        refops.assert_same(dtype, a[1], b[1], op)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_pipeline_special_cases(dtype):
    for S in (2, 3, 5, 8):
        xs = inputs(dtype, S, 333, seed=S)
        a = replay("allreduce", "pipeline", xs, dtype, "sum", S=S, M=1)
        b = replay("allreduce", "ring", xs, dtype, "sum")
        for r in range(S):
            refops.assert_same(dtype, a[r], b[r], f"pipe({S},1) vs ring")
    for M in (2, 3, 8):
        xs = inputs(dtype, M, 333, seed=M + 50)
        a = replay("allreduce", "pipeline", xs, dtype, "sum", S=1, M=M)
        want = co.left_fold(dtype, "sum", xs)
        for r in range(M):
            refops.assert_same(dtype, a[r], want, f"pipe(1,{M}) vs left fold")


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
def test_single_rank_is_identity(algo):
    xs = inputs("fp32", 1, 100)
    out = replay("allreduce", algo, xs, "fp32", "sum", **algo_kwargs(algo, 1))
    assert np.array_equal(out[0], xs[0])


@pytest.mark.parametrize("algo", ["ring", "rhd", "pipeline"])
@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather"])
def test_window_and_step_range_replay(algo, coll):
    dtype = "bf16"
    P = 8 if algo != "pipeline" else 8
    kw = dict(S=2, M=4, loop_bytes=200) if algo == "pipeline" else {}
    L = 1001
    xs = inputs(dtype, P, L, seed=3)
    full = replay(coll, algo, xs, dtype, "sum", **kw)
    rng = np.random.default_rng(0)
    for _ in range(6):
        w0 = int(rng.integers(0, L))
        w1 = int(rng.integers(w0, L + 1))
        win = replay(coll, algo, [x[w0:w1].copy() for x in xs], dtype, "sum", L=L, w0=w0, **kw)
        for r in range(P):
            refops.assert_same(dtype, win[r], full[r][w0:w1], f"window [{w0},{w1})")
    nsteps = oracle.num_steps(coll, algo, P, kw.get("S", 1), kw.get("M", 1))
    for cut in range(nsteps + 1):
        part = replay(coll, algo, xs, dtype, "sum", last_step=cut, **kw)
        oracle.run(coll, algo, part, dtype, "sum", first_step=cut, **kw)
        for r in range(P):
            refops.assert_same(dtype, part[r], full[r], f"cut at {cut}")


@pytest.mark.parametrize("algo,kw", [("ring", {}), ("rhd", {}), ("pipeline", dict(S=2, M=3, loop_bytes=4096)),
                                     ("flat", {}), ("tree", dict(M=3)), ("hier", dict(S=2, M=3))])
@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather", "reduce", "broadcast"])
def test_parallel_replay_equals_the_single_thread_replay(algo, kw, coll):
    """run_parallel (disjoint windows side by side, ragged cuts) gives every
    bit of the one-thread replay, for every algorithm and collective it offers."""
    dtype, P, L = "fp16", 6, 50_021
    xs = inputs(dtype, P, L, seed=9)
    try:
        full = replay(coll, algo, xs, dtype, "sum", root=4, **kw)
    except oracle.OracleError as e:
        assert e.code == oracle.EUNSUPPORTED
        return
    for T in (2, 5, 12):
        par = [x.copy() for x in xs]
        used = oracle.run_parallel(coll, algo, par, dtype, "sum", threads=T, root=4, **kw)
        assert used == T
        for r in range(P):
            assert np.array_equal(par[r].view(np.uint16), full[r].view(np.uint16)), (T, r)


def test_rooted_collectives_need_rhd_and_a_valid_root():
    xs = inputs("fp32", 6, 10)
    for algo in ("ring", "pipeline"):
        with pytest.raises(oracle.OracleError) as e:
            oracle.run("reduce", algo, [x.copy() for x in xs], "fp32", "sum", S=2, M=3)
        assert e.value.code == oracle.EUNSUPPORTED
    for root in (-1, 6):
        with pytest.raises(oracle.OracleError) as e:
            oracle.run("broadcast", "rhd", [x.copy() for x in xs], "fp32", "sum", root=root)
        assert e.value.code == oracle.EINVAL
