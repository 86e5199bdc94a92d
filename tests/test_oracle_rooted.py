"""Pins of the oracle's RHD collectives beyond AllReduce: stand-alone
reduce-scatter / all-gather for P not a power of two, Reduce and Broadcast
with a root (page "HCCL RHD 算法深度解析", section "耗时计算", Table 1).

- values: integer results exact against a brute-force sum (numpy); float
  results bit-exact against the closed-order evaluators; Broadcast copies
  the root's vector bit for bit to every rank.
- ownership: reduce-scatter leaves segment g of the P-way ceiling split on
  rank g ("保证 Scatter 的顺序"); Reduce leaves everything on the root.
- step counts: reduce-scatter / all-gather floor(log2 p) + 2, Reduce
  2 floor(log2 p) + 1 (2 log2 p for powers of two), Broadcast ceil(log2 p).
- the table's per-step maxima: the non-uniform reduce-scatter's halving step
  i exchanges at most ceil(p / 2^i) shares of n/p; Reduce moves
  (2 (p'-1)/p' + 1) n and reduces ((p'-1)/p' + 1) n on its critical path
  (2 (p-1)/p n and (p-1)/p n for powers of two); Broadcast moves
  ceil(log2 p) n.
"""
from collections import defaultdict
from fractions import Fraction
import math

import numpy as np
import pytest

import closed_order as co
import oracle
import refops
import synth

NP2 = [3, 5, 6, 7, 9, 10, 11, 12, 13, 17, 24]


def ints(P, L, seed=0):
    return [synth.generate("int32", L, synth.UNIFORM_INT, -(2 ** 20), 2 ** 20, seed=seed, stream=60, rank=r)
            for r in range(P)]


def floats(dtype, P, L, seed=0):
    return [synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=61, rank=r) for r in range(P)]


def replay(coll, xs, dtype, op="sum", **kw):
    b = [x.copy() for x in xs]
    oracle.run(coll, "rhd", b, dtype, op, **kw)
    return b


def trace(coll, P, L, **kw):
    b = [np.zeros(L, np.int32) for _ in range(P)]
    return oracle.run(coll, "rhd", b, "int32", "sum", trace=True, trace_cap=1 << 18, **kw)


@pytest.mark.parametrize("P", NP2)
def test_np2_reduce_scatter_and_all_gather_values(P):
    for L in (P - 1, P, 3 * P + 2, 301):
        xs = ints(P, L, seed=L)
        want = np.stack([x.astype(np.int64) for x in xs]).sum(axis=0).astype(np.int32)
        rs = replay("reduce_scatter", xs, "int32")
        for g in range(P):
            b, e = refops.seg_bounds(L, P, g)
            assert np.array_equal(rs[g][b:e], want[b:e]), (P, L, g)
        ag_in = [np.zeros(L, np.int32) for _ in range(P)]
        for g in range(P):
            b, e = refops.seg_bounds(L, P, g)
            ag_in[g][b:e] = want[b:e]
        ag = replay("all_gather", ag_in, "int32")
        for r in range(P):
            assert np.array_equal(ag[r], want), (P, L, r)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_np2_reduce_scatter_order(dtype):
    for P in NP2:
        L = 7 * P + 3
        xs = floats(dtype, P, L, seed=P)
        rs = replay("reduce_scatter", xs, dtype)
        want = co.rhd_reduce_scatter_np2_value(dtype, "sum", xs)
        for g in range(P):
            b, e = refops.seg_bounds(L, P, g)
            refops.assert_same(dtype, rs[g][b:e], want[b:e], f"P={P} g={g}")


@pytest.mark.parametrize("P", [2, 3, 4, 5, 6, 7, 8, 12, 13, 16])
def test_reduce_to_every_root(P):
    L = 5 * P + 1
    xs = ints(P, L, seed=P)
    want = np.stack([x.astype(np.int64) for x in xs]).sum(axis=0).astype(np.int32)
    fx = floats("bf16", P, L, seed=P)
    for root in range(P):
        out = replay("reduce", xs, "int32", root=root)
        assert np.array_equal(out[root], want), (P, root)
        fo = replay("reduce", fx, "bf16", root=root)
        refops.assert_same("bf16", fo[root], co.rhd_reduce_value("bf16", "sum", fx, root), f"P={P} root={root}")


@pytest.mark.parametrize("P", [2, 3, 4, 5, 6, 7, 8, 12, 13, 16])
def test_broadcast_from_every_root(P):
    L = 3 * P + 4
    xs = floats("fp32", P, L, seed=P)
    for root in range(P):
        out = replay("broadcast", xs, "fp32", root=root)
        for r in range(P):
            assert np.array_equal(out[r].view(np.uint32), xs[root].view(np.uint32)), (P, root, r)


def test_step_counts():
    for P in range(2, 33):
        k = P.bit_length() - 1
        pow2 = P == 1 << k
        assert oracle.num_steps("reduce_scatter", "rhd", P) == k + (0 if pow2 else 2)
        assert oracle.num_steps("all_gather", "rhd", P) == k + (0 if pow2 else 2)
        assert oracle.num_steps("reduce", "rhd", P) == 2 * k + (0 if pow2 else 1)
        assert oracle.num_steps("broadcast", "rhd", P) == math.ceil(math.log2(P))
        for coll in ("reduce_scatter", "all_gather"):
            assert sorted({t["step"] for t in trace(coll, P, 4 * P)}) == list(range(oracle.num_steps(coll, "rhd", P)))
        for root in (0, P - 1, P // 2):
            for coll in ("reduce", "broadcast"):
                steps = sorted({t["step"] for t in trace(coll, P, 4 * P, root=root)})
                assert steps == list(range(oracle.num_steps(coll, "rhd", P)))


def _per_step(tr, kind=None):
    out = defaultdict(lambda: defaultdict(int))
    for t in tr:
        if kind is None or t["kind"] == kind:
            out[t["step"]][t["dst"]] += t["count"]
    return {s: max(v.values()) for s, v in out.items()}


@pytest.mark.parametrize("P", NP2)
def test_np2_reduce_scatter_table_maxima(P):
    q = 16
    L = P * q  # every share n/p = q elements
    k = P.bit_length() - 1
    mx = _per_step(trace("reduce_scatter", P, L))
    assert mx[0] == L                           # Reduce: the whole vector
    for i in range(1, k + 1):                   # halving step i: ceil(p / 2^i) shares
        assert mx[i] == math.ceil(P / 2 ** i) * q, (P, i)
    assert mx[k + 1] == q                       # Scatter: one share


@pytest.mark.parametrize("P", [4, 5, 6, 7, 8, 12, 13, 16])
def test_reduce_and_broadcast_table_forms(P):
    k = P.bit_length() - 1
    pp = 1 << k
    L = pp * P * 4
    for root in (0, P - 1):
        tr = trace("reduce", P, L, root=root)
        beta = sum(_per_step(tr).values())
        gamma = sum(_per_step(tr, "reduce").values())
        if P == pp:
            assert Fraction(beta) == 2 * Fraction(P - 1, P) * L
            assert Fraction(gamma) == Fraction(P - 1, P) * L
        else:
            assert Fraction(beta) == (2 * Fraction(pp - 1, pp) + 1) * L
            assert Fraction(gamma) == (Fraction(pp - 1, pp) + 1) * L
        tb = trace("broadcast", P, L, root=root)
        assert sum(_per_step(tb).values()) == math.ceil(math.log2(P)) * L
