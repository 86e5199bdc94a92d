"""Pins of the oracle's Flat, K-ary tree and non-pipelined hierarchical
AllReduce (pages: topology article "AllReduce算法实现" for Flat and Tree;
pipeline article "与其它分级算法的关系" for the hierarchical stages).

- values exact for integers against a brute-force sum (numpy);
- order bit-exact against the closed-order evaluators;
- step counts: Flat 2; Tree 2 x depth of its heap-ordered tree, which is
  the page's 2 log_K N rounds whenever N is a power of K; hierarchical 2S;
- special cases: hierarchical (S, 1) == ring (S); hierarchical (1, M) ==
  pipeline (1, M) == left fold; tree with every rank a child of the root
  (K >= P-1) == Flat;
- HBM bytes of the in-place fused steps: Flat (2P+1) D.
"""
import math
from collections import defaultdict

import numpy as np
import pytest

import closed_order as co
import oracle
import refops
import synth


def ints(P, L, seed=0):
    return [synth.generate("int32", L, synth.UNIFORM_INT, -(2 ** 20), 2 ** 20, seed=seed, stream=62, rank=r)
            for r in range(P)]


def floats(dtype, P, L, seed=0):
    return [synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=63, rank=r) for r in range(P)]


def replay(algo, xs, dtype, op="sum", **kw):
    b = [x.copy() for x in xs]
    oracle.run("allreduce", algo, b, dtype, op, **kw)
    return b


VARIANTS = [("flat", P, {}) for P in (2, 3, 5, 8, 16)] + \
           [("tree", P, dict(M=K)) for P in (2, 3, 7, 8, 13, 16) for K in (2, 3, 4)] + \
           [("hier", S * M, dict(S=S, M=M)) for S, M in ((2, 4), (4, 2), (3, 3), (4, 8), (1, 4), (4, 1))]


@pytest.mark.parametrize("algo,P,kw", VARIANTS)
def test_integer_values_exact(algo, P, kw):
    for L in (1, P - 1, 3 * P + 2, 500):
        if L < 1:
            continue
        xs = ints(P, L, seed=L)
        want = np.stack([x.astype(np.int64) for x in xs]).sum(axis=0).astype(np.int32)
        out = replay(algo, xs, "int32", **kw)
        for r in range(P):
            assert np.array_equal(out[r], want), (algo, P, kw, L, r)


@pytest.mark.parametrize("algo,P,kw", VARIANTS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_order(algo, P, kw, dtype):
    L = 4 * P + 3
    xs = floats(dtype, P, L, seed=P)
    out = replay(algo, xs, dtype, **kw)
    if algo == "flat":
        want = co.left_fold(dtype, "sum", xs)
    elif algo == "tree":
        want = co.tree_allreduce(dtype, "sum", xs, kw["M"])
    else:
        want = co.hier_allreduce(dtype, "sum", xs, kw["S"], kw["M"])
    for r in range(P):
        refops.assert_same(dtype, out[r], want, f"{algo} {kw} r={r}")


def test_step_counts():
    for P in (2, 3, 8, 16, 33):
        assert oracle.num_steps("allreduce", "flat", P) == 2
    for K in (2, 3, 4):
        for d in (1, 2, 3):
            N = K ** d
            assert oracle.num_steps("allreduce", "tree", N, 1, K) == 2 * d  # the page's 2 log_K N
        for P in (2, 5, 11, 20):
            depth, i = 0, P - 1
            while i > 0:
                i, depth = (i - 1) // K, depth + 1
            assert oracle.num_steps("allreduce", "tree", P, 1, K) == 2 * depth
    for S, M in ((2, 4), (4, 8), (3, 1)):
        assert oracle.num_steps("allreduce", "hier", S * M, S, M) == 2 * S
    for algo, P, kw in VARIANTS:
        b = [np.zeros(4 * P, np.int32) for _ in range(P)]
        tr = oracle.run("allreduce", algo, b, "int32", "sum", trace=True, **kw)
        steps = sorted({t["step"] for t in tr})
        n = oracle.num_steps("allreduce", algo, P, kw.get("S", 1), kw.get("M", 1))
        if algo == "hier" and kw["M"] == 1:
            n -= 1  # the closing intra-server step has no peers to send to
        assert steps == list(range(n))


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_special_cases(dtype):
    for S in (2, 3, 5):
        xs = floats(dtype, S, 101, seed=S)
        a = replay("hier", xs, dtype, S=S, M=1)
        b = replay("ring", xs, dtype)
        for r in range(S):
            refops.assert_same(dtype, a[r], b[r], "hier(S,1) vs ring")
    for M in (2, 4, 6):
        xs = floats(dtype, M, 101, seed=M)
        a = replay("hier", xs, dtype, S=1, M=M)
        b = replay("pipeline", xs, dtype, S=1, M=M)
        want = co.left_fold(dtype, "sum", xs)
        for r in range(M):
            refops.assert_same(dtype, a[r], want, "hier(1,M) vs left fold")
            refops.assert_same(dtype, b[r], want, "pipeline(1,M) vs left fold")
    for P in (3, 5, 8):
        xs = floats(dtype, P, 101, seed=P + 9)
        a = replay("tree", xs, dtype, M=P)
        b = replay("flat", xs, dtype)
        for r in range(P):
            refops.assert_same(dtype, a[r], b[r], "tree(K >= P-1) vs flat")


def test_flat_hbm_bytes():
    for P in (2, 5, 8):
        L = 64
        b = [np.zeros(L, np.int32) for _ in range(P)]
        tr = oracle.run("allreduce", "flat", b, "int32", "sum", trace=True)
        total = 0
        for s in sorted({t["step"] for t in tr}):
            reads, writes = set(), set()
            for t in (t for t in tr if t["step"] == s):
                reads.add((t["src"], t["begin"], t["count"]))
                writes.add((t["dst"], t["begin"], t["count"]))
            total += sum(c for *_, c in reads) + sum(c for *_, c in writes)
        assert total == (2 * P + 1) * L


def test_variants_are_allreduce_only():
    xs = ints(4, 8)
    for algo, kw in (("flat", {}), ("tree", dict(M=2)), ("hier", dict(S=2, M=2))):
        with pytest.raises(oracle.OracleError) as e:
            oracle.run("reduce_scatter", algo, [x.copy() for x in xs], "int32", "sum", **kw)
        assert e.value.code == oracle.EUNSUPPORTED
