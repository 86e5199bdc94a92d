"""Pins of the oracle's schedule shape: step counts, the 5-rank RHD example and
the byte closed forms of the pages' cost tables.

- steps at P = 8: ring 14, RHD 6 (page "HCCL Ring AllReduce 与 RHD 对比",
  section on recursive halving-doubling); RHD with P not a power of two:
  2 floor(log2 P) + 2 (page "HCCL RHD 算法深度解析", Table 1); pipeline:
  (S - 1) ring steps + 1 intra-server step per phase (page "HCCL Pipeline
  分级流水算法深度解析", Table 1).
- the 5-rank example (tests/golden/rhd_5rank_example.txt).
- per-rank bytes received: 2 D (P-1)/P for ring and power-of-two RHD
  AllReduce (ring section of the first page; Table 1 of the RHD page);
  critical path of non-power-of-two RHD: (2 (p'-1)/p' + 2) D transferred
  and ((p'-1)/p' + 1) D reduced (Table 1 of the RHD page); pipeline:
  (S - 1) blocks of D/P between servers per phase (Table 1 of the pipeline page).
- algorithmic HBM bytes of in-place steps (each distinct block read once and
  written once): 5 D (P-1) for ring / RHD AllReduce; for the S x M pipeline
  (M+1) + (S-1)(M+2) blocks of D/P per rank in reduce-scatter and
  (S-1)(M+1) + M in all-gather (in each ring step the block a rank forwards
  to the next server is the block it passes to its own server's peers, so it
  is read once for M writes), 74 D in all for 4 x 8.
"""
import os
from collections import defaultdict
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def trace_of(coll, algo, P, L, dtype="int32", **kw):
    bufs = [np.zeros(L, oracle.NP_STORAGE[dtype]) for _ in range(P)]
    return oracle.run(coll, algo, bufs, dtype, "sum", trace=True, trace_cap=1 << 18, **kw)


def test_step_counts_printed_by_the_pages():
    assert oracle.num_steps("allreduce", "ring", 8) == 14
    assert oracle.num_steps("allreduce", "rhd", 8) == 6
    for P in (3, 5, 6, 7, 9, 12, 17, 31):
        k = P.bit_length() - 1
        assert oracle.num_steps("allreduce", "rhd", P) == 2 * k + 2
    for P in (2, 4, 16, 32):
        k = P.bit_length() - 1
        assert oracle.num_steps("allreduce", "rhd", P) == 2 * k
        assert oracle.num_steps("reduce_scatter", "rhd", P) == k
    for S, M in ((4, 8), (2, 2), (1, 4), (5, 1)):
        assert oracle.num_steps("allreduce", "pipeline", S * M, S, M) == 2 * S
        assert oracle.num_steps("reduce_scatter", "pipeline", S * M, S, M) == S
    for P in (2, 3, 8, 16):
        assert oracle.num_steps("allreduce", "ring", P) == 2 * (P - 1)
        assert oracle.num_steps("reduce_scatter", "ring", P) == P - 1


@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather"])
@pytest.mark.parametrize("algo,P,kw", [("ring", 8, {}), ("rhd", 8, {}), ("rhd", 5, {}),
                                       ("pipeline", 32, dict(S=4, M=8))])
def test_trace_step_count_matches(coll, algo, P, kw):
    if algo == "rhd" and coll != "allreduce" and P & (P - 1):
        return
    tr = trace_of(coll, algo, P, 64 * P, **kw)
    steps = sorted({t["step"] for t in tr})
    assert steps == list(range(oracle.num_steps(coll, algo, P, kw.get("S", 1), kw.get("M", 1))))


def _load_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "rhd_5rank_example.txt"), encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        step, kind, who, frac = line.split()
        rows.append((int(step), kind, who, Fraction(frac)))
    return rows


def test_rhd_five_rank_example():
    L = 64
    tr = trace_of("allreduce", "rhd", 5, L)
    rows = _load_golden()
    assert sorted({t["step"] for t in tr}) == [r[0] for r in rows]
    for step, kind, who, frac in rows:
        recs = [t for t in tr if t["step"] == step]
        assert all(t["kind"] == kind for t in recs), step
        assert all(Fraction(t["count"], L) == frac for t in recs), step
        if "->" in who:
            a, b = (int(x) for x in who.split("->"))
            assert [(t["src"], t["dst"]) for t in recs] == [(a, b)]
        else:
            members = {int(x) for x in who.strip("{}").split(",")}
            assert {t["dst"] for t in recs} == members and {t["src"] for t in recs} == members
            pairs = {(t["src"], t["dst"]) for t in recs}
            assert all((d, s) in pairs for (s, d) in pairs)  # partners exchange


def _recv_bytes(tr, e):
    per_rank = defaultdict(int)
    for t in tr:
        if t["src"] != t["dst"]:
            per_rank[t["dst"]] += t["count"] * e
    return per_rank


@pytest.mark.parametrize("algo", ["ring", "rhd"])
@pytest.mark.parametrize("P", [2, 4, 8, 16])
def test_per_rank_received_bytes(algo, P):
    L, e = 48 * P, 4
    D = L * e
    tr = trace_of("allreduce", algo, P, L)
    rb = _recv_bytes(tr, e)
    assert all(Fraction(rb[r]) == Fraction(2 * D * (P - 1), P) for r in range(P))
    red = defaultdict(int)
    for t in tr:
        if t["kind"] == "reduce":
            red[t["dst"]] += t["count"] * e
    assert all(Fraction(red[r]) == Fraction(D * (P - 1), P) for r in range(P))


@pytest.mark.parametrize("P", [3, 5, 6, 7, 12, 13])
def test_rhd_non_power_of_two_critical_path(P):
    pp = 1 << (P.bit_length() - 1)
    L, e = 16 * pp * 3, 4
    D = L * e
    tr = trace_of("allreduce", "rhd", P, L)
    beta = gamma = 0
    for s in sorted({t["step"] for t in tr}):
        recs = [t for t in tr if t["step"] == s]
        per = defaultdict(int)
        red = defaultdict(int)
        for t in recs:
            per[t["dst"]] += t["count"] * e
            if t["kind"] == "reduce":
                red[t["dst"]] += t["count"] * e
        beta += max(per.values())
        gamma += max(red.values()) if red else 0
    assert Fraction(beta) == (2 * Fraction(pp - 1, pp) + 2) * D
    assert Fraction(gamma) == (Fraction(pp - 1, pp) + 1) * D


def test_pipeline_inter_server_bytes_and_total():
    S, M = 4, 8
    P = S * M
    L, e = 64 * P, 2
    D = L * e
    for coll, phases in (("reduce_scatter", 1), ("all_gather", 1), ("allreduce", 2)):
        tr = trace_of(coll, "pipeline", P, L, dtype="bf16", S=S, M=M)
        inter = defaultdict(int)
        for t in tr:
            if t["src"] // M != t["dst"] // M:
                inter[t["dst"]] += t["count"] * e
        assert all(inter[g] == phases * (S - 1) * D // P for g in range(P))


def _hbm_bytes(tr, e):
    """Distinct reads + writes per step, as an in-place fused step moves them."""
    total = 0
    for s in sorted({t["step"] for t in tr}):
        reads, writes = set(), set()
        for t in (t for t in tr if t["step"] == s):
            reads.add((t["src"], t["begin"], t["count"]))
            writes.add((t["dst"], t["begin"], t["count"]))
            if t["kind"] == "reduce":
                reads.add((t["dst"], t["begin"], t["count"]))
        total += sum(c for _, _, c in reads) * e + sum(c for _, _, c in writes) * e
    return total


@pytest.mark.parametrize("algo,P", [("ring", 4), ("ring", 8), ("rhd", 8), ("rhd", 5), ("rhd", 16)])
def test_algorithmic_hbm_bytes_ring_rhd(algo, P):
    L, e = 4 * 64 * P, 4
    D = L * e
    tr = trace_of("allreduce", algo, P, L)
    assert _hbm_bytes(tr, e) == 5 * D * (P - 1)
    if algo == "ring":
        assert _hbm_bytes(trace_of("reduce_scatter", algo, P, L), e) == 3 * D * (P - 1)
        assert _hbm_bytes(trace_of("all_gather", algo, P, L), e) == 2 * D * (P - 1)


def test_algorithmic_hbm_bytes_pipeline_4x8():
    S, M = 4, 8
    P = S * M
    L, e = 32 * P, 2
    D = L * e
    tr = trace_of("allreduce", "pipeline", P, L, dtype="bf16", S=S, M=M)
    assert _hbm_bytes(tr, e) == 74 * D
    blocks = (M + 1) + (S - 1) * (M + 2) + (S - 1) * (M + 1) + M
    assert blocks == 74
