"""The five workloads at their full sizes, on the GPU, against the oracle.

Every workload is compared with the oracle's replay of the whole vector of
every rank, bit for bit, the sweep's largest size included (1 GiB per rank:
16 GiB of rank buffers and as much for the pristine copies and the oracle's).
Large replays run as disjoint windows on the host's cores (oracle.run_parallel:
the same arithmetic, window by window).  Accuracy against the binary64 direct
sum: norm-wise relative error <= 1e-5 (fp32) or 2^-7 (P-1) (fp16 / bf16), and
the per-element bound of a (P-1)-addition sum (above 64 Mi elements per rank,
on the first 64 Mi).

Workloads:
  ring_p4   ring AllReduce, P=4, L=4096, fp32 integers in [-8, 8]
  ring_p8   ring AllReduce, P=8, L=64 Mi fp32 N(0, 1e-3)  (the benchmark's workload)
  rhd       RHD AllReduce, P in {8, 5}, bf16 N(0,1) sum and int32 U[-2^20, 2^20] max,
            1 KiB .. 64 KiB per rank
  sweep     ring and RHD AllReduce / reduce-scatter / all-gather, P=16, fp16 N(0, 0.01),
            4 KiB .. 1 GiB per rank in powers of 4
  pipe      pipeline AllReduce, 4 servers x 8 ranks, 32 MiB loops, bf16 N(0, 1e-2), 512 MiB per rank
"""
import sys

import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
import synth
from gpu_util import TORCH, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ranks_identical(bufs, dtype):
    iv = {1: torch.int8, 2: torch.int16, 4: torch.int32}[torch.tensor([], dtype=TORCH[dtype]).element_size()]
    b0 = bufs[0].view(iv)
    return all(torch.equal(b.view(iv), b0) for b in bufs[1:])


def bits(dtype, x):
    return np.ascontiguousarray(x).view({4: np.uint32, 2: np.uint16, 1: np.uint8}[x.dtype.itemsize])


def assert_same_fast(dtype, got, want, what):
    """Bit equality of whole vectors; only on a mismatch the NaN-aware
    comparison (any two NaNs equal) decides and reports."""
    if np.array_equal(bits(dtype, got), bits(dtype, want)):
        return
    refops.assert_same(dtype, got, want, what)


def sum_accuracy(dtype, y, xs, chunk=1 << 20):
    """Per-element bound of a (P-1)-addition sum over the whole vector, and
    the norm-wise relative error against the binary64 direct sum."""
    num = den = 0.0
    for a in range(0, y.size, chunk):
        b = min(y.size, a + chunk)
        part = [x[a:b] for x in xs]
        assert refops.sum_bound_ok(dtype, y[a:b], part).all(), f"per-element bound fails in [{a},{b})"
        exact = np.zeros(b - a)
        for x in part:
            exact += refops.to_f64(dtype, x)
        num += float(np.sum((refops.to_f64(dtype, y[a:b]) - exact) ** 2))
        den += float(np.sum(exact ** 2))
    return np.sqrt(num / den)


def check_full(coll, algo, xs, dev, dtype, *, S=1, M=1, loop_bytes=0, op="sum"):
    """Oracle replay of the whole vectors (run in windows on the host's cores)
    against every rank's GPU buffer; a reduce-scatter compares each rank's
    own segment.  Returns the oracle's result."""
    P, L = len(xs), xs[0].size
    want = [x.copy() for x in xs]
    T = oracle.run_parallel(coll, algo, want, dtype, op, S=S, M=M, loop_bytes=loop_bytes)
    say(f"  oracle replay of {algo} {coll} P={P} L={L} on {T} threads done")
    for r in range(P):
        got = to_host(dev[r], dtype)
        if coll == "reduce_scatter":
            b, e = refops.seg_bounds(L, P, r)
            assert_same_fast(dtype, got[b:e], want[r][b:e], f"{algo} rs rank {r}")
        else:
            assert_same_fast(dtype, got, want[r], f"{algo} {coll} rank {r}")
        del got
    return want


def test_ring_p4_fp32_integers():
    P, L = 4, 4096
    xs = synth.rank_inputs("ring_p4_fp32_int", P, L)
    dev = [to_dev(x, "fp32") for x in xs]
    with hc.Comm(P, "ring") as c:
        assert c.plan_info("allreduce", L, "fp32")["nsteps"] == 6
        c.allreduce(dev, "fp32", "sum")
        torch.cuda.synchronize()
    want = [x.copy() for x in xs]
    oracle.run("allreduce", "ring", want, "fp32", "sum")
    exact = np.stack([x.astype(np.int64) for x in xs]).sum(axis=0).astype(np.float32)
    for r in range(P):
        got = to_host(dev[r], "fp32")
        assert np.array_equal(got.view(np.uint32), want[r].view(np.uint32))
        assert np.array_equal(got, exact)


@pytest.mark.parametrize("columns", [False, True])
def test_ring_p8_fp32_64Mi(columns):
    """The benchmark's workload, every element of every rank against the oracle."""
    P, L = 8, 64 << 20
    say(f"case ring_p8 fp32 64Mi columns={columns}: generate and upload")
    xs = synth.rank_inputs("ring_p8_fp32_grad", P, L)
    dev = [to_dev(x, "fp32") for x in xs]
    with hc.Comm(P, "ring") as c:
        if columns:
            c.set_columns(1 << 40)
            c.set_exec_mode("columns")
            assert c.exec_choice("allreduce", L, "fp32") == "columns"
        else:
            assert c.exec_choice("allreduce", L, "fp32") == "steps"
        say("case ring_p8 fp32 64Mi: allreduce")
        c.allreduce(dev, "fp32", "sum")
        torch.cuda.synchronize()
    want = check_full("allreduce", "ring", xs, dev, "fp32")
    assert sum_accuracy("fp32", want[0], xs) <= 1e-5
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("exec_mode", ["steps", "auto"])
@pytest.mark.parametrize("P", [8, 5])
def test_rhd_small_messages(P, exec_mode):
    for kib in (1, 2, 4, 8, 16, 32, 64):
        for recipe, op in (("rhd_bf16_normal", "sum"), ("rhd_int32_uniform", "max")):
            dtype = synth.RECIPES[recipe]["dtype"]
            L = kib * 1024 // np.dtype(refops.STORAGE[dtype]).itemsize
            say(f"case rhd P={P} {kib} KiB {dtype} {op}")
            xs = synth.rank_inputs(recipe, P, L)
            dev = [to_dev(x, dtype) for x in xs]
            with hc.Comm(P, "rhd") as c:
                c.set_exec_mode(exec_mode)
                assert c.plan_info("allreduce", L, dtype)["nsteps"] == 6
                c.allreduce(dev, dtype, op)
                torch.cuda.synchronize()
            want = [x.copy() for x in xs]
            oracle.run("allreduce", "rhd", want, dtype, op)
            for r in range(P):
                refops.assert_same(dtype, to_host(dev[r], dtype), want[r], f"rank {r}")
            if op == "max":
                exact = np.stack(xs).max(axis=0)
                assert np.array_equal(to_host(dev[0], dtype), exact)
            else:
                ok = refops.sum_bound_ok(dtype, want[0], xs)
                assert ok.all()
                exact = np.stack([refops.to_f64(dtype, x) for x in xs]).sum(axis=0)
                rel = np.linalg.norm(refops.to_f64(dtype, want[0]) - exact) / np.linalg.norm(exact)
                assert rel <= 2.0 ** -7 * (P - 1)


SWEEP = [4096 * 4 ** i for i in range(10)]  # bytes per rank: 4 KiB .. 1 GiB
ACCURACY_ELEMS = 64 << 20  # the binary64 accuracy bound is checked on at most this many leading elements


@pytest.mark.parametrize("nbytes", SWEEP)
def test_sweep_p16_fp16(nbytes):
    P, dtype, recipe = 16, "fp16", "sweep_p16_fp16"
    L = nbytes // 2
    say(f"case sweep P=16 fp16 {nbytes} B/rank: upload")
    xs = synth.rank_inputs(recipe, P, L)
    pristine = [to_dev(x, dtype) for x in xs]
    dev = [torch.empty_like(t) for t in pristine]
    for algo in ("ring", "rhd"):
        with hc.Comm(P, algo) as c:
            for coll in ("allreduce", "reduce_scatter", "all_gather"):
                for d, p in zip(dev, pristine):
                    d.copy_(p)
                say(f"case sweep {algo} {coll} {nbytes} B/rank")
                getattr(c, coll)(dev, dtype, "sum")
                torch.cuda.synchronize()
                if coll != "reduce_scatter":
                    assert ranks_identical(dev, dtype)
                want = check_full(coll, algo, xs, dev, dtype)
                if coll == "allreduce":
                    n = min(L, ACCURACY_ELEMS)
                    assert sum_accuracy(dtype, want[0][:n], [x[:n] for x in xs]) <= 2.0 ** -7 * (P - 1)
                del want
    del dev, pristine, xs
    torch.cuda.empty_cache()


def test_pipeline_4x8_bf16_512MiB():
    S, M = 4, 8
    P, dtype, recipe = S * M, "bf16", "pipe_4x8_bf16"
    L = 256 << 20  # 512 MiB per rank
    loop_bytes = 32 << 20
    say("case pipeline 4x8 bf16 512MiB: generate and upload")
    xs = synth.rank_inputs(recipe, P, L)
    dev = [to_dev(x, dtype) for x in xs]
    with hc.Comm(P, "pipeline", S, M, loop_bytes) as c:
        assert c.plan_info("allreduce", L, dtype)["nsteps"] == 2 * S
        say("case pipeline 4x8: allreduce")
        c.allreduce(dev, dtype, "sum")
        torch.cuda.synchronize()
    want = check_full("allreduce", "pipeline", xs, dev, dtype, S=S, M=M, loop_bytes=loop_bytes)
    assert sum_accuracy(dtype, want[0], xs) <= 2.0 ** -7 * (P - 1)
    del dev, want
    torch.cuda.empty_cache()
