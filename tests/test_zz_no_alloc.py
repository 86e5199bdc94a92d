"""The no-allocation AllReduce (hbmc_allreduce_noalloc) against hbmc_allreduce.

Both calls go through the C ABI on the same inputs; the no-allocation one
takes its step kernels' item tables from the library's fixed device array.
Each case makes two calls in a row on one communicator, the second with a
smaller input (so the array holds the first call's larger table when the
second copies its own in), and compares every rank bit for bit with
hbmc_allreduce's result, which the oracle checks too.  A schedule whose
table does not fit the array is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import allreduce_reduction_amd as hc
import oracle
import refops
import synth
from gpu_util import strided_buffers, to_dev, to_host

pytestmark = pytest.mark.gpu


def inputs(dtype, P, L, seed):
    if dtype in ("int32", "int8"):
        lo, hi = (-(2 ** 20), 2 ** 20) if dtype == "int32" else (-128, 127)
        return [synth.generate(dtype, L, synth.UNIFORM_INT, lo, hi, seed=seed, stream=95, rank=r)
                for r in range(P)]
    return [synth.generate(dtype, L, synth.NORMAL, 1.0, seed=seed, stream=95, rank=r) for r in range(P)]


CASES = [
    # (algo, P, S, M, loop_bytes, dtype, op, L_first, L_second)
    ("ring", 8, 0, 0, 0, "fp32", "sum", 1 << 20, 4096 + 3),
    ("rhd", 5, 0, 0, 0, "bf16", "sum", 300_001, 1000),
    ("rhd", 16, 0, 0, 0, "fp16", "max", 1 << 18, 77),
    ("ring", 3, 0, 0, 0, "int8", "sum", 100_003, 65),
    ("pipeline", 32, 4, 8, 1 << 16, "bf16", "sum", 1 << 20, 40_000),  # steps of hundreds of items
    ("flat", 6, 0, 0, 0, "int32", "prod", 50_000, 999),
    ("auto", 8, 0, 0, 0, "fp32", "min", 1 << 16, 5),
]


@pytest.mark.parametrize("algo,P,S,M,loop,dtype,op,L1,L2", CASES)
def test_noalloc_matches_allreduce(algo, P, S, M, loop, dtype, op, L1, L2):
    with hc.Comm(P, algo, S, M, loop) as ref, hc.Comm(P, algo, S, M, loop) as na:
        for call, L in enumerate((L1, L2)):
            print(f"case noalloc {algo} P={P} {dtype} {op} L={L} call {call}", flush=True)
            xs = inputs(dtype, P, L, seed=call + 3)
            want = [to_dev(x, dtype) for x in xs]
            got = [to_dev(x, dtype) for x in xs]
            ref.allreduce(want, dtype, op)
            na.allreduce_noalloc(got, dtype, op)
            torch.cuda.synchronize()
            expect = [x.copy() for x in xs]
            oracle.run("allreduce", ref.auto_choice("allreduce", L, dtype) if algo == "auto" else algo,
                       expect, dtype, op, S=S or 1, M=M or 1, loop_bytes=loop)
            for r in range(P):
                w = to_host(want[r], dtype)
                refops.assert_same(dtype, to_host(got[r], dtype), w, f"call {call} rank {r} vs hbmc_allreduce")
                refops.assert_same(dtype, w, expect[r], f"call {call} rank {r} vs oracle")


def test_noalloc_unaligned_phases_and_back_to_back_on_one_stream():
    """Buffers of different 16-byte phases (element-wise kernel, items from the
    array), then two different shapes back to back on one stream with no
    synchronisation between them: the second copy into the array waits for
    the first call's kernels."""
    P, dtype = 4, "fp16"
    xs = inputs(dtype, P, 20_011, seed=5)
    views, _back = strided_buffers(xs, dtype, [0, 1, 3, 6])
    ref_views, _rb = strided_buffers(xs, dtype, [0, 1, 3, 6])
    ys = inputs(dtype, P, 9_000, seed=6)
    a = [to_dev(y, dtype) for y in ys]
    b = [to_dev(y, dtype) for y in ys]
    with hc.Comm(P, "ring") as ref, hc.Comm(P, "ring") as na:
        ref.allreduce(ref_views, dtype, "sum")
        ref.allreduce(b, dtype, "sum")
        na.allreduce_noalloc(views, dtype, "sum")
        na.allreduce_noalloc(a, dtype, "sum")
        torch.cuda.synchronize()
    for r in range(P):
        refops.assert_same(dtype, to_host(views[r], dtype), to_host(ref_views[r], dtype), f"phased rank {r}")
        refops.assert_same(dtype, to_host(a[r], dtype), to_host(b[r], dtype), f"second shape rank {r}")


def test_noalloc_refuses_a_table_beyond_the_array():
    """A 4 x 8 pipeline with 1 KiB loops over 128 KiB per rank has 8 x 128 x 32
    items, beyond the array's 13107: HBMC_ERR_SCRATCH, buffers untouched."""
    P, dtype, L = 32, "bf16", 1 << 16
    xs = inputs(dtype, P, L, seed=8)
    bufs = [to_dev(x, dtype) for x in xs]
    lib = hc.load_library()
    with hc.Comm(P, "pipeline", 4, 8, 1024) as c:
        arr = (ctypes.c_void_p * P)(*[t.data_ptr() for t in bufs])
        rc = lib.hbmc_allreduce_noalloc(c._h, arr, L, hc.DTYPE[dtype], hc.OP["sum"], None)
        assert rc == 5  # HBMC_ERR_SCRATCH
        torch.cuda.synchronize()
    for r in range(P):
        assert np.array_equal(to_host(bufs[r], dtype), xs[r])
