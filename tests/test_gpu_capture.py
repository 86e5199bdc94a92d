"""Direct calls captured into a HIP graph by the caller (torch.cuda.graph).

After the first call of a (collective, count, dtype) shape, which builds and
uploads that shape's tables, a call only enqueues kernels on the current
stream, so a caller may capture it.  Each launch form is captured once and
replayed several times, with the inputs restored eagerly and the device
synchronised between replays; every replay must equal the eager result.
"""
import pytest
import torch

import allreduce_reduction_amd as hc
import refops
from gpu_util import to_dev, to_host
from test_gpu_parity import comm_for, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,algo,P,L,dtype", [
    ("steps", "ring", 8, 50_001, "bf16"),
    ("lds", "rhd", 8, 4096 + 3, "fp32"),
    ("fused", "rhd", 5, 300, "int32"),
    ("columns", "ring", 5, 20_000, "fp16"),
    ("steps", "pipeline", 8, 30_000, "bf16"),
    ("auto", "rhd", 16, 1 << 16, "fp16"),
    ("regs", "ring", 8, 20_003, "bf16"),
    ("flow", "ring", 8, 50_001, "fp32"),
    ("flow", "rhd", 6, 30_000, "int8"),
])
def test_capture_after_first_call(mode, algo, P, L, dtype):
    xs = make_inputs(dtype, "sum", P, L, seed=L)
    comm, _, _ = comm_for(algo, P, 8192 if algo == "pipeline" else 0)
    with comm:
        comm.set_exec_mode(mode)
        if mode == "columns":
            comm.set_columns(1 << 40, 1024)
        if mode != "auto":
            assert comm.exec_choice("allreduce", L, dtype) == mode
        ref = [to_dev(x, dtype) for x in xs]
        comm.allreduce(ref, dtype, "sum")  # first call of the shape: tables built here
        torch.cuda.synchronize()
        want = [to_host(t, dtype) for t in ref]
        bufs = [to_dev(x, dtype) for x in xs]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            comm.allreduce(bufs, dtype, "sum")
        for rep in range(3):
            for b, x in zip(bufs, xs):
                b.copy_(to_dev(x, dtype))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for r in range(P):
                refops.assert_same(dtype, to_host(bufs[r], dtype), want[r], f"{mode} replay {rep} rank {r}")
        del g
