"""Benchmark: ring AllReduce of P=8 logical ranks on one GPU.

Workload: 8 ranks x 64 Mi fp32 elements (256 MiB per rank), values N(0, 1e-3)
from the seeded generator, sum, ring reduce-scatter + all-gather (14 steps,
one fused kernel launch per step).  A "step" of this benchmark is one whole
AllReduce.

Reported (one JSON line):
  value      busbw = algbw * 2(P-1)/P, algbw = D / t, D = bytes per rank
  pct_hbm    algorithmic HBM bytes of the AllReduce (5 D (P-1)) / t / 8 TB/s
  roofline   the ring reduce-scatter step kernel: algorithmic bytes per launch
             (3 bytes per segment byte, 8 segments) / its mean duration from
             HIP events recorded between the steps on the launch stream
  cpu_baseline  the CPU oracle replaying the same AllReduce (single thread)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s


def measured_traffic():
    """HBM bytes per launch of the ring reduce step from the committed counter
    summary, or None once the kernel source differs from the one measured."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "ring_rs_step_p8_fp32_64Mi_hbm_traffic.md")
    src = b"".join(open(os.path.join(ROOT, "allreduce_reduction_amd", "csrc", f), "rb").read()
                   for f in ("step_kernels.hip", "launch.hpp"))
    digest = hashlib.sha256(src).hexdigest()[:16]
    try:
        kv = dict(line.strip().split(": ", 1) for line in open(path, encoding="utf-8")
                  if line.strip().startswith(("traffic_bytes_per_launch:", "kernel_source_sha256_16:")))
    except OSError:
        return None
    if kv.get("kernel_source_sha256_16") != digest:
        return None
    return int(kv["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--P", type=int, default=8)
    ap.add_argument("--elems", type=int, default=64 << 20, help="elements per rank")
    ap.add_argument("--cpu-reps", type=int, default=4, help="oracle AllReduces timed for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--algo", default="ring", choices=["ring", "rhd"])
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (P logical ranks share its HBM); --gpus {a.gpus} "
              "is not supported", file=sys.stderr)
        sys.exit(2)
    if a.steps > 35:
        # values grow by P per AllReduce; 35 passes of x8 stay finite in fp32
        print("--steps above 35 would overflow the fp32 inputs; use at most 35", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import allreduce_reduction_amd as hc
    import synth

    P, L = a.P, a.elems
    dtype, e = "fp32", 4
    D = L * e
    dev = torch.device("cuda:0")
    recipe = synth.RECIPES["ring_p8_fp32_grad"]

    # inputs: generated on the host, resident in HBM before timing
    host = torch.empty(L, dtype=torch.float32).pin_memory()
    bufs = []
    for r in range(P):
        synth.fill_ptr(host.data_ptr(), dtype, L, recipe["dist"], recipe["p0"], recipe["p1"],
                       seed=0, stream=recipe["stream"], rank=r)
        bufs.append(host.to(dev, non_blocking=False).clone())
    torch.cuda.synchronize()

    comm = hc.Comm(P, a.algo)
    info = comm.plan_info("allreduce", L, dtype)
    nsteps = info["nsteps"]
    rs_steps = list(range(nsteps // 2)) if a.algo == "ring" else [s for s in range(nsteps)
                                                                   if comm.step_info("allreduce", L, dtype, s)["hbm_bytes"] > 0][:1]
    rs_bytes = comm.step_info("allreduce", L, dtype, rs_steps[0])["hbm_bytes"]
    stream = torch.cuda.current_stream()

    # warmup (whole AllReduces)
    for _ in range(a.warmup):
        comm.allreduce(bufs, dtype, "sum")
    torch.cuda.synchronize()

    # timed region: K AllReduces, each issued step by step with events between
    # the steps (same launches as hbmc_allreduce, plus event markers)
    K = a.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        for s in range(nsteps):
            ev[k][s].record(stream)
            comm.run_steps("allreduce", bufs, s, s + 1, dtype, "sum")
        ev[k][nsteps].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    wall = (t1 - t0) / K
    gpu_ms = [ev[k][0].elapsed_time(ev[k][nsteps]) for k in range(K)]
    t = float(np.median(gpu_ms)) / 1e3
    step_ms = np.array([[ev[k][s].elapsed_time(ev[k][s + 1]) for s in range(nsteps)] for k in range(K)])
    rs_ms = float(step_ms[:, rs_steps].mean())
    ag_steps = [s for s in range(nsteps) if s not in rs_steps]
    ag_ms = float(step_ms[:, ag_steps].mean()) if ag_steps and a.algo == "ring" else None

    algbw = D / t
    busbw = algbw * 2 * (P - 1) / P
    achieved = rs_bytes / (rs_ms / 1e3)

    out = {
        "metric": "AllReduce busbw GB/s on 1 GPU (P simulated ranks) + % of HBM peak",
        "value": round(busbw / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(t * 1e3, 4),
        "wall_ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{a.algo} allreduce sum, P={P} ranks x {L} fp32 elements "
                               f"({D >> 20} MiB/rank), N(0,1e-3)",
                   "P": P, "elems_per_rank": L, "algo": a.algo, "kernel_launches": nsteps},
        "algbw_GBps": round(algbw / 1e9, 3),
        "pct_hbm": round(100 * info["hbm_bytes"] / t / HBM_PEAK, 2),
        "roofline": {"bound": "hbm", "kernel": "step_vec<fp32,sum,recv_fold,2,1> (ring reduce step)",
                     "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": measured_traffic() if (P, L, a.algo) == (8, 64 << 20, "ring") else None,
                     "bytes_per_launch": rs_bytes, "mean_launch_us": round(rs_ms * 1e3, 2)},
    }
    if ag_ms:
        ag_bytes = comm.step_info("allreduce", L, dtype, ag_steps[0])["hbm_bytes"]
        out["copy_step"] = {"kernel": "step_vec<fp32,copy,1,1> (ring all-gather step)",
                            "mean_launch_us": round(ag_ms * 1e3, 2),
                            "achieved_GBps": round(ag_bytes / (ag_ms / 1e3) / 1e9, 1)}

    if not a.no_cpu:
        import oracle
        xs = [np.empty(L, np.float32) for _ in range(P)]
        times = []
        for rep in range(a.cpu_reps):
            for r in range(P):
                synth.fill_ptr(xs[r].ctypes.data, dtype, L, recipe["dist"], recipe["p0"], recipe["p1"],
                               seed=0, stream=recipe["stream"], rank=r)
            c0 = time.perf_counter()
            oracle.run("allreduce", a.algo, xs, dtype, "sum")
            times.append(time.perf_counter() - c0)
        tc = float(np.median(times))
        out["cpu_baseline"] = {"value": round(D / tc * 2 * (P - 1) / P / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the full workload, {a.cpu_reps} AllReduces replayed by the "
                                         f"single-threaded oracle, median {tc:.2f} s each"}
    comm.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
