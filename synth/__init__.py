"""Seeded synthetic inputs (counter-based, regenerable by window).

Shared by the oracle's tests and the GPU path's tests and bench; holds no part
of the reduction.  The generator is a C library (``libsynth.so``) built next to
this file; see ``synth.c`` for the definition of every draw.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2, "int32": 3, "int8": 4}
# numpy storage type for each element type; bf16 is carried as raw uint16 bits
NP_STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16,
              "int32": np.int32, "int8": np.int8}
ESIZE = {"fp32": 4, "fp16": 2, "bf16": 2, "int32": 4, "int8": 1}

UNIFORM_INT = 0
NORMAL = 1

# Input recipes of the five workloads: (element type, distribution, p0, p1).
# ``stream`` keys a workload's sequence so two workloads never share values.
RECIPES = {
    # ring AllReduce, P=4, L=4096, integers U{-8..8} stored as fp32
    "ring_p4_fp32_int": dict(dtype="fp32", dist=UNIFORM_INT, p0=-8.0, p1=8.0, stream=1),
    # ring AllReduce, P=8, L=64Mi, gradient-like fp32 N(0, 1e-3)
    "ring_p8_fp32_grad": dict(dtype="fp32", dist=NORMAL, p0=1e-3, p1=0.0, stream=2),
    # RHD AllReduce, P in {8,5}, 1..64 KiB per rank: bf16 N(0,1) and int32 U[-2^20, 2^20]
    "rhd_bf16_normal": dict(dtype="bf16", dist=NORMAL, p0=1.0, p1=0.0, stream=3),
    "rhd_int32_uniform": dict(dtype="int32", dist=UNIFORM_INT, p0=-(2.0 ** 20), p1=2.0 ** 20, stream=4),
    # ring vs RHD sweep, P=16, fp16 N(0, 0.01)
    "sweep_p16_fp16": dict(dtype="fp16", dist=NORMAL, p0=0.01, p1=0.0, stream=5),
    # two-level pipeline, 4 servers x 8 ranks, bf16 N(0, 1e-2)
    "pipe_4x8_bf16": dict(dtype="bf16", dist=NORMAL, p0=1e-2, p1=0.0, stream=6),
}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int]
        _lib = lib
    return _lib


def _threads(nthreads):
    if nthreads is not None:
        return int(nthreads)
    return max(1, min(16, len(os.sched_getaffinity(0))))


def fill_ptr(ptr: int, dtype: str, n: int, dist: int, p0: float, p1: float = 0.0, *,
             seed: int = 0, stream: int = 0, rank: int = 0, first: int = 0,
             nthreads: int | None = None) -> None:
    """Write elements ``first .. first+n-1`` of one rank's sequence to host memory at ``ptr``."""
    rc = _load().synth_fill(ctypes.c_void_p(ptr), DTYPE_CODE[dtype], int(dist), float(p0), float(p1),
                            int(seed), int(stream), int(rank), int(first), int(n), _threads(nthreads))
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")


def generate(dtype: str, n: int, dist: int, p0: float, p1: float = 0.0, *, seed: int = 0,
             stream: int = 0, rank: int = 0, first: int = 0,
             nthreads: int | None = None) -> np.ndarray:
    """Return elements ``first .. first+n-1`` of one rank's sequence as a numpy array."""
    out = np.empty(int(n), dtype=NP_STORAGE[dtype])
    if n:
        fill_ptr(out.ctypes.data, dtype, n, dist, p0, p1, seed=seed, stream=stream, rank=rank,
                 first=first, nthreads=nthreads)
    return out


def rank_inputs(recipe: str, P: int, L: int, *, seed: int = 0, first: int = 0,
                n: int | None = None) -> list[np.ndarray]:
    """Inputs of all P ranks for a named recipe (elements ``first .. first+n-1``)."""
    r = RECIPES[recipe]
    n = L - first if n is None else n
    return [generate(r["dtype"], n, r["dist"], r["p0"], r["p1"], seed=seed, stream=r["stream"],
                     rank=k, first=first) for k in range(P)]
