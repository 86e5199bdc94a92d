"""ctypes binding of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg import this package.  The library (``liboracle.so``) is plain C built from
``oracle.c`` next to this file; see ``oracle.h`` for what each call computes
and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE = {"fp32": 0, "fp16": 1, "bf16": 2, "int32": 3, "int8": 4}
OP = {"sum": 0, "prod": 1, "max": 2, "min": 3}
ALGO = {"ring": 0, "rhd": 1, "pipeline": 2, "flat": 3, "tree": 4, "hier": 5}
COLL = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2, "reduce": 3, "broadcast": 4}
KIND = {0: "copy", 1: "reduce", 2: "fold", 3: "fold_recv"}
NP_STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16,
              "int32": np.int32, "int8": np.int8}

OK, EINVAL, EUNSUPPORTED, ENOMEM, ECONFLICT = 0, -1, -2, -3, -4


class TraceRec(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("kind", ctypes.c_int32), ("dst", ctypes.c_int32),
                ("src", ctypes.c_int32), ("slot", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("begin", ctypes.c_uint64), ("count", ctypes.c_uint64)]


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle returned {code}")
        self.code = code


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_round_f32.restype = ci
        L.orc_round_f32.argtypes = [ci, vp, vp, sz]
        L.orc_widen.restype = ci
        L.orc_widen.argtypes = [ci, vp, vp, sz]
        L.orc_combine.restype = ci
        L.orc_combine.argtypes = [ci, ci, vp, vp, vp, sz]
        L.orc_direct.restype = ci
        L.orc_direct.argtypes = [ci, ci, ci, ctypes.POINTER(vp), sz, vp, vp]
        L.orc_num_steps.restype = ctypes.c_long
        L.orc_num_steps.argtypes = [ci, ci, ci, ci, ci, sz, ci, sz]
        L.orc_collective.restype = ci
        L.orc_collective.argtypes = [ci, ci, ci, ci, ci, sz, ci, ctypes.POINTER(vp), sz, sz, sz, ci, ci,
                                     ctypes.c_long, ctypes.c_long, ctypes.POINTER(TraceRec), sz,
                                     ctypes.POINTER(sz)]
        _lib = L
    return _lib


def _check(rc):
    if rc != OK:
        raise OracleError(rc)


def round_f32(dtype: str, x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 / bfloat16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.uint16)
    _check(lib().orc_round_f32(DTYPE[dtype], x.ctypes.data, out.ctypes.data, x.size))
    return out


def widen(dtype: str, h: np.ndarray) -> np.ndarray:
    """binary16 / bfloat16 bit patterns -> binary32 (exact)."""
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.size, np.float32)
    _check(lib().orc_widen(DTYPE[dtype], h.ctypes.data, out.ctypes.data, h.size))
    return out


def combine(dtype: str, op: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Elementwise a (op) b in the element type (storage arrays)."""
    a = np.ascontiguousarray(a, dtype=NP_STORAGE[dtype])
    b = np.ascontiguousarray(b, dtype=NP_STORAGE[dtype])
    out = np.empty_like(a)
    _check(lib().orc_combine(DTYPE[dtype], OP[op], a.ctypes.data, b.ctypes.data, out.ctypes.data,
                             a.size))
    return out


def direct(dtype: str, op: str, xs: list[np.ndarray]) -> np.ndarray:
    """The definition: op over ranks per element, binary64 (floats) or wrapped int64 (ints)."""
    n = xs[0].size
    xs = [np.ascontiguousarray(x, dtype=NP_STORAGE[dtype]) for x in xs]
    ptrs = (ctypes.c_void_p * len(xs))(*[x.ctypes.data for x in xs])
    if dtype in ("int32", "int8"):
        out = np.empty(n, np.int64)
        _check(lib().orc_direct(DTYPE[dtype], OP[op], len(xs), ptrs, n, None, out.ctypes.data))
    else:
        out = np.empty(n, np.float64)
        _check(lib().orc_direct(DTYPE[dtype], OP[op], len(xs), ptrs, n, out.ctypes.data, None))
    return out


def num_steps(coll: str, algo: str, P: int, S: int = 1, M: int = 1) -> int:
    return int(lib().orc_num_steps(COLL[coll], ALGO[algo], P, S, M, 0, 0, 0))


def threads_available() -> int:
    """Host threads a parallel replay uses: the CPUs this process may run on,
    at most 16 (a single GPU's usual share of a multi-GPU host's cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_parallel(coll: str, algo: str, bufs: list[np.ndarray], dtype: str, op: str, *,
                 threads: int | None = None, S: int = 1, M: int = 1, loop_bytes: int = 0,
                 root: int = 0) -> int:
    """The whole replay of ``run`` (all steps, full vectors), as ``threads``
    windowed replays of disjoint element ranges run side by side.

    Every step combines the operands of an element at that element's own
    offset in each rank, so an element's result depends only on its values
    in every rank and on the segment / block / loop it lies in: each window,
    replayed with the full-size schedule, equals that window of the full
    replay (the windowed-replay pins hold this).  The arithmetic is the
    oracle's own, unchanged; ctypes releases the GIL for each call.  Returns
    the number of threads used."""
    from concurrent.futures import ThreadPoolExecutor

    P = len(bufs)
    n = bufs[0].size if P else 0
    T = threads_available() if threads is None else max(1, int(threads))
    T = max(1, min(T, n // 4096 if n >= 4096 else 1))
    if T == 1:
        run(coll, algo, bufs, dtype, op, S=S, M=M, loop_bytes=loop_bytes, root=root)
        return 1
    for b in bufs:
        if b.dtype != NP_STORAGE[dtype] or not b.flags.c_contiguous or b.size != n:
            raise ValueError("buffers must be contiguous storage arrays of one length")
    cuts = [n * k // T for k in range(T + 1)]

    def window(k):
        w0, w1 = cuts[k], cuts[k + 1]
        if w1 <= w0:
            return OK
        views = [b[w0:w1] for b in bufs]
        ptrs = (ctypes.c_void_p * P)(*[v.ctypes.data for v in views])
        tlen = ctypes.c_size_t(0)
        return lib().orc_collective(COLL[coll], ALGO[algo], P, S, M, loop_bytes, root, ptrs, n, w0, w1,
                                    DTYPE[dtype], OP[op], 0, -1, None, 0, ctypes.byref(tlen))

    with ThreadPoolExecutor(max_workers=T) as ex:
        codes = list(ex.map(window, range(T)))
    for rc in codes:
        _check(rc)
    return T


def run(coll: str, algo: str, bufs: list[np.ndarray], dtype: str, op: str, *, L: int | None = None,
        w0: int = 0, S: int = 1, M: int = 1, loop_bytes: int = 0, root: int = 0,
        first_step: int = 0, last_step: int = -1, trace: bool = False, trace_cap: int = 1 << 16):
    """Replay a collective in place on ``bufs`` (numpy storage arrays, one per rank).

    ``bufs[r]`` holds elements ``w0 .. w0+len-1`` of a vector of ``L`` elements
    per rank.  Returns the trace (list of dicts) when ``trace`` is set.
    """
    P = len(bufs)
    n = bufs[0].size if P else 0
    L = n + w0 if L is None else L
    for b in bufs:
        if b.dtype != NP_STORAGE[dtype] or not b.flags.c_contiguous or b.size != n:
            raise ValueError("buffers must be contiguous storage arrays of one length")
    ptrs = (ctypes.c_void_p * max(P, 1))(*[b.ctypes.data for b in bufs])
    recs = (TraceRec * trace_cap)() if trace else None
    tlen = ctypes.c_size_t(0)
    rc = lib().orc_collective(COLL[coll], ALGO[algo], P, S, M, loop_bytes, root, ptrs, L, w0, w0 + n,
                              DTYPE[dtype], OP[op], first_step, last_step, recs,
                              trace_cap if trace else 0, ctypes.byref(tlen))
    _check(rc)
    if not trace:
        return None
    if tlen.value > trace_cap:
        raise ValueError(f"trace needs {tlen.value} records")
    return [dict(step=r.step, kind=KIND[r.kind], dst=r.dst, src=r.src, slot=r.slot,
                 begin=r.begin, count=r.count) for r in recs[:tlen.value]]
