"""Python binding of the hbmcoll C ABI (``include/hbmcoll.h``).

Argument marshalling only: every step of a collective runs in the gfx950
kernels of ``libhbmcoll.so``.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhbmcoll.so")

OK = 0
STATUS = {0: "HBMC_OK", 1: "HBMC_ERR_INVALID_ARG", 2: "HBMC_ERR_UNSUPPORTED", 3: "HBMC_ERR_HIP",
          4: "HBMC_ERR_NOMEM", 5: "HBMC_ERR_SCRATCH"}
DTYPE = {"fp32": 0, "fp16": 1, "bf16": 2, "int32": 3, "int8": 4}
ESIZE = {"fp32": 4, "fp16": 2, "bf16": 2, "int32": 4, "int8": 1}
OP = {"sum": 0, "prod": 1, "max": 2, "min": 3}
ALGO = {"ring": 0, "rhd": 1, "pipeline": 2, "env": 3, "flat": 4, "tree": 5, "hier": 6, "auto": 7,
        "auto_rules": 8}
ALGO_NAME = {v: k for k, v in ALGO.items()}
COLL = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2, "reduce": 3, "broadcast": 4}
MODE = {0: "copy", 1: "fold", 2: "recv_fold"}
EXEC = {"auto": 0, "steps": 1, "fused": 2, "columns": 3, "lds": 4, "regs": 5, "flow": 6}
_EXEC_NAME = {v: k for k, v in EXEC.items()}

# every symbol include/hbmcoll.h declares
EXPORTS = ("hbmc_comm_create", "hbmc_comm_destroy", "hbmc_allreduce", "hbmc_reduce_scatter",
           "hbmc_all_gather", "hbmc_reduce", "hbmc_broadcast", "hbmc_collective_oop", "hbmc_run_steps", "hbmc_plan_info", "hbmc_plan_step_info",
           "hbmc_plan_items", "hbmc_status_string", "hbmc_graph_create", "hbmc_graph_add",
           "hbmc_graph_build", "hbmc_graph_launch", "hbmc_graph_destroy", "hbmc_comm_set_cost_model",
           "hbmc_auto_choice", "hbmc_comm_set_fused_limit",
           "hbmc_comm_set_columns", "hbmc_plan_chunks",
           "hbmc_comm_set_exec_mode", "hbmc_exec_choice", "hbmc_exec_bytes", "hbmc_allreduce_noalloc",
           "hbmc_comm_set_flow", "hbmc_comm_flow_timeouts", "hbmc_plan_flow")


class HbmcError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        msg = STATUS.get(code, str(code))
        try:
            msg += ": " + load_library().hbmc_status_string(code).decode()
        except Exception:  # noqa: BLE001 - the code is still reported
            pass
        super().__init__(f"{what}: {msg}" if what else msg)
        self.code = code


class Item(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("mode", ctypes.c_int32), ("nsrc", ctypes.c_int32),
                ("ndst", ctypes.c_int32), ("begin", ctypes.c_uint64), ("count", ctypes.c_uint64),
                ("rank", ctypes.c_uint8 * 128)]


class Chunk(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_uint64), ("count", ctypes.c_uint32), ("item", ctypes.c_uint32),
                ("step", ctypes.c_uint32), ("dep_lo", ctypes.c_uint32), ("dep_hi", ctypes.c_uint32),
                ("pad", ctypes.c_uint32)]


class FlowTile(ctypes.Structure):
    _fields_ = [("col", ctypes.c_uint32), ("seq", ctypes.c_uint32), ("step", ctypes.c_uint32),
                ("c_lo", ctypes.c_uint32), ("c_hi", ctypes.c_uint32), ("pad", ctypes.c_uint32)]


class FlowChunk(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_uint64), ("count", ctypes.c_uint32), ("item", ctypes.c_uint32)]


_lib = None


def load_library():
    """Load ``libhbmcoll.so`` (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, ci, u64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64)
        L.hbmc_comm_create.restype = ci
        L.hbmc_comm_create.argtypes = [ci, ci, ci, ci, sz, ctypes.POINTER(vp)]
        L.hbmc_comm_destroy.restype = ci
        L.hbmc_comm_destroy.argtypes = [vp]
        for name in ("hbmc_allreduce", "hbmc_reduce_scatter", "hbmc_all_gather", "hbmc_allreduce_noalloc"):
            f = getattr(L, name)
            f.restype = ci
            f.argtypes = [vp, ctypes.POINTER(vp), sz, ci, ci, vp]
        L.hbmc_reduce.restype = ci
        L.hbmc_reduce.argtypes = [vp, ctypes.POINTER(vp), sz, ci, ci, ci, vp]
        L.hbmc_broadcast.restype = ci
        L.hbmc_broadcast.argtypes = [vp, ctypes.POINTER(vp), sz, ci, ci, vp]
        L.hbmc_collective_oop.restype = ci
        L.hbmc_collective_oop.argtypes = [vp, ci, ci, ctypes.POINTER(vp), ctypes.POINTER(vp), sz, ci, ci, vp]
        L.hbmc_run_steps.restype = ci
        L.hbmc_run_steps.argtypes = [vp, ci, ci, ctypes.POINTER(vp), sz, ci, ci, ci, ci, vp]
        L.hbmc_plan_info.restype = ci
        L.hbmc_plan_info.argtypes = [vp, ci, ci, sz, ci, ctypes.POINTER(ci), u64p, u64p]
        L.hbmc_plan_step_info.restype = ci
        L.hbmc_plan_step_info.argtypes = [vp, ci, ci, sz, ci, ci, ctypes.POINTER(ci), u64p]
        L.hbmc_plan_items.restype = ci
        L.hbmc_plan_items.argtypes = [vp, ci, ci, sz, ci, ctypes.POINTER(Item), sz, ctypes.POINTER(sz)]
        L.hbmc_plan_chunks.restype = ci
        L.hbmc_plan_chunks.argtypes = [vp, ci, ci, sz, ci, ctypes.c_uint64, ctypes.POINTER(Chunk), sz,
                                       ctypes.POINTER(sz), ctypes.POINTER(ctypes.c_uint32), sz, ctypes.POINTER(sz)]
        L.hbmc_graph_create.restype = ci
        L.hbmc_graph_create.argtypes = [ctypes.POINTER(vp)]
        L.hbmc_graph_add.restype = ci
        L.hbmc_graph_add.argtypes = [vp, vp, ci, ci, ctypes.POINTER(vp), sz, ci, ci]
        L.hbmc_graph_build.restype = ci
        L.hbmc_graph_build.argtypes = [vp]
        L.hbmc_graph_launch.restype = ci
        L.hbmc_graph_launch.argtypes = [vp, vp]
        L.hbmc_graph_destroy.restype = ci
        L.hbmc_graph_destroy.argtypes = [vp]
        L.hbmc_comm_set_fused_limit.restype = ci
        L.hbmc_comm_set_fused_limit.argtypes = [vp, ctypes.c_uint64]
        L.hbmc_comm_set_columns.restype = ci
        L.hbmc_comm_set_columns.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint64]
        L.hbmc_comm_set_flow.restype = ci
        L.hbmc_comm_set_flow.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_uint32]
        L.hbmc_comm_flow_timeouts.restype = ci
        L.hbmc_comm_flow_timeouts.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
        L.hbmc_plan_flow.restype = ci
        L.hbmc_plan_flow.argtypes = [vp, ci, ci, sz, ci, ci, ci, ctypes.c_uint64, ctypes.POINTER(FlowTile), sz,
                                     ctypes.POINTER(sz), ctypes.POINTER(FlowChunk), sz, ctypes.POINTER(sz)]
        L.hbmc_comm_set_exec_mode.restype = ci
        L.hbmc_comm_set_exec_mode.argtypes = [vp, ci]
        L.hbmc_exec_choice.restype = ci
        L.hbmc_exec_choice.argtypes = [vp, ci, ci, sz, ci, ci, ci, ctypes.POINTER(ci)]
        L.hbmc_exec_bytes.restype = ci
        L.hbmc_exec_bytes.argtypes = [vp, ci, ci, sz, ci, ci, ci, ci, u64p]
        L.hbmc_comm_set_cost_model.restype = ci
        L.hbmc_comm_set_cost_model.argtypes = [vp, ctypes.c_double, ctypes.c_double]
        L.hbmc_auto_choice.restype = ci
        L.hbmc_auto_choice.argtypes = [vp, ci, ci, sz, ci, ctypes.POINTER(ci)]
        L.hbmc_status_string.restype = ctypes.c_char_p
        L.hbmc_status_string.argtypes = [ci]
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise HbmcError(rc, what)


_TORCH_DTYPES = None


def _torch_dtypes():
    global _TORCH_DTYPES
    if _TORCH_DTYPES is None:
        import torch
        _TORCH_DTYPES = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16",
                         torch.int32: "int32", torch.int8: "int8"}
    return _TORCH_DTYPES


def _torch_dtype_name(t) -> str:
    name = _torch_dtypes().get(t.dtype)
    if name is None:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return name


def _ptrs(bufs):
    """(void*[P], count, dtype) from a list of device tensors or raw addresses."""
    P = len(bufs)
    if P and hasattr(bufs[0], "data_ptr"):
        b0 = bufs[0]
        dt = _torch_dtype_name(b0)
        t0, n = b0.dtype, b0.numel()
        addrs = []
        for b in bufs:
            if not hasattr(b, "data_ptr"):
                raise TypeError("buffers must be all tensors or all raw device addresses")
            if b.dtype != t0 or not b.is_cuda or not b.is_contiguous() or b.numel() != n:
                raise ValueError("buffers must be contiguous device tensors of one dtype and size")
            addrs.append(b.data_ptr())
        return (ctypes.c_void_p * P)(*addrs), n, dt
    arr = (ctypes.c_void_p * max(P, 1))()
    for i, b in enumerate(bufs):
        arr[i] = int(b)
    return arr, None, None


def _args(bufs, dtype, count):
    """(void*[P], count, dtype name) for a call: count and dtype default to
    the tensors'; raw addresses need both given."""
    arr, n, dt = _ptrs(bufs)
    dtype = dtype or dt
    count = n if count is None else count
    if count is None or dtype is None:
        raise ValueError("raw device addresses need an explicit count and dtype")
    return arr, count, dtype


_RAW_STREAM = None


def _stream(stream) -> int:
    """The stream handle: the given torch stream or raw handle, else the
    current device's current torch stream."""
    global _RAW_STREAM
    if stream is None:
        import torch
        if _RAW_STREAM is None:
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            _RAW_STREAM = (lambda: raw(torch.cuda.current_device())) if raw else \
                (lambda: torch.cuda.current_stream().cuda_stream)
        return _RAW_STREAM()
    return int(getattr(stream, "cuda_stream", stream))


class Comm:
    """A communicator of P logical ranks (P buffers on one GPU)."""

    def __init__(self, nranks: int, algo: str = "ring", servers: int = 0, ranks_per_server: int = 0,
                 loop_bytes: int = 0):
        self.P = nranks
        self.algo = algo
        self.S, self.M = servers, ranks_per_server
        self._h = ctypes.c_void_p()
        _check(load_library().hbmc_comm_create(nranks, ALGO[algo], servers, ranks_per_server, loop_bytes,
                                               ctypes.byref(self._h)), "hbmc_comm_create")

    # -- lifetime
    def close(self) -> None:
        if self._h:
            _check(load_library().hbmc_comm_destroy(self._h), "hbmc_comm_destroy")
            self._h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- collectives
    def _coll(self, fn, bufs, dtype, op, count, stream):
        arr, count, dtype = _args(bufs, dtype, count)
        _check(getattr(load_library(), fn)(self._h, arr, count, DTYPE[dtype], OP[op], _stream(stream)), fn)

    def allreduce(self, bufs, dtype=None, op="sum", *, count=None, stream=None):
        self._coll("hbmc_allreduce", bufs, dtype, op, count, stream)

    def allreduce_noalloc(self, bufs, dtype=None, op="sum", *, count=None, stream=None):
        """AllReduce whose kernels take their tables from the library's fixed
        device array (no device allocation; see hbmc_allreduce_noalloc)."""
        self._coll("hbmc_allreduce_noalloc", bufs, dtype, op, count, stream)

    def reduce_scatter(self, bufs, dtype=None, op="sum", *, count=None, stream=None):
        self._coll("hbmc_reduce_scatter", bufs, dtype, op, count, stream)

    def all_gather(self, bufs, dtype=None, op="sum", *, count=None, stream=None):
        self._coll("hbmc_all_gather", bufs, dtype, op, count, stream)

    def reduce(self, bufs, dtype=None, op="sum", *, root=0, count=None, stream=None):
        arr, count, dtype = _args(bufs, dtype, count)
        _check(load_library().hbmc_reduce(self._h, arr, count, DTYPE[dtype], OP[op], root, _stream(stream)),
               "hbmc_reduce")

    def broadcast(self, bufs, dtype=None, *, root=0, count=None, stream=None):
        arr, count, dtype = _args(bufs, dtype, count)
        _check(load_library().hbmc_broadcast(self._h, arr, count, DTYPE[dtype], root, _stream(stream)),
               "hbmc_broadcast")

    def out_of_place(self, coll, send, recv, dtype=None, op="sum", *, root=0, count=None, stream=None):
        """Collective from `send` into `recv` (LocalCopy first where they differ)."""
        sarr, n, dt = _ptrs(send)
        rarr, n2, dt2 = _ptrs(recv)
        if n is not None and (n != n2 or dt != dt2):
            raise ValueError("send and recv must match in size and dtype")
        dtype = dtype or dt
        count = n if count is None else count
        if count is None or dtype is None:
            raise ValueError("raw device addresses need an explicit count and dtype")
        _check(load_library().hbmc_collective_oop(self._h, COLL[coll], root, sarr, rarr, count, DTYPE[dtype],
                                                  OP[op], _stream(stream)), "hbmc_collective_oop")

    def run_steps(self, coll, bufs, first, last, dtype=None, op="sum", *, root=0, count=None, stream=None):
        arr, count, dtype = _args(bufs, dtype, count)
        _check(load_library().hbmc_run_steps(self._h, COLL[coll], root, arr, count, DTYPE[dtype], OP[op],
                                             first, last, _stream(stream)), "hbmc_run_steps")

    def set_exec_mode(self, mode: str):
        """Launch form of every call: "auto" (default), "steps", "fused", "columns", "lds", "regs" or
        "flow"."""
        _check(load_library().hbmc_comm_set_exec_mode(self._h, EXEC[mode]), "hbmc_comm_set_exec_mode")

    def exec_choice(self, coll: str, count: int, dtype: str, root: int = 0, first: int = 0, last: int = 0) -> str:
        """Launch form a call (or steps [first, last)) would take, host only."""
        m = ctypes.c_int()
        _check(load_library().hbmc_exec_choice(self._h, COLL[coll], root, count, DTYPE[dtype], first, last,
                                               ctypes.byref(m)), "hbmc_exec_choice")
        return _EXEC_NAME[m.value]

    def exec_bytes(self, coll: str, count: int, dtype: str, mode: str = "auto", root: int = 0,
                   first: int = 0, last: int = 0) -> int:
        """Bytes a call (or steps [first, last)) moves to and from memory in a
        launch form (see hbmc_exec_bytes), host only."""
        b = ctypes.c_uint64()
        _check(load_library().hbmc_exec_bytes(self._h, COLL[coll], root, count, DTYPE[dtype], first, last,
                                              EXEC[mode], ctypes.byref(b)), "hbmc_exec_bytes")
        return b.value

    def set_flow(self, tile_bytes: int = 16 << 10, wgs_per_cu: int = 8, tiles_per_ticket: int = 1,
                 wait_us: int = 1_000_000, unreachable: bool = False):
        """Flow form: tile length per rank buffer, workgroups per compute unit,
        tiles per ticket, bound on each wait (us); `unreachable` makes every
        wait give up (a test of the give-up path)."""
        _check(load_library().hbmc_comm_set_flow(self._h, tile_bytes, wgs_per_cu, tiles_per_ticket, wait_us,
                                                 1 if unreachable else 0), "hbmc_comm_set_flow")

    def flow_timeouts(self) -> int:
        """Flow-form waits that gave up since the last call (then reset; waits for the device)."""
        n = ctypes.c_uint32()
        _check(load_library().hbmc_comm_flow_timeouts(self._h, ctypes.byref(n)), "hbmc_comm_flow_timeouts")
        return n.value

    def set_fused_limit(self, max_bytes: int):
        """Single-workgroup form eligible for calls moving at most max_bytes."""
        _check(load_library().hbmc_comm_set_fused_limit(self._h, max_bytes), "hbmc_comm_set_fused_limit")

    def set_columns(self, max_total_bytes: int, column_bytes: int = 0):
        """Column form eligible for calls over at most max_total_bytes (P * count * e);
        column_bytes 0 picks the column length."""
        _check(load_library().hbmc_comm_set_columns(self._h, max_total_bytes, column_bytes),
               "hbmc_comm_set_columns")

    # -- AUTO selection (host only)
    def set_cost_model(self, alpha_us: float, beta_gbps: float):
        _check(load_library().hbmc_comm_set_cost_model(self._h, alpha_us, beta_gbps), "hbmc_comm_set_cost_model")

    def auto_choice(self, coll: str, count: int, dtype: str, root: int = 0) -> str:
        a = ctypes.c_int()
        _check(load_library().hbmc_auto_choice(self._h, COLL[coll], root, count, DTYPE[dtype], ctypes.byref(a)),
               "hbmc_auto_choice")
        return ALGO_NAME[a.value]

    # -- schedule facts (host only)
    def plan_info(self, coll: str, count: int, dtype: str, root: int = 0):
        n = ctypes.c_int()
        b = ctypes.c_uint64()
        r = ctypes.c_uint64()
        _check(load_library().hbmc_plan_info(self._h, COLL[coll], root, count, DTYPE[dtype], ctypes.byref(n),
                                             ctypes.byref(b), ctypes.byref(r)), "hbmc_plan_info")
        return dict(nsteps=n.value, hbm_bytes=b.value, max_recv_bytes=r.value)

    def step_info(self, coll: str, count: int, dtype: str, step: int, root: int = 0):
        n = ctypes.c_int()
        b = ctypes.c_uint64()
        _check(load_library().hbmc_plan_step_info(self._h, COLL[coll], root, count, DTYPE[dtype], step,
                                                  ctypes.byref(n), ctypes.byref(b)), "hbmc_plan_step_info")
        return dict(nitems=n.value, hbm_bytes=b.value)

    def plan_items(self, coll: str, count: int, dtype: str, root: int = 0):
        n = ctypes.c_size_t()
        L = load_library()
        _check(L.hbmc_plan_items(self._h, COLL[coll], root, count, DTYPE[dtype], None, 0, ctypes.byref(n)),
               "hbmc_plan_items")
        arr = (Item * max(n.value, 1))()
        _check(L.hbmc_plan_items(self._h, COLL[coll], root, count, DTYPE[dtype], arr, n.value,
                                 ctypes.byref(n)), "hbmc_plan_items")
        out = []
        for it in arr[:n.value]:
            ranks = list(it.rank[:it.nsrc + it.ndst])
            out.append(dict(step=it.step, mode=MODE[it.mode], begin=it.begin, count=it.count,
                            src=ranks[:it.nsrc], dst=ranks[it.nsrc:]))
        return out

    def plan_chunks(self, coll: str, count: int, dtype: str, chunk_bytes: int, root: int = 0):
        """Column-kernel chunks (dicts: begin, count, item, step, deps) of a collective (host only)."""
        L = load_library()
        n, nd = ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.hbmc_plan_chunks(self._h, COLL[coll], root, count, DTYPE[dtype], chunk_bytes, None, 0,
                                  ctypes.byref(n), None, 0, ctypes.byref(nd)), "hbmc_plan_chunks")
        arr = (Chunk * max(n.value, 1))()
        deps = (ctypes.c_uint32 * max(nd.value, 1))()
        _check(L.hbmc_plan_chunks(self._h, COLL[coll], root, count, DTYPE[dtype], chunk_bytes, arr, n.value,
                                  ctypes.byref(n), deps, nd.value, ctypes.byref(nd)), "hbmc_plan_chunks")
        return [dict(begin=c.begin, count=c.count, item=c.item, step=c.step, deps=list(deps[c.dep_lo:c.dep_hi]))
                for c in arr[:n.value]]

    def plan_flow(self, coll: str, count: int, dtype: str, tile_bytes: int, root: int = 0, first: int = 0,
                  last: int = -1):
        """Flow-kernel tables of steps [first, last) (host only): tiles in ticket
        order (dicts: col, seq, step, chunks) and chunks (dicts: begin, count,
        item)."""
        L = load_library()
        nt, nc = ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.hbmc_plan_flow(self._h, COLL[coll], root, count, DTYPE[dtype], first, last, tile_bytes, None, 0,
                                ctypes.byref(nt), None, 0, ctypes.byref(nc)), "hbmc_plan_flow")
        tiles = (FlowTile * max(nt.value, 1))()
        chunks = (FlowChunk * max(nc.value, 1))()
        _check(L.hbmc_plan_flow(self._h, COLL[coll], root, count, DTYPE[dtype], first, last, tile_bytes, tiles,
                                nt.value, ctypes.byref(nt), chunks, nc.value, ctypes.byref(nc)), "hbmc_plan_flow")
        return ([dict(col=t.col, seq=t.seq, step=t.step, chunks=range(t.c_lo, t.c_hi)) for t in tiles[:nt.value]],
                [dict(begin=c.begin, count=c.count, item=c.item) for c in chunks[:nc.value]])


class Graph:
    """Graph mode: add collectives, build once, launch many times."""

    def __init__(self):
        self._h = ctypes.c_void_p()
        self._keep = []  # buffer-pointer arrays stay alive with the graph
        _check(load_library().hbmc_graph_create(ctypes.byref(self._h)), "hbmc_graph_create")

    def add(self, comm: Comm, coll: str, bufs, dtype=None, op="sum", *, root=0, count=None):
        arr, count, dtype = _args(bufs, dtype, count)
        self._keep.append((arr, list(bufs)))
        _check(load_library().hbmc_graph_add(self._h, comm._h, COLL[coll], root, arr, count, DTYPE[dtype],
                                             OP[op]), "hbmc_graph_add")

    def build(self):
        _check(load_library().hbmc_graph_build(self._h), "hbmc_graph_build")

    def launch(self, stream=None):
        _check(load_library().hbmc_graph_launch(self._h, _stream(stream)), "hbmc_graph_launch")

    def close(self):
        if self._h:
            _check(load_library().hbmc_graph_destroy(self._h), "hbmc_graph_destroy")
            self._h = ctypes.c_void_p()
            self._keep = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
