"""Independent element ops for pinning the oracle (numpy / torch library arithmetic).

These never call the oracle.  binary16 arithmetic is numpy's float16 (its
loops widen to binary32, operate, and round to nearest even), bfloat16 is
torch's CPU bfloat16 arithmetic (same scheme), binary32 is numpy float32,
integers wrap in numpy.  max/min follow the reading that NaN in either operand
gives the canonical quiet NaN and that -0 orders below +0.
"""
from __future__ import annotations

import numpy as np
import torch

STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16,
           "int32": np.int32, "int8": np.int8}
CANON_NAN = {"fp32": np.uint32(0x7FC00000), "fp16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
FLOATS = ("fp32", "fp16", "bf16")
INTS = ("int32", "int8")


def to_f64(dtype: str, x: np.ndarray) -> np.ndarray:
    """Exact widening of storage arrays to float64 (library conversions)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return np.asarray(x).astype(np.float64)


def from_f32(dtype: str, x: np.ndarray) -> np.ndarray:
    """binary32 -> storage, round to nearest even (library conversions)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x.copy()
    if dtype == "fp16":
        return x.astype(np.float16)
    t = torch.from_numpy(x.copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits(dtype, x):
    return np.ascontiguousarray(x).view(np.uint32 if dtype == "fp32" else np.uint16)


def _maxmin(dtype, op, a, b):
    fa, fb = to_f64(dtype, a), to_f64(dtype, b)
    nan = np.isnan(fa) | np.isnan(fb)
    if op == "max":
        pick_b = (fb > fa) | ((fa == fb) & np.signbit(fa) & ~np.signbit(fb))
    else:
        pick_b = (fb < fa) | ((fa == fb) & ~np.signbit(fa) & np.signbit(fb))
    ab, bb = _bits(dtype, a), _bits(dtype, b)
    out = np.where(pick_b, bb, ab)
    out = np.where(nan, CANON_NAN[dtype], out)
    return out.astype(ab.dtype).view(STORAGE[dtype])


def combine(dtype: str, op: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=STORAGE[dtype])
    b = np.ascontiguousarray(b, dtype=STORAGE[dtype])
    if dtype in INTS:
        if op == "sum":
            return (a + b).astype(STORAGE[dtype])
        if op == "prod":
            return (a * b).astype(STORAGE[dtype])
        return np.maximum(a, b) if op == "max" else np.minimum(a, b)
    if op in ("max", "min"):
        return _maxmin(dtype, op, a, b)
    with np.errstate(all="ignore"):
        if dtype in ("fp32", "fp16"):
            return (a + b) if op == "sum" else (a * b)
        ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
        tc = (ta + tb) if op == "sum" else (ta * tb)
        return tc.view(torch.int16).numpy().view(np.uint16).copy()


def same(dtype: str, x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Elementwise bit equality, with any two NaNs counted equal."""
    x = np.ascontiguousarray(x, dtype=STORAGE[dtype])
    y = np.ascontiguousarray(y, dtype=STORAGE[dtype])
    if dtype in INTS:
        return x == y
    eq = _bits(dtype, x) == _bits(dtype, y)
    return eq | (np.isnan(to_f64(dtype, x)) & np.isnan(to_f64(dtype, y)))


def assert_same(dtype: str, x: np.ndarray, y: np.ndarray, what: str = "") -> None:
    ok = same(dtype, x, y)
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} differ; first at {i}: "
                             f"{np.asarray(x).ravel()[i]!r} vs {np.asarray(y).ravel()[i]!r}")


def seg_bounds(n: int, m: int, k: int) -> tuple[int, int]:
    """Ceiling split of n into m parts: part k."""
    q = -(-n // m) if m else 0
    return min(k * q, n), min((k + 1) * q, n)


def unit_roundoff(dtype: str) -> float:
    return {"fp32": 2.0 ** -24, "fp16": 2.0 ** -11, "bf16": 2.0 ** -8}[dtype]


def min_subnormal(dtype: str) -> float:
    return {"fp32": 2.0 ** -149, "fp16": 2.0 ** -24, "bf16": 2.0 ** -133}[dtype]


def sum_bound_ok(dtype: str, y: np.ndarray, xs: list[np.ndarray]) -> np.ndarray:
    """Per-element error bound of a P-term sum rounded after every addition:
    |Y - Y64| <= gamma_{P-1} * sum|X_i| + (P-1) * eta, gamma_n = n u / (1 - n u)."""
    P = len(xs)
    u = unit_roundoff(dtype)
    n = max(P - 1, 0)
    gamma = n * u / (1 - n * u)
    X = np.stack([to_f64(dtype, x) for x in xs])
    exact = X.sum(axis=0)
    absum = np.abs(X).sum(axis=0)
    yv = to_f64(dtype, y)
    err = np.abs(yv - exact)
    tol = gamma * absum + n * 0.5 * min_subnormal(dtype)
    finite = np.isfinite(exact) & np.isfinite(yv)
    return ~finite | (err <= tol)
