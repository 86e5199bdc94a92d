"""Pins of the oracle's conversions and element ops against library arithmetic.

The oracle's binary16 / bfloat16 conversions are written from the IEEE 754
formats; here they are compared with numpy's float16 and torch's bfloat16
conversions (both round to nearest even) on every 16-bit pattern, on every
tie between neighbouring 16-bit values, and on random binary32 patterns.
Its element ops (binary32 op, rounded back per operation; integer wrap;
ordered max/min with canonical NaN) are compared with numpy / torch arithmetic.
"""
import numpy as np
import pytest
import torch

import oracle
import refops

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _rand_f32_bits(n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_widen_every_pattern(dtype):
    got = oracle.widen(dtype, ALL16)
    want = refops.to_f64(dtype, ALL16.view(refops.STORAGE[dtype])).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_trip_every_pattern(dtype):
    back = oracle.round_f32(dtype, oracle.widen(dtype, ALL16))
    f = refops.to_f64(dtype, ALL16.view(refops.STORAGE[dtype]))
    ok = ~np.isnan(f)
    assert np.array_equal(back[ok], ALL16[ok])
    canon = 0x7E00 if dtype == "fp16" else 0x7FC0
    assert np.all((back[~ok] & 0x7FFF) == canon)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_every_tie(dtype):
    """Midpoints between neighbouring finite values must round to the even one."""
    vals = refops.to_f64(dtype, ALL16.view(refops.STORAGE[dtype]))
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    pos = np.unique(pos)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in binary32
    for sgn in (1.0, -1.0):
        m = (sgn * mids).astype(np.float32)
        got = oracle.round_f32(dtype, m)
        want = refops.from_f32(dtype, m).view(np.uint16)
        assert np.array_equal(got, want)
        # and the chosen neighbour has an even significand
        assert np.all((got & 1) == 0)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_random_patterns(dtype):
    x = _rand_f32_bits(400_000, 1)
    got = oracle.round_f32(dtype, x)
    want = refops.from_f32(dtype, x).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) if dtype == "fp16" else np.all((got[nan] & 0x7F80) == 0x7F80)


def test_fp16_overflow_and_underflow_edges():
    edges = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e9, 2.0 ** -24, 2.0 ** -25,
                      2.0 ** -25 * 1.0000001, 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12),
                      1e-40, 0.0, -0.0], np.float32)
    x = np.concatenate([edges, -edges])
    assert np.array_equal(oracle.round_f32("fp16", x), refops.from_f32("fp16", x).view(np.uint16))


def test_bf16_overflow_and_subnormal_edges():
    big = np.float32(np.finfo(np.float32).max)
    edges = np.array([big, 3.3895314e38, 3.4e38, 1e-38, 1e-40, 1e-45, 2.0 ** -133, 2.0 ** -134,
                      2.0 ** -126, 0.0, -0.0, np.inf], np.float32)
    x = np.concatenate([edges, -edges])
    assert np.array_equal(oracle.round_f32("bf16", x), refops.from_f32("bf16", x).view(np.uint16))


def _specials(dtype):
    if dtype == "fp32":
        v = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-38,
                      3.4e38, -3.4e38, 1.5, 2.5, 16777216.0, 1.0 + 2 ** -23], np.float32)
        return v
    if dtype == "fp16":
        return np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 6e-8, -6e-8, 6.1e-5,
                         65504, -65504, 1.5, 2049, 0.333], np.float16)
    if dtype == "bf16":
        f = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40, 1e-38, 3e38,
                      -3e38, 1.5, 257.0, 0.333], np.float32)
        return refops.from_f32("bf16", f)
    info = np.iinfo(refops.STORAGE[dtype])
    return np.array([0, 1, -1, info.max, info.min, info.max - 1, info.min + 1, 2, -2],
                    refops.STORAGE[dtype])


def _randvals(dtype, n, rng):
    if dtype == "fp32":
        a = rng.standard_normal(n).astype(np.float32) * np.float32(10.0) ** rng.integers(-40, 39, n).astype(np.float32)
        return a.astype(np.float32)
    if dtype == "fp16":
        return rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16).view(np.float16)
    if dtype == "bf16":
        return rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    info = np.iinfo(refops.STORAGE[dtype])
    return rng.integers(info.min, info.max + 1, n).astype(refops.STORAGE[dtype])


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16", "int32", "int8"])
@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
def test_combine_matches_library_arithmetic(dtype, op):
    rng = np.random.default_rng(7)
    sp = _specials(dtype)
    a = np.concatenate([np.repeat(sp, sp.size), _randvals(dtype, 200_000, rng)])
    b = np.concatenate([np.tile(sp, sp.size), _randvals(dtype, 200_000, rng)])
    got = oracle.combine(dtype, op, a, b)
    want = refops.combine(dtype, op, a, b)
    refops.assert_same(dtype, got, want, f"{dtype} {op}")
    if op in ("max", "min") and dtype in refops.FLOATS:
        # canonical NaN exactly, not merely "a NaN"
        bits = got.view(np.uint32 if dtype == "fp32" else np.uint16)
        nan = np.isnan(refops.to_f64(dtype, got))
        assert np.all(bits[nan] == refops.CANON_NAN[dtype])


def test_fp32_subnormals_are_kept():
    a = np.array([1e-45, 1e-44, 1e-39], np.float32)
    got = oracle.combine("fp32", "sum", a, a)
    assert np.all(got > 0) and np.array_equal(got, a + a)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_half_ops_are_correctly_rounded(dtype):
    """binary32 op then one rounding equals the correctly rounded 16-bit op
    (double rounding is innocuous for + and x when 24 >= 2p + 2)."""
    rng = np.random.default_rng(11)
    a = rng.integers(0, 1 << 16, 300_000, dtype=np.uint32).astype(np.uint16)
    b = rng.integers(0, 1 << 16, 300_000, dtype=np.uint32).astype(np.uint16)
    fa = refops.to_f64(dtype, a.view(refops.STORAGE[dtype]))
    fb = refops.to_f64(dtype, b.view(refops.STORAGE[dtype]))
    ok = np.isfinite(fa) & np.isfinite(fb)
    for op, exact in (("sum", fa + fb), ("prod", fa * fb)):
        got = oracle.combine(dtype, op, a.view(refops.STORAGE[dtype]), b.view(refops.STORAGE[dtype]))
        g = refops.to_f64(dtype, got)
        # exact binary64 result for binary16 sums/products; round it once via torch
        t = torch.from_numpy(exact).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
        want = t.to(torch.float64).numpy()
        sel = ok & np.isfinite(want) & np.isfinite(g)
        if dtype == "fp16" or op == "prod":
            # binary64 holds these exactly (fp16 sums, all products of 8/11-bit significands)
            assert np.array_equal(g[sel], want[sel]), (dtype, op)
