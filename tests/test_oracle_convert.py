"""Pins of the oracle's 16-bit conversions against library routines.

binary16 <-> binary32: numpy's float16 (round to nearest even).
bfloat16 <-> binary32: torch's bfloat16 on the CPU (round to nearest even).
Widening is checked on all 65,536 patterns; narrowing on random and
boundary binary32 patterns.  NaN is compared as NaN; its sign is kept by the
oracle (and by numpy), while torch's bfloat16 cast drops it.
"""

import numpy as np
import pytest
import torch

import oracle

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _same(a: np.ndarray, b: np.ndarray, nan_sign: bool = True):
    an, bn = np.isnan(a), np.isnan(b)
    assert np.array_equal(an, bn)
    if nan_sign:
        assert np.array_equal(np.signbit(a[an]), np.signbit(b[bn]))
    assert np.array_equal(a[~an].view(np.uint32), b[~bn].view(np.uint32))


def test_widen_f16_exhaustive():
    got = oracle.widen("f16", ALL16)
    ref = ALL16.view(np.float16).astype(np.float32)
    _same(got, ref)


def test_widen_bf16_exhaustive():
    got = oracle.widen("bf16", ALL16)
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).float().numpy()
    _same(got, ref)


def _boundary_f32() -> np.ndarray:
    vals = []
    # binary16 ties and neighbours around every binade edge, max finite, overflow
    for e in range(-26, 17):
        base = np.float32(2.0 ** e)
        vals += [base, np.nextafter(base, np.float32(0)), np.nextafter(base, np.float32(np.inf))]
    h = np.arange(0, 0x7c00, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    h_next = np.arange(1, 0x7c01, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    mid = ((h.astype(np.float64) + h_next.astype(np.float64)) / 2).astype(np.float32)
    vals += list(mid) + list(np.nextafter(mid, np.float32(0))) + list(
        np.nextafter(mid, np.float32(np.inf)))
    vals += [65504.0, 65519.996, 65520.0, 65536.0, 1e30, np.inf, 5.96e-8, 2.98e-8, 2.9802322e-8,
             1e-45, 1.17549435e-38, 3.3895314e38, 3.3961776e38, 3.4028235e38, 0.0]
    # bf16 ties: low 16 bits exactly 0x8000 with both parities
    b = np.arange(0, 0x7f800000, 0x00012345, dtype=np.uint64).astype(np.uint32)
    vals += list(((b & 0xFFFF0000) | 0x8000).view(np.float32))
    vals += list(((b & 0xFFFF0000) | 0x7FFF).view(np.float32))
    vals += list(((b & 0xFFFF0000) | 0x8001).view(np.float32))
    v = np.array(vals, dtype=np.float32)
    return np.concatenate([v, -v, np.array([np.nan, -np.nan], np.float32)])


def _random_f32(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("which", ["boundary", "random"])
def test_narrow_f16_vs_numpy(which):
    x = _boundary_f32() if which == "boundary" else _random_f32(2_000_000, 1)
    got = oracle.narrow("f16", x).view(np.float16).astype(np.float32)
    ref = x.astype(np.float16).astype(np.float32)
    _same(got, ref)


def test_narrow_f16_small_magnitudes_vs_numpy():
    # dense sweep of the binary16 subnormal and low-normal range
    rng = np.random.default_rng(2)
    x = (rng.uniform(-1, 1, 2_000_000) * 2.0 ** rng.integers(-27, -10, 2_000_000)).astype(
        np.float32)
    got = oracle.narrow("f16", x).view(np.float16).astype(np.float32)
    _same(got, x.astype(np.float16).astype(np.float32))


@pytest.mark.parametrize("which", ["boundary", "random"])
def test_narrow_bf16_vs_torch(which):
    x = _boundary_f32() if which == "boundary" else _random_f32(2_000_000, 3)
    got = oracle.widen("bf16", oracle.narrow("bf16", x))
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    # torch maps every NaN to one negative NaN; the oracle keeps the sign.
    _same(got, ref, nan_sign=False)
    nan = np.isnan(x)
    assert np.array_equal(np.signbit(got[nan]), np.signbit(x[nan]))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_roundtrip_all_patterns(dt):
    w = oracle.widen(dt, ALL16)
    back = oracle.narrow(dt, w)
    ok = ~np.isnan(w)
    assert np.array_equal(back[ok], ALL16[ok])
    assert np.all(np.isnan(oracle.widen(dt, back[~ok])))


def test_scalar_entry_points_agree_with_arrays():
    L = oracle.lib()
    for h in (0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x7C00, 0x8001, 0xFBFF):
        assert np.float32(L.oracle_f16_to_f32(h)) == oracle.widen("f16", np.array([h], np.uint16))[0]
    for x in (1.0, 65520.0, 1e-8, -3.3961776e38):
        assert L.oracle_f32_to_f16(x) == oracle.narrow("f16", np.array([x], np.float32))[0]
        assert L.oracle_f32_to_bf16(x) == oracle.narrow("bf16", np.array([x], np.float32))[0]
