"""Helpers for the GPU parity tests: host copies, the bars, a threaded oracle call.

The bars (per element): w, m, v within 1e-6 relative per step (2e-6 after
up to 10 chained steps), where y = 0 requires x = 0 and y = +-inf requires
the same inf; the 16-bit working copy within 1 ulp (ordered-integer
distance); the fp32 mean and all indexing bit-exact.  NaN must meet NaN.
Differences in bits are counted and reported (the expected count is 0).
"""

from __future__ import annotations

import os
import sys
import threading

import numpy as np
import pytest
import torch

import oracle

DEV = "cuda"
LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.float32, copy=False)


def to_dev_u16(bits: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(dtype).to(DEV)


def check_f32(got: np.ndarray, want: np.ndarray, tol: float, what: str) -> int:
    """Apply the fp32 bar; return the number of elements whose bits differ."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({int((gn != wn).sum())})"
    inf = np.isinf(want)
    assert np.array_equal(got[inf], want[inf]), f"{what}: inf mismatch"
    fin = ~wn & ~inf
    zero = fin & (want == 0)
    assert np.all(got[zero] == 0), f"{what}: {int((got[zero] != 0).sum())} nonzero where 0"
    nz = fin & (want != 0)
    if nz.any():
        rel = np.abs(got[nz].astype(np.float64) - want[nz]) / np.abs(want[nz].astype(np.float64))
        worst = float(rel.max())
        assert worst <= tol, f"{what}: max rel err {worst:.3g} > {tol:g}"
    same = (got.view(np.uint32) == want.view(np.uint32)) | (gn & wn)
    return int((~same).sum())


def _ordered16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def nan16(b: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f16":
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def check_param(got: np.ndarray, want: np.ndarray, dt: str, what: str) -> int:
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    assert got.shape == want.shape, what
    gn, wn = nan16(got, dt), nan16(want, dt)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    ok = ~wn
    dist = np.abs(_ordered16(got[ok]) - _ordered16(want[ok]))
    if dist.size:
        assert int(dist.max()) <= 1, f"{what}: {int((dist > 1).sum())} elements beyond 1 ulp"
    return int((got[ok] != want[ok]).sum())


def oracle_step_threaded(gdt, grads, w, m, v, pdt, t, form="standard", lr=LR, b1=B1, b2=B2,
                         eps=EPS, threads=None) -> np.ndarray:
    """oracle.step_elems over n elements split into contiguous ranges run on
    several threads (elements are independent, so the result is identical)."""
    n = w.size
    threads = threads or min(16, os.cpu_count() or 1)
    param = np.empty(n, np.uint16)
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    errs = []

    def run(a, b):
        try:
            if b > a:
                oracle.step_elems(gdt, [g[a:b] for g in grads], w[a:b], m[a:b], v[a:b], pdt,
                                  lr, b1, b2, eps, t, form, param=param[a:b])
        except Exception as ex:  # pragma: no cover
            errs.append(ex)

    ths = [threading.Thread(target=run, args=(int(bounds[i]), int(bounds[i + 1])))
           for i in range(threads)]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    if errs:
        raise errs[0]
    return param
