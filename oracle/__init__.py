"""ctypes loader for the CPU oracle (liboracle.so, built from zs_oracle.cpp).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  The product
library (adam_zs_shard_amd) never imports it and has no CPU fallback.

Wrappers take and return numpy arrays; 16-bit values travel as uint16 bit
patterns so the oracle sees exactly the bits the caller holds.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F16, BF16 = 1, 2
STANDARD, PAGE1_LITERAL, SGD, SGD_MOMENTUM = 0, 1, 2, 3
DTYPES = {"f16": F16, "bf16": BF16}
FORMS = {"standard": STANDARD, "page1_literal": PAGE1_LITERAL, "sgd": SGD,
         "sgd_momentum": SGD_MOMENTUM}

_i64p = C.POINTER(C.c_int64)
_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_u16p = C.POINTER(C.c_uint16)
_u16pp = C.POINTER(_u16p)

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with g++ (no FMA contraction, no fast-math)."""
    import subprocess

    src = os.path.join(HERE, "zs_oracle.cpp")
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        L.oracle_f16_to_f32.argtypes = [C.c_uint16]
        L.oracle_f16_to_f32.restype = C.c_float
        L.oracle_bf16_to_f32.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f32.restype = C.c_float
        L.oracle_f32_to_f16.argtypes = [C.c_float]
        L.oracle_f32_to_f16.restype = C.c_uint16
        L.oracle_f32_to_bf16.argtypes = [C.c_float]
        L.oracle_f32_to_bf16.restype = C.c_uint16
        L.oracle_widen.argtypes = [C.c_int32, _u16p, _f32p, C.c_int64]
        L.oracle_widen.restype = C.c_int32
        L.oracle_narrow.argtypes = [C.c_int32, _f32p, _u16p, C.c_int64]
        L.oracle_narrow.restype = C.c_int32
        L.oracle_plan_shards.argtypes = [C.c_int64, C.c_int32, _i64p, _i64p, _i64p]
        L.oracle_plan_shards.restype = C.c_int32
        L.oracle_adam_scalars.argtypes = [C.c_double, C.c_double, C.c_double, C.c_double,
                                          C.c_int64, C.c_int32, _f32p]
        L.oracle_adam_scalars.restype = C.c_int32
        L.oracle_grad_mean.argtypes = [C.c_int32, C.c_int32, _u16pp, C.c_int64, _f32p]
        L.oracle_grad_mean.restype = C.c_int32
        L.oracle_adam_apply.argtypes = [_f32p, _f32p, _f32p, _f32p, _u16p, C.c_int32, C.c_int64,
                                        C.c_double, C.c_double, C.c_double, C.c_double,
                                        C.c_int64, C.c_int32]
        L.oracle_adam_apply.restype = C.c_int32
        L.oracle_step_elems.argtypes = [C.c_int32, C.c_int32, _u16pp, _f32p, _f32p, _f32p, _u16p,
                                        C.c_int32, C.c_int64, C.c_double, C.c_double, C.c_double,
                                        C.c_double, C.c_int64, C.c_int32]
        L.oracle_step_elems.restype = C.c_int32
        L.oracle_shard_step.argtypes = [C.c_int64, C.c_int32, C.c_int32, _u16pp, C.c_int32,
                                        C.c_int64, _f32p, _f32p, _f32p, _u16p, C.c_int32,
                                        C.c_int64, C.c_double, C.c_double, C.c_double,
                                        C.c_double, C.c_int64, C.c_int32]
        L.oracle_shard_step.restype = C.c_int32
        L.oracle_locate.argtypes = [_i64p, C.c_int32, C.c_int64, _i64p]
        L.oracle_locate.restype = C.c_int32
        L.oracle_shard_pieces.argtypes = [_i64p, C.c_int32, C.c_int64, C.c_int64, _i32p, _i64p,
                                          _i64p, _i64p, C.c_int32]
        L.oracle_shard_pieces.restype = C.c_int32
        L.oracle_mp_bytes_per_param.argtypes = [C.c_int32, C.c_double, C.c_double]
        L.oracle_mp_bytes_per_param.restype = C.c_double
        L.oracle_p1_floats.argtypes = [C.c_int32, C.c_int64, C.c_int32]
        L.oracle_p1_floats.restype = C.c_double
        _lib = L
    return _lib


# ----------------------------------------------------------------- helpers

def _ptr(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data_as(t)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} returned status {rc}")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _ptr_table(arrs):
    tab = (_u16p * len(arrs))(*[_ptr(a, _u16p) for a in arrs])
    return C.cast(tab, _u16pp), tab


def plan_shards(n: int, p: int):
    """(M, starts[p], ends[p]) as Python ints."""
    m = C.c_int64()
    s = np.zeros(p, np.int64)
    e = np.zeros(p, np.int64)
    _check(lib().oracle_plan_shards(n, p, C.byref(m), _ptr(s, _i64p), _ptr(e, _i64p)),
           "plan_shards")
    return int(m.value), [int(x) for x in s], [int(x) for x in e]


def adam_scalars(lr, b1, b2, eps, t, p=1) -> np.ndarray:
    out = np.zeros(9, np.float32)
    _check(lib().oracle_adam_scalars(lr, b1, b2, eps, t, p, _ptr(out, _f32p)), "adam_scalars")
    return out


def widen(dtype: str, bits) -> np.ndarray:
    bits = _u16(bits)
    out = np.empty(bits.shape, np.float32)
    _check(lib().oracle_widen(DTYPES[dtype], _ptr(bits, _u16p), _ptr(out, _f32p), bits.size),
           "widen")
    return out


def narrow(dtype: str, x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _check(lib().oracle_narrow(DTYPES[dtype], _ptr(x, _f32p), _ptr(out, _u16p), x.size),
           "narrow")
    return out


def grad_mean(dtype: str, grads) -> np.ndarray:
    """grads: list of P uint16 arrays of equal length -> fp32 mean."""
    gs = [_u16(g) for g in grads]
    n = gs[0].size
    out = np.empty(n, np.float32)
    tab, keep = _ptr_table(gs)
    _check(lib().oracle_grad_mean(DTYPES[dtype], len(gs), tab, n, _ptr(out, _f32p)), "grad_mean")
    del keep
    return out


def adam_apply(g, w, m, v, pdtype, lr, b1, b2, eps, t, form="standard"):
    """In-place Adam on float32 arrays w, m, v; returns the 16-bit param bits."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    n = g.size
    param = np.empty(n, np.uint16)
    _check(lib().oracle_adam_apply(_ptr(g, _f32p), _ptr(w, _f32p), _ptr(m, _f32p),
                                   _ptr(v, _f32p), _ptr(param, _u16p), DTYPES[pdtype], n,
                                   lr, b1, b2, eps, t, FORMS[form]), "adam_apply")
    return param


def step_elems(gdtype, grads, w, m, v, pdtype, lr, b1, b2, eps, t, form="standard",
               param=None):
    """Fused step on compact arrays: grads is a list of P uint16 arrays of n;
    w, m, v (float32, n) are updated in place; returns the param bits."""
    gs = [_u16(g) for g in grads]
    n = w.size
    if param is None:
        param = np.empty(n, np.uint16)
    tab, keep = _ptr_table(gs)
    _check(lib().oracle_step_elems(DTYPES[gdtype], len(gs), tab, _ptr(w, _f32p),
                                   _ptr(m, _f32p), _ptr(v, _f32p), _ptr(param, _u16p),
                                   DTYPES[pdtype], n, lr, b1, b2, eps, t, FORMS[form]),
           "step_elems")
    del keep
    return param


def shard_step(n, p, k, grads, gdtype, grad_base, w, m, v, param, pdtype, param_base,
               lr, b1, b2, eps, t, form="standard"):
    """Per-shard step with the global index map (all arrays updated in place)."""
    gs = [_u16(g) for g in grads]
    tab, keep = _ptr_table(gs)
    pr = param if param.dtype == np.uint16 else param.view(np.uint16)
    _check(lib().oracle_shard_step(n, p, k, tab, DTYPES[gdtype], grad_base, _ptr(w, _f32p),
                                   _ptr(m, _f32p), _ptr(v, _f32p), _ptr(pr, _u16p),
                                   DTYPES[pdtype], param_base, lr, b1, b2, eps, t, FORMS[form]),
           "shard_step")
    del keep


def locate(numel, j: int):
    nm = np.ascontiguousarray(numel, dtype=np.int64)
    off = C.c_int64()
    t = lib().oracle_locate(_ptr(nm, _i64p), nm.size, j, C.byref(off))
    return int(t), int(off.value)


def shard_pieces(numel, lo: int, hi: int, cap: int = 1 << 16):
    """List of (tensor, tensor_off, range_off, len) where [lo, hi) meets each tensor."""
    nm = np.ascontiguousarray(numel, dtype=np.int64)
    t = np.zeros(cap, np.int32)
    to = np.zeros(cap, np.int64)
    ro = np.zeros(cap, np.int64)
    ln = np.zeros(cap, np.int64)
    cnt = lib().oracle_shard_pieces(_ptr(nm, _i64p), nm.size, lo, hi, _ptr(t, _i32p),
                                    _ptr(to, _i64p), _ptr(ro, _i64p), _ptr(ln, _i64p), cap)
    if cnt < 0:
        raise ValueError("shard_pieces: cap exceeded")
    return [(int(t[i]), int(to[i]), int(ro[i]), int(ln[i])) for i in range(cnt)]


def mp_bytes_per_param(stage: int, ndev: float, k_bytes: float = 12.0) -> float:
    return lib().oracle_mp_bytes_per_param(stage, float(ndev), float(k_bytes))


def p1_floats(scheme: int, n: int, p: int) -> float:
    return lib().oracle_p1_floats(scheme, n, p)
