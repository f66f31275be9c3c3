"""Parity of the host-CPU offload update (zs_cpu_adam_step) with the oracle.

Page "ZeRO 技术原理：进阶与 Offload" §2.2 Offload 策略: the CPU receives the
shard's 16-bit gradient and runs the update and float2half on the fp32 state
kept in host memory; §1.6.2: multithreaded SIMD.  The library's AVX2 code must
equal the oracle's scalar sequence bit for bit on the widened gradient, for
every form, dtype pair, thread count and tail length.  Host-only: these run
without a GPU.
"""

import numpy as np
import pytest

import oracle
from adam_zs_shard_amd import zshard as z
from gpu_util import check_f32, check_param

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8
FORMS = ["standard", "page1_literal", "sgd", "sgd_momentum"]
CANARY = np.uint32(0x7FC0DEAD)


def _grad16(rng, n, dt, scale=1e-2):
    return oracle.narrow(dt, (rng.standard_normal(n) * scale).astype(np.float32))


def _state(rng, n):
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    return w, m, v


def _both(g16, gdt, pdt, w, m, v, form, steps, threads, null_unused=False):
    """Run the library and the oracle side by side; return both results."""
    n = w.size
    uses_m = form != "sgd"
    uses_v = form in ("standard", "page1_literal")
    lw, lm, lv = w.copy(), m.copy(), v.copy()
    ow, om, ov = w.copy(), m.copy(), v.copy()
    lp = np.zeros(n, np.uint16)
    for t in range(1, steps + 1):
        g = g16[t - 1]
        z.zs_cpu_adam_step(g, gdt, lw, lm if (uses_m or not null_unused) else None,
                           lv if (uses_v or not null_unused) else None, lp, pdt, n,
                           z.hparams(LR, B1, B2, EPS, t, form), threads=threads)
        op = oracle.adam_apply(oracle.widen(gdt, g), ow, om, ov, pdt, LR, B1, B2, EPS, t, form)
    return (lw, lm, lv, lp), (ow, om, ov, op)


def _assert_same(lib, ref, pdt, what):
    (lw, lm, lv, lp), (ow, om, ov, op) = lib, ref
    d = check_f32(lw, ow, 0.0, f"w {what}") + check_f32(lm, om, 0.0, f"m {what}")
    d += check_f32(lv, ov, 0.0, f"v {what}") + check_param(lp, op, pdt, f"param {what}")
    assert d == 0, f"{d} elements differ in bits ({what})"


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("gdt,pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
                                     ("bf16", "f16")])
def test_matches_oracle(form, gdt, pdt):
    rng = np.random.default_rng(hash((form, gdt, pdt)) % 2**32)
    n = 100_003
    g16 = [_grad16(rng, n, gdt) for _ in range(3)]
    w, m, v = _state(rng, n)
    lib, ref = _both(g16, gdt, pdt, w, m, v, form, 3, threads=4)
    _assert_same(lib, ref, pdt, f"{form} {gdt}->{pdt}")


@pytest.mark.parametrize("threads", [1, 2, 3, 7, 16])
def test_thread_counts_agree(threads):
    rng = np.random.default_rng(11)
    n = 300_017
    g16 = [_grad16(rng, n, "bf16") for _ in range(2)]
    w, m, v = _state(rng, n)
    lib, ref = _both(g16, "bf16", "bf16", w, m, v, "standard", 2, threads=threads)
    _assert_same(lib, ref, "bf16", f"{threads} threads")


def test_every_tail_length():
    rng = np.random.default_rng(12)
    for n in range(0, 18):
        g16 = [_grad16(rng, max(n, 1), "f16")[:n]]
        w, m, v = _state(rng, n)
        lib, ref = _both(g16, "f16", "f16", w, m, v, "page1_literal", 1, threads=1)
        _assert_same(lib, ref, "f16", f"n={n}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_special_values(dt):
    # zeros of both signs, subnormal and huge gradients, inf and NaN, and
    # weights that overflow or underflow the 16-bit copy
    pos_inf = 0x7C00 if dt == "f16" else 0x7F80
    nan = 0x7E00 if dt == "f16" else 0x7FC0
    sub = 0x0001
    big = 0x7BFF if dt == "f16" else 0x7F7F
    pat = np.array([0x0000, 0x8000, sub, 0x8000 | sub, big, 0x8000 | big, pos_inf,
                    0x8000 | pos_inf, nan, 0x3C00, 0xBC00, 0x0400], np.uint16)
    g = np.tile(pat, 7)[:80]
    n = g.size
    w = np.tile(np.array([0.0, -0.0, 1e-30, 7e4, -7e4, 3.0e38, 1e-45, 0.5], np.float32), 10)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for form in FORMS:
        lib, ref = _both([g], dt, dt, w, m, v, form, 1, threads=1)
        _assert_same(lib, ref, dt, f"special {form}")


@pytest.mark.parametrize("form", ["sgd", "sgd_momentum"])
def test_unused_state_null_or_untouched(form):
    rng = np.random.default_rng(13)
    n = 50_001
    g16 = [_grad16(rng, n, "f16") for _ in range(2)]
    w, m, v = _state(rng, n)
    lib, ref = _both(g16, "f16", "f16", w, m, v, form, 2, threads=3, null_unused=True)
    (lw, lm, lv, lp), (ow, om, ov, op) = lib, ref
    assert check_f32(lw, ow, 0.0, "w") == 0 and check_param(lp, op, "f16", "param") == 0
    if form == "sgd_momentum":
        assert check_f32(lm, om, 0.0, "m") == 0
    # canary-filled unused buffers passed in come back untouched
    cm = np.full(n, CANARY, np.uint32).view(np.float32)
    cv = cm.copy()
    wm = w.copy()
    mm = m.copy() if form == "sgd_momentum" else cm
    z.zs_cpu_adam_step(g16[0], "f16", wm, mm, cv, None, 0, n,
                       z.hparams(LR, B1, B2, EPS, 1, form), threads=2)
    assert np.all(cv.view(np.uint32) == CANARY)
    if form == "sgd":
        assert np.all(cm.view(np.uint32) == CANARY)


def test_argument_errors():
    n = 64
    g = np.zeros(n, np.uint16)
    w, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    hp = z.hparams(LR, B1, B2, EPS, 1)

    def call(**kw):
        a = dict(g=g, gdt="f16", w=w, m=m, v=v, param=p, pdt="f16", n=n, hp=hp)
        a.update(kw)
        return z.zs_cpu_adam_step(a["g"], a["gdt"], a["w"], a["m"], a["v"], a["param"],
                                  a["pdt"], a["n"], a["hp"], check=False)

    assert call() == z.ZS_OK
    assert call(n=0, w=None) == z.ZS_OK                 # nothing to do
    assert call(n=-1) == z.ZS_ERR_ARG
    assert call(gdt=3) == z.ZS_ERR_DTYPE
    assert call(pdt=7) == z.ZS_ERR_DTYPE
    assert call(w=None) == z.ZS_ERR_NULL
    assert call(v=None) == z.ZS_ERR_NULL
    assert call(hp=z.hparams(LR, B1, B2, EPS, 0)) == z.ZS_ERR_ARG
    assert call(hp=z.hparams(LR, 1.0, B2, EPS, 1)) == z.ZS_ERR_ARG
    assert call(hp=z.hparams(LR, B1, B2, EPS, 1, form=4)) == z.ZS_ERR_ARG
    assert call(m=w) == z.ZS_ERR_ALIAS                  # m on top of w
    assert call(param=w.view(np.uint16)[:n]) == z.ZS_ERR_ALIAS
    big = np.zeros(4 * n, np.uint16)
    assert call(g=big[:n], param=big[n // 2:n // 2 + n]) == z.ZS_ERR_ALIAS
