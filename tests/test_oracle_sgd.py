"""Pins of the oracle's two SGD forms.

Page "深度学习专题：模型训练的数据并行（三）" §(一) Adam 优化器 gives the SGD
update w_{t+1} = w_t - lr * g_{t+1}.  Page "ZeRO 技术原理：进阶与 Offload"
§1.1.1 names SGD with momentum and the momentum buffer it stores, without a
formula; the oracle takes the plain heavy-ball reading m <- beta1*m + g,
w <- w - lr*m (m0 = 0).

Pins: exact dyadic closed forms (every intermediate value representable, so
the fp32 result must equal the rational one bit for bit), momentum with
beta1 = 0 reducing to SGD, the untouched state arrays, the fused step with a
rank mean, and torch.optim.SGD (a library routine) for both forms.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _f32(x: Fraction) -> np.float32:
    y = np.float32(float(x))
    assert Fraction(float(y)) == x, "test value not representable in fp32"
    return y


@pytest.mark.parametrize("k", [1, 3, 6])
def test_sgd_dyadic_closed_form(k):
    # lr = 2^-4, g = +-2^-k, w0 = j/64: w_T = w0 - T*lr*g exactly in fp32
    lr = Fraction(1, 16)
    n, T = 64, 8
    w0 = [Fraction(j - 32, 64) for j in range(n)]
    g = [Fraction((-1) ** j, 2 ** k) for j in range(n)]
    w = np.array([_f32(x) for x in w0], np.float32)
    m = np.full(n, 7.0, np.float32)
    v = np.full(n, 9.0, np.float32)
    ga = np.array([_f32(x) for x in g], np.float32)
    for t in range(1, T + 1):
        oracle.adam_apply(ga, w, m, v, "bf16", float(lr), 0.9, 0.999, 1e-8, t, "sgd")
        want = [a - t * lr * b for a, b in zip(w0, g)]
        assert np.array_equal(w, np.array([_f32(x) for x in want], np.float32))
    assert np.all(m == 7.0) and np.all(v == 9.0), "SGD touched its unused state"


def test_momentum_dyadic_closed_form():
    # beta1 = 1/2, lr = 2^-3, g = +-2^-2: m_t = g*(2 - 2^(1-t)), w_t = w_{t-1} - lr*m_t
    b1, lr = Fraction(1, 2), Fraction(1, 8)
    n, T = 32, 10
    w0 = [Fraction(j, 32) for j in range(n)]
    g = [Fraction(-1 if j % 3 else 1, 4) for j in range(n)]
    w = np.array([_f32(x) for x in w0], np.float32)
    m = np.zeros(n, np.float32)
    v = np.full(n, 5.0, np.float32)
    ga = np.array([_f32(x) for x in g], np.float32)
    wr, mr = list(w0), [Fraction(0)] * n
    for t in range(1, T + 1):
        oracle.adam_apply(ga, w, m, v, "f16", float(lr), float(b1), 0.999, 1e-8, t,
                          "sgd_momentum")
        mr = [b1 * a + b for a, b in zip(mr, g)]
        wr = [a - lr * b for a, b in zip(wr, mr)]
        assert all(x == y * (2 - Fraction(2) ** (1 - t)) for x, y in zip(mr, g))
        assert np.array_equal(m, np.array([_f32(x) for x in mr], np.float32))
        assert np.array_equal(w, np.array([_f32(x) for x in wr], np.float32))
    assert np.all(v == 5.0), "momentum SGD touched v"


def test_momentum_with_zero_beta_is_sgd():
    rng = np.random.default_rng(5)
    n = 100_000
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    a, b = w0.copy(), w0.copy()
    ma, va = np.zeros(n, np.float32), np.zeros(n, np.float32)
    mb, vb = ma.copy(), va.copy()
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        pa = oracle.adam_apply(g, a, ma, va, "bf16", 1e-3, 0.0, 0.999, 1e-8, t, "sgd_momentum")
        pb = oracle.adam_apply(g, b, mb, vb, "bf16", 1e-3, 0.9, 0.999, 1e-8, t, "sgd")
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(pa, pb)


def test_fused_step_sgd_uses_the_rank_mean():
    # four ranks whose fp32 mean is exact: the step equals SGD on that mean
    rng = np.random.default_rng(6)
    n, p = 4096, 4
    bits = [oracle.narrow("f16", (rng.integers(-64, 64, n) / 256.0).astype(np.float32))
            for _ in range(p)]
    mean = sum(oracle.widen("f16", b).astype(np.float64) for b in bits) / p
    w0 = (rng.integers(-512, 512, n) / 1024.0).astype(np.float32)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.step_elems("f16", bits, w, m, v, "f16", 0.125, 0.9, 0.999, 1e-8, 1, "sgd")
    want = (w0.astype(np.float64) - 0.125 * mean).astype(np.float32)
    assert np.array_equal(w, want)


@pytest.mark.parametrize("momentum", [0.0, 0.9])
def test_matches_torch_sgd(momentum):
    rng = np.random.default_rng(7)
    n, T, lr = 200_000, 10, 1e-2
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.SGD([p], lr=lr, momentum=momentum, foreach=False)
    form = "sgd_momentum" if momentum else "sgd"
    for t in range(1, T + 1):
        g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        oracle.adam_apply(g, w, m, v, "f16", lr, momentum, 0.999, 1e-8, t, form)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        tw = p.detach().numpy()
        # each step moves w by about lr*|m| <= t*lr*0.05; torch may round that
        # product and the subtraction differently (a fused multiply-add)
        assert np.max(np.abs(w - tw) / np.maximum(np.abs(tw), t * lr * 1e-2)) < 1e-6
        if momentum:
            tm = opt.state[p]["momentum_buffer"].numpy()
            assert np.max(np.abs(m - tm) / np.maximum(np.abs(tm), 1e-30)) < 1e-6


def test_unknown_form_rejected():
    g = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        oracle.lib()  # built
        from oracle import _check, lib, _ptr, _f32p  # noqa: F401
        st = lib().oracle_adam_apply(_ptr(g, _f32p), _ptr(g.copy(), _f32p), _ptr(g.copy(), _f32p),
                                     _ptr(g.copy(), _f32p), None, 1, 4, 1e-3, 0.9, 0.999, 1e-8, 1,
                                     4)
        _check(st, "adam_apply")
