"""Pins of the oracle's Adam update (both forms) and of the fused step.

Page "深度学习专题：模型训练的数据并行（三）" §(一) Adam 优化器: update
w_{t+1} = w_t - lr * m_{t+1} / (sqrt(v_{t+1}) + eps) and the moment/variance
equations with the (1 - beta^{t+1}) denominators (the page-1 literal form);
page "ZeRO 技术原理：进阶与 Offload" §1.1.1: exponentially weighted moving
averages, i.e. standard Adam (Kingma & Ba, its ref. 10), which stores the raw
averages and bias-corrects at use.

Pins: closed forms for a constant gradient, the |g| = eps and g = 0 special
cases, exact-rational recurrences of the literal form and its fp32 overflow
step, torch.optim.Adam (a library routine) for the standard form, and the
ZeRO invariant that the sharded update equals the replicated one.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def _run(g_steps, w0, form, m0=None, v0=None, pdt="f16"):
    n = w0.size
    w = w0.astype(np.float32).copy()
    m = np.zeros(n, np.float32) if m0 is None else m0.copy()
    v = np.zeros(n, np.float32) if v0 is None else v0.copy()
    hist = []
    for t, g in enumerate(g_steps, start=1):
        param = oracle.adam_apply(g, w, m, v, pdt, LR, B1, B2, EPS, t, form)
        hist.append((w.copy(), m.copy(), v.copy(), param))
    return hist


def test_constants_derived_in_double_and_rounded_once():
    c = oracle.adam_scalars(LR, B1, B2, EPS, 1, 64).view(np.uint32)
    want = [0x3F666666, 0x3DCCCCCD, 0x3F7FBE77, 0x3A83126F, 0x3DCCCCCD, 0x3A83126F,
            0x3A83126F, 0x322BCC77, 0x42800000]
    assert [int(x) for x in c] == want
    # 1 - beta2 evaluated in fp32 instead would be off by 1.3e-5 relative
    c2_f32 = np.float32(1.0) - np.float32(0.999)
    assert abs(float(c2_f32) / 1e-3 - 1) > 1e-5
    # 1 - beta^t uses the exact power for large t
    ct = oracle.adam_scalars(LR, B1, B2, EPS, 1000, 1)
    assert ct[4] == np.float32(1.0 - 0.9 ** 1000) and ct[5] == np.float32(1.0 - 0.999 ** 1000)


@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_zero_gradient_is_a_fixed_point(form):
    w0 = np.random.default_rng(0).standard_normal(1000).astype(np.float32) * 0.02
    hist = _run([np.zeros(1000, np.float32)] * 5, w0, form)
    for w, m, v, _ in hist:
        assert np.array_equal(w.view(np.uint32), w0.view(np.uint32))
        assert np.all(m == 0) and np.all(v == 0)


@pytest.mark.parametrize("gval", [0.5, 1e-3, 1e-8, 1e2, -0.75, -3e-5, 7.0])
def test_standard_constant_gradient_closed_form(gval):
    # With g constant, m_t = (1-b1^t) g and v_t = (1-b2^t) g^2, so the
    # corrected moments are g and g^2 and every step moves w by
    # -lr * g / (|g| + eps).
    g = np.float32(gval)
    T = 10
    hist = _run([np.full(4, g, np.float32)] * T, np.zeros(4, np.float32), "standard")
    step = LR * float(g) / (abs(float(g)) + EPS)
    w_prev = 0.0
    for t, (w, m, v, _) in enumerate(hist, start=1):
        mh = float(m[0]) / (1 - B1 ** t)
        vh = float(v[0]) / (1 - B2 ** t)
        assert abs(mh / float(g) - 1) < 1e-6
        assert abs(vh / float(g) ** 2 - 1) < 1e-6
        dw = w_prev - float(w[0])
        assert abs(dw / step - 1) < 2e-6, (t, dw, step)
        w_prev = float(w[0])


def test_step_one_closed_form_random_gradients():
    rng = np.random.default_rng(1)
    g = (rng.standard_normal(100000) * 10.0 ** rng.integers(-7, 3, 100000)).astype(np.float32)
    (w, m, v, _), = _run([g], np.zeros(g.size, np.float32), "standard")
    want = -LR * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + EPS)
    assert np.max(np.abs(w / want - 1)) < 2e-6


def test_gradient_equal_to_eps_moves_half_lr():
    g = np.float32(EPS)
    (w, _, _, _), = _run([np.full(3, g)], np.zeros(3, np.float32), "standard")
    assert abs(-float(w[0]) / (LR / 2) - 1) < 1e-6


def test_standard_matches_torch_adam():
    # P = 1: the step is plain Adam on the given gradient.
    rng = np.random.default_rng(2)
    n, T = 200_000, 10
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    grads = [(sign * np.abs(rng.standard_normal(n)) * 1e-2).astype(np.float32) for _ in range(T)]
    hist = _run(grads, w0, "standard")

    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.Adam([p], lr=LR, betas=(B1, B2), eps=EPS, foreach=False)
    for t in range(T):
        p.grad = torch.from_numpy(grads[t].copy())
        opt.step()
        st = opt.state[p]
        w, m, v, _ = hist[t]
        tw, tm, tv = p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
        assert np.max(np.abs(m - tm) / np.abs(tm)) < 1e-6
        assert np.max(np.abs(v - tv) / np.abs(tv)) < 1e-6
        # Each step moves w by at most lr and the two sides round that step
        # differently (a few ulp of it), so after t steps w may differ by a
        # few e-7 of t*lr: measure against max(|w|, t*lr).
        assert np.max(np.abs(w - tw) / np.maximum(np.abs(tw), (t + 1) * LR)) < 1e-6


def _literal_coeffs(T):
    b1, b2 = Fraction(9, 10), Fraction(999, 1000)
    a, b = [None, Fraction(1)], [None, Fraction(1)]
    for t in range(2, T + 1):
        a.append((b1 * a[-1] + 1 - b1) / (1 - b1 ** t))
        b.append((b2 * b[-1] + 1 - b2) / (1 - b2 ** t))
    return a, b


def test_literal_coefficients_closed_form():
    a, b = _literal_coeffs(20)
    assert abs(float(a[2]) - 5.26316) < 1e-5 and abs(float(b[2]) - 500.25) < 1e-3
    assert abs(float(a[5]) - 103.538) < 1e-3 and abs(float(b[5]) / 8.35e9 - 1) < 1e-3
    assert abs(float(b[20]) / 4.439e38 - 1) < 1e-3


@pytest.mark.parametrize("gval", [1e-3, -0.25, 1.0, 10.0, 100.0])
def test_literal_constant_gradient_and_overflow(gval):
    # Literal form with constant g: m_t = a_t g, v_t = b_t g^2.  v overflows
    # fp32 at the first t with b_t g^2 beyond FLT_MAX; then sqrt(v) = inf,
    # the update is 0 and w stops moving, without NaN.
    T = 20
    a, b = _literal_coeffs(T)
    fmax = Fraction(float(np.finfo(np.float32).max))
    g = np.float32(gval)
    gq = Fraction(float(g))
    hist = _run([np.full(2, g)] * T, np.zeros(2, np.float32), "page1_literal")
    overflow_t = next((t for t in range(1, T + 1) if b[t] * gq * gq > fmax), None)
    expected_first = {1.0: 20, 10.0: 19, 100.0: 18}.get(abs(gval))
    assert overflow_t == expected_first
    w_prev = np.float32(0)
    for t, (w, m, v, _) in enumerate(hist, start=1):
        assert abs(float(m[0]) / float(a[t] * gq) - 1) < 1e-6 * t
        if overflow_t is not None and t >= overflow_t:
            assert np.isposinf(v[0])
            assert w[0] == w_prev
        else:
            assert np.isfinite(v[0])
            assert abs(float(v[0]) / float(b[t] * gq * gq) - 1) < 1e-6 * t
        assert not np.isnan(w[0])
        w_prev = w[0]


def test_forms_agree_at_step_one():
    rng = np.random.default_rng(3)
    g = (rng.standard_normal(50000) * 1e-2).astype(np.float32)
    w0 = (rng.standard_normal(50000) * 0.02).astype(np.float32)
    (ws, ms, vs, ps), = _run([g], w0, "standard")
    (wl, ml, vl, pl), = _run([g], w0, "page1_literal")
    assert np.array_equal(ws.view(np.uint32), wl.view(np.uint32))
    assert np.array_equal(ps, pl)
    assert not np.array_equal(ms, ml)


@pytest.mark.parametrize("gdt,pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16")])
def test_fused_step_equals_mean_then_adam(gdt, pdt):
    rng = np.random.default_rng(4)
    p, n = 5, 3000
    x = (rng.standard_normal((p, n)) * 1e-2).astype(np.float32)
    grads = [oracle.narrow(gdt, x[r]) for r in range(p)]
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w1, m1, v1 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    par1 = oracle.step_elems(gdt, grads, w1, m1, v1, pdt, LR, B1, B2, EPS, 1)
    w2, m2, v2 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    par2 = oracle.adam_apply(oracle.grad_mean(gdt, grads), w2, m2, v2, pdt, LR, B1, B2, EPS, 1)
    for a_, b_ in ((w1, w2), (m1, m2), (v1, v2)):
        assert np.array_equal(a_.view(np.uint32), b_.view(np.uint32))
    assert np.array_equal(par1, par2)
    assert np.array_equal(par1, oracle.narrow(pdt, w1))


@pytest.mark.parametrize("n,p", [(1003, 4), (17, 8), (8, 4), (5, 8)])
def test_sharded_update_equals_replicated_update(n, p):
    # ZeRO invariant ([DP-III] §(三): the states of different parameters are
    # independent, so partitioning them does not change the update): running
    # every rank's shard step with full-length buffers reproduces the
    # unsharded data-parallel Adam step on the mean gradient, bit for bit.
    rng = np.random.default_rng(n * 10 + p)
    x = (rng.standard_normal((p, n)) * 1e-2).astype(np.float32)
    grads = [oracle.narrow("f16", x[r]) for r in range(p)]
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    M, s, e = oracle.plan_shards(n, p)
    param = np.full(n, 0x7777, np.uint16)
    wsh = w0.copy()
    msh, vsh = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in (1, 2, 3):
        for k in range(p):
            sl = slice(s[k], e[k])
            w_k, m_k, v_k = wsh[sl].copy(), msh[sl].copy(), vsh[sl].copy()
            oracle.shard_step(n, p, k, grads, "f16", 0, w_k, m_k, v_k, param, "f16", 0,
                              LR, B1, B2, EPS, t)
            wsh[sl], msh[sl], vsh[sl] = w_k, m_k, v_k
    wr, mr, vr = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = oracle.grad_mean("f16", grads)
    for t in (1, 2, 3):
        pr = oracle.adam_apply(g, wr, mr, vr, "f16", LR, B1, B2, EPS, t)
    assert np.array_equal(wsh.view(np.uint32), wr.view(np.uint32))
    assert np.array_equal(msh.view(np.uint32), mr.view(np.uint32))
    assert np.array_equal(vsh.view(np.uint32), vr.view(np.uint32))
    assert np.array_equal(param, pr)


def test_shard_step_slice_layout_and_param_base():
    # grad_base / param_base map global index j to buffer offsets: a rank's
    # gradients given as slices of its shard, and a param buffer that starts
    # at the shard, give the same numbers as full-length buffers.
    rng = np.random.default_rng(5)
    n, p, k = 1001, 4, 2
    M, s, e = oracle.plan_shards(n, p)
    x = (rng.standard_normal((p, n)) * 1e-2).astype(np.float32)
    full = [oracle.narrow("bf16", x[r]) for r in range(p)]
    sl = [f[s[k]:e[k]].copy() for f in full]
    w0 = (rng.standard_normal(e[k] - s[k]) * 0.02).astype(np.float32)
    zs = lambda: np.zeros(e[k] - s[k], np.float32)  # noqa: E731
    wa, ma, va = w0.copy(), zs(), zs()
    pa = np.zeros(n, np.uint16)
    oracle.shard_step(n, p, k, full, "bf16", 0, wa, ma, va, pa, "bf16", 0, LR, B1, B2, EPS, 1)
    wb, mb, vb = w0.copy(), zs(), zs()
    pb = np.zeros(e[k] - s[k], np.uint16)
    oracle.shard_step(n, p, k, sl, "bf16", s[k], wb, mb, vb, pb, "bf16", s[k], LR, B1, B2, EPS, 1)
    assert np.array_equal(wa, wb) and np.array_equal(pa[s[k]:e[k]], pb)
    assert np.all(pa[:s[k]] == 0) and np.all(pa[e[k]:] == 0)


def test_bad_arguments_rejected():
    g = np.zeros(4, np.float32)
    w, m, v = g.copy(), g.copy(), g.copy()
    for kw in (dict(t=0), dict(b1=1.0), dict(b2=-0.1), dict(lr=float("inf"))):
        args = dict(lr=LR, b1=B1, b2=B2, eps=EPS, t=1)
        args.update(kw)
        with pytest.raises(ValueError):
            oracle.adam_apply(g, w, m, v, "f16", args["lr"], args["b1"], args["b2"],
                              args["eps"], args["t"])
