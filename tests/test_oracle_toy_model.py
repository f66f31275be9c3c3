"""The pages' 4-layer scalar model as a worked ZeRO-3 example for the oracle.

Page "深度学习专题：模型训练的数据并行（三）", §(四) ZeRO-3 层间流水线优化 /
1. 前向传播和反向传播的计算资料: scalar input x, layers h_m = ReLU(w_m h_{m-1} + b_m)
for m = 1..3, y = w_4 h_3 + b_4, loss L = (y - x)^2 / 2, and the printed
backward formulas.  2. 层间流水线: 4 GPUs, GPU-m stores layer m's (w_m, b_m),
each trains on a quarter of the mini-batch; after reduce-scatter GPU-m
updates layer m.

Checks: the printed backward formulas agree with torch autograd; the
oracle's per-shard step over the 4 shards (N=8, P=4, M=2) equals
torch.optim.Adam on the whole model with the averaged gradient.
"""

import numpy as np
import torch

import oracle

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def page_forward_backward(wb, x):
    """Gradients of L for one sample, from the page's printed formulas."""
    w1, b1, w2, b2, w3, b3, w4, b4 = wb
    relu = lambda z: max(z, 0.0)  # noqa: E731
    h1 = relu(w1 * x + b1)
    h2 = relu(w2 * h1 + b2)
    h3 = relu(w3 * h2 + b3)
    y = w4 * h3 + b4
    dy = y - x
    dw4, db4 = dy * h3, dy
    dh3 = dy * w4
    i3 = 1.0 if h3 > 0 else 0.0
    dw3, db3 = dh3 * h2 * i3, dh3 * i3
    dh2 = dh3 * w3 * i3
    i2 = 1.0 if h2 > 0 else 0.0
    dw2, db2 = dh2 * h1 * i2, dh2 * i2
    dh1 = dh2 * w2 * i2
    i1 = 1.0 if h1 > 0 else 0.0
    dw1, db1 = dh1 * x * i1, dh1 * i1
    return np.array([dw1, db1, dw2, db2, dw3, db3, dw4, db4])


def torch_grads(wb, x):
    t = torch.tensor(wb, dtype=torch.float64, requires_grad=True)
    h = torch.tensor(x, dtype=torch.float64)
    xin = h
    for m in range(3):
        h = torch.relu(t[2 * m] * h + t[2 * m + 1])
    y = t[6] * h + t[7]
    loss = 0.5 * (y - xin) ** 2
    loss.backward()
    return t.grad.numpy()


def test_page_backward_formulas_match_autograd():
    rng = np.random.default_rng(0)
    for _ in range(200):
        wb = rng.standard_normal(8)
        x = float(rng.standard_normal())
        assert np.allclose(page_forward_backward(wb, x), torch_grads(wb, x), rtol=1e-12,
                           atol=1e-12)


def test_zero3_toy_step_equals_replicated_adam():
    rng = np.random.default_rng(1)
    P, N, T = 4, 8, 6
    M, s, e = oracle.plan_shards(N, P)
    w = (rng.standard_normal(N) * 0.5 + 0.5).astype(np.float32)   # mostly active ReLUs
    shards = [dict(w=w[s[k]:e[k]].copy(), m=np.zeros(M, np.float32),
                   v=np.zeros(M, np.float32)) for k in range(P)]
    param = oracle.narrow("f16", w)            # the fp16 working copy all ranks read
    ref = torch.nn.Parameter(torch.from_numpy(w.copy()))
    opt = torch.optim.Adam([ref], lr=LR, betas=(B1, B2), eps=EPS, foreach=False)
    for t in range(1, T + 1):
        # each GPU: its quarter of the mini-batch (2 samples), fp16 working weights
        wb = oracle.widen("f16", param).astype(np.float64)
        xs = rng.standard_normal((P, 2))
        local = [np.mean([page_forward_backward(wb, x) for x in xs[r]], axis=0) for r in
                 range(P)]
        gbits = [oracle.narrow("f16", g.astype(np.float32)) for g in local]
        for k in range(P):
            sh = shards[k]
            oracle.shard_step(N, P, k, gbits, "f16", 0, sh["w"], sh["m"], sh["v"], param, "f16",
                              0, LR, B1, B2, EPS, t)
        # replicated data-parallel Adam on the mean of the same fp16 gradients
        g = np.mean([oracle.widen("f16", b).astype(np.float64) for b in gbits], axis=0)
        ref.grad = torch.from_numpy(g.astype(np.float32))
        opt.step()
        w_sharded = np.concatenate([sh["w"] for sh in shards])
        tw = ref.detach().numpy()
        assert np.max(np.abs(w_sharded - tw) / np.maximum(np.abs(tw), t * LR)) < 1e-6
        # every shard wrote its layer's fp16 copy into the full buffer
        assert np.array_equal(param, oracle.narrow("f16", w_sharded))


def _f32_canonical(gbits, w, m, v, t, p):
    """numpy float32 scalar evaluation of the same operation order (compile
    check of the built oracle: catches FMA contraction or excess precision)."""
    f = np.float32
    B1f, C1f, B2f, C2f = f(B1), f(1.0 - B1), f(B2), f(1.0 - B2)
    BC1, BC2 = f(1.0 - B1 ** t), f(1.0 - B2 ** t)
    s = f(gbits[0])
    for r in range(1, p):
        s = f(s + f(gbits[r]))
    g = f(s / f(p))
    mm = f(f(B1f * m) + f(C1f * g))
    vv = f(f(B2f * v) + f(C2f * f(g * g)))
    mh, vh = f(mm / BC1), f(vv / BC2)
    d = f(f(np.sqrt(vh)) + f(EPS))
    return f(w - f(f(LR) * f(mh / d))), mm, vv


def test_built_oracle_has_no_contraction():
    rng = np.random.default_rng(2)
    P, n = 4, 8
    for t in range(1, 4):
        x = (rng.standard_normal((P, n)) * 10.0 ** rng.integers(-4, 1, (P, n))).astype(np.float32)
        gb = [oracle.narrow("f16", x[r]) for r in range(P)]
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
        wo, mo, vo = w.copy(), m.copy(), v.copy()
        oracle.step_elems("f16", gb, wo, mo, vo, "f16", LR, B1, B2, EPS, t)
        gv = [oracle.widen("f16", b) for b in gb]
        for i in range(n):
            ew, em, ev = _f32_canonical([g[i] for g in gv], w[i], m[i], v[i], t, P)
            assert (wo[i], mo[i], vo[i]) == (ew, em, ev)
