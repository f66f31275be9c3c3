"""GPU parity of the SGD forms (ZS_SGD, ZS_SGD_MOMENTUM) against the oracle.

Plain SGD (w - lr*g, page "深度学习专题：模型训练的数据并行（三）" §(一)) and
heavy-ball momentum SGD (m = beta1*m + g, w - lr*m; the reading of page
"ZeRO 技术原理：进阶与 Offload" §1.1.1) through every entry point: the fused
single-tensor step, the chunk table and the unfused Adam-step call, with the
state a form does not use passed as NULL, or as canary-filled buffers that
must come back untouched.
"""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for, WORKLOADS, make
from zs_synth.gen import normal, fill_pattern
from gpu_util import (DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, check_f32, check_param,
                      oracle_step_threaded)

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
CANARY = 0x7FC0DEAD  # a NaN pattern no update can produce from these inputs
CHUNK = 28 * 256 * 8


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _canary(n):
    return fill_pattern(torch.empty(n, dtype=torch.float32, device=DEV), CANARY)


def _untouched(t):
    return bool((t.view(torch.int32) == (CANARY - (1 << 32))).all())


@pytest.mark.parametrize("form", ["sgd", "sgd_momentum"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("null_state", [True, False])
def test_fused_all_shards(form, dt, null_state):
    n, p, steps = 1_000_003, 4, 3
    M, s, e = oracle.plan_shards(n, p)
    gh = {(r, t): normal(n, 1e-2, seed_for(70, r, t), TD[dt]) for r in range(p)
          for t in range(1, steps + 1)}
    par = torch.zeros(n, dtype=TD[dt], device=DEV)
    ph = np.zeros(n, np.uint16)
    for k in range(p):
        L = e[k] - s[k]
        w0 = normal(L, 0.02, seed_for(71, k))
        w = w0.to(DEV)
        if form == "sgd":
            m = None if null_state else _canary(L)
        else:
            m = torch.zeros(L, device=DEV)
        v = None if null_state else _canary(L)
        wh, mh, vh = w0.numpy().copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
        for t in range(1, steps + 1):
            gd = [gh[(r, t)].to(DEV) for r in range(p)]
            z.zs_fused_shard_step(n, p, k, gd, w, m, v, par, z.hparams(LR, B1, B2, EPS, t, form))
            bits = [gh[(r, t)].view(torch.int16).numpy().view(np.uint16)[s[k]:e[k]]
                    for r in range(p)]
            ph[s[k]:e[k]] = oracle_step_threaded(dt, bits, wh, mh, vh, dt, t, form)
        torch.cuda.synchronize()
        d = check_f32(f32(w), wh, 2e-6, f"w k={k}")
        if form == "sgd_momentum":
            d += check_f32(f32(m), mh, 2e-6, f"m k={k}")
        elif m is not None:
            assert _untouched(m), "SGD wrote m"
        if v is not None:
            assert _untouched(v), f"{form} wrote v"
        assert d == 0, f"{d} elements differ in bits, shard {k}"
    assert check_param(u16(par), ph, dt, "param") == 0


@pytest.mark.parametrize("form", ["sgd", "sgd_momentum"])
def test_fused_mid_size_shard(form):
    # one round and a bit over the CUs: whole chunks plus rank-batched pieces
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    L, p = (cu + cu // 3) * CHUNK + 8 * 97 + 3, 3
    n = L * p
    w0 = normal(L, 0.02, seed_for(72))
    w, m = w0.to(DEV), torch.zeros(L, device=DEV)
    par = torch.zeros(L, dtype=torch.bfloat16, device=DEV)
    wh, mh, vh = w0.numpy().copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in (1, 2):
        gh = [normal(L, 1e-3, seed_for(73, r, t), torch.bfloat16) for r in range(p)]
        z.zs_fused_shard_step(n, p, 0, [g.to(DEV) for g in gh], w, m, None, par,
                              z.hparams(LR, B1, B2, EPS, t, form))
        ph = oracle_step_threaded("bf16", [g.view(torch.int16).numpy().view(np.uint16) for g in gh],
                                  wh, mh, vh, "bf16", t, form)
    torch.cuda.synchronize()
    d = check_f32(f32(w), wh, 2e-6, "w") + check_param(u16(par), ph, "bf16", "param")
    if form == "sgd_momentum":
        d += check_f32(f32(m), mh, 2e-6, "m")
    assert d == 0


def test_multi_tensor_momentum_without_v():
    wl = WORKLOADS["gpt2_small_p8"]
    numel = [x for _, x in wl.tensors]
    p, k, chunk = wl.p, 2, 65536
    M, s, e = oracle.plan_shards(wl.n, p)
    L = e[k] - s[k]
    pieces, nchunks = z.zs_plan_chunks(numel, p, k, chunk)
    w0 = normal(L, 0.02, seed_for(74))
    w, m = w0.to(DEV), torch.zeros(L, device=DEV)
    params = {t: torch.zeros(numel[t], dtype=torch.bfloat16, device=DEV)
              for (t, _, _, _) in pieces}
    grads = [torch.empty(L, dtype=torch.bfloat16, device=DEV) for _ in range(p)]
    ptrs = [dict(w=w.data_ptr() + 4 * so, m=m.data_ptr() + 4 * so, v=None,
                 param=params[t].data_ptr() + 2 * to, grads=[g.data_ptr() + 2 * so for g in grads])
            for (t, to, so, ln) in pieces]
    nb = z.zs_mt_workspace_bytes(len(pieces), nchunks, p)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    table = z.zs_mt_upload(pieces, ptrs, p, "bf16", "bf16", chunk, ws, nb)
    assert table.state == z.ZS_STATE_M
    # a step that needs v is refused before anything runs
    assert z.zs_fused_shard_step_multi(table, z.hparams(LR, B1, B2, EPS, 1),
                                       check=False) == z.ZS_ERR_NULL
    wh, mh, vh = w0.numpy().copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in (1, 2, 3):
        gh = [normal(L, 1e-3, seed_for(75, r, t), torch.bfloat16) for r in range(p)]
        for r in range(p):
            grads[r].copy_(gh[r].to(DEV))
        z.zs_fused_shard_step_multi(table, z.hparams(LR, B1, B2, EPS, t, "sgd_momentum"))
        ph = oracle_step_threaded("bf16", [g.view(torch.int16).numpy().view(np.uint16) for g in gh],
                                  wh, mh, vh, "bf16", t, "sgd_momentum")
    torch.cuda.synchronize()
    d = check_f32(f32(w), wh, 2e-6, "w") + check_f32(f32(m), mh, 2e-6, "m")
    for (t, to, so, ln) in oracle.shard_pieces(numel, s[k], e[k]):
        d += check_param(u16(params[t][to:to + ln]), ph[so:so + ln], "bf16", f"tensor {t}")
    assert d == 0


@pytest.mark.parametrize("form", ["sgd", "sgd_momentum"])
def test_adam_step_entry_point(form):
    L = 123_457
    g = normal(L, 1e-2, seed_for(76)).numpy()
    w0 = normal(L, 0.02, seed_for(77)).numpy()
    gd, wd = torch.from_numpy(g.copy()).to(DEV), torch.from_numpy(w0.copy()).to(DEV)
    md = torch.zeros(L, device=DEV) if form == "sgd_momentum" else None
    par = torch.empty(L, dtype=torch.float16, device=DEV)
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in (1, 2, 3):
        z.zs_adam_step(gd, wd, md, None, par, L, z.hparams(LR, B1, B2, EPS, t, form))
        ph = oracle.adam_apply(g, wh, mh, vh, "f16", LR, B1, B2, EPS, t, form)
    torch.cuda.synchronize()
    d = check_f32(f32(wd), wh, 2e-6, "w") + check_param(u16(par), ph, "f16", "param")
    if md is not None:
        d += check_f32(f32(md), mh, 2e-6, "m")
    assert d == 0


def test_zero_7p5b_p64_momentum_sampled():
    # the bench's largest shape, momentum SGD, sampled against the oracle
    wl = WORKLOADS["zero_7p5b_p64"]
    k = wl.shards[-1]
    M, s, e = oracle.plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    w = make.initial_w(wl, k, L, DEV)
    m = torch.zeros_like(w)
    param = torch.empty(wl.n, dtype=torch.float16, device=DEV)
    rng = np.random.default_rng(78)
    idx = np.unique(np.concatenate([np.arange(64), L - 64 + np.arange(64),
                                    rng.integers(0, L, 4000)]))
    idev = torch.from_numpy(idx).to(DEV)
    ws, ms, vs = f32(w[idev]).copy(), np.zeros(idx.size, np.float32), np.zeros(idx.size,
                                                                             np.float32)
    for t in (1, 2):
        grads = [make.normal_grad(wl, r, t, L, DEV, stream=k) for r in range(wl.p)]
        z.zs_fused_shard_step(wl.n, wl.p, k, grads, w, m, None, param,
                              z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, t, "sgd_momentum"),
                              grad_base=s[k])
        gs = [u16(g[idev]) for g in grads]
        del grads
        ph = oracle.step_elems("f16", gs, ws, ms, vs, "f16", wl.lr, wl.beta1, wl.beta2, wl.eps, t,
                               "sgd_momentum")
        torch.cuda.synchronize()
        d = check_f32(f32(w[idev]), ws, 2e-6, "w") + check_f32(f32(m[idev]), ms, 2e-6, "m")
        d += check_param(u16(param[s[k] + idev]), ph, "f16", "param")
        assert d == 0, f"{d} sampled values differ at t={t}"
        say(f"  7.5B momentum step {t}: {idx.size} samples bit-identical")


@pytest.mark.parametrize("form", ["sgd", "sgd_momentum"])
def test_adam_step_entry_point_whole_chunks(form):
    # a length with whole chunks for at least half the CUs takes the chunked
    # update kernel; v (and for plain SGD m) passed as NULL
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    L = (cu + cu // 4) * CHUNK + 8 * 333 + 5
    g = normal(L, 1e-2, seed_for(79)).numpy()
    w0 = normal(L, 0.02, seed_for(80)).numpy()
    gd, wd = torch.from_numpy(g.copy()).to(DEV), torch.from_numpy(w0.copy()).to(DEV)
    md = torch.zeros(L, device=DEV) if form == "sgd_momentum" else None
    par = torch.empty(L, dtype=torch.bfloat16, device=DEV)
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in (1, 2):
        z.zs_adam_step(gd, wd, md, None, par, L, z.hparams(LR, B1, B2, EPS, t, form))
        ph = oracle.adam_apply(g, wh, mh, vh, "bf16", LR, B1, B2, EPS, t, form)
    torch.cuda.synchronize()
    d = check_f32(f32(wd), wh, 2e-6, "w") + check_param(u16(par), ph, "bf16", "param")
    if md is not None:
        d += check_f32(f32(md), mh, 2e-6, "m")
    assert d == 0
