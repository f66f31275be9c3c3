"""GPU parity of the fused per-shard step (zs_fused_shard_step) against the
CPU oracle, element by element, on seeded synthetic inputs."""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import WORKLOADS, seed_for
from zs_synth import make
from zs_synth.gen import normal
from gpu_util import (DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, to_dev_u16, check_f32,
                      check_param, oracle_step_threaded)

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16}
SENTINEL = 0x5A5A


def hp(t, form="standard"):
    return z.hparams(LR, B1, B2, EPS, t, form)


def _rand_bits(n, dt, std, seed):
    x = normal(n, std, seed, TD[dt])
    return x.view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def test_tiny_p4_all_shards_three_steps():
    """N=1,000,003 over P=4 (last shard short), fp16 full-length rank
    buffers, all shards, 3 chained steps, standard Adam."""
    wl = WORKLOADS["tiny_p4"]
    n, p = wl.n, wl.p
    M, s, e = oracle.plan_shards(n, p)
    param_d = torch.empty(n, dtype=torch.float16, device=DEV)
    param_d.view(torch.int16).fill_(SENTINEL)
    param_h = np.full(n, SENTINEL, np.uint16)
    W = {k: make.initial_w(wl, k, e[k] - s[k]) for k in wl.shards}
    wd = {k: W[k].to(DEV) for k in wl.shards}
    md = {k: torch.zeros_like(wd[k]) for k in wl.shards}
    vd = {k: torch.zeros_like(wd[k]) for k in wl.shards}
    wh = {k: W[k].numpy().copy() for k in wl.shards}
    mh = {k: np.zeros_like(wh[k]) for k in wl.shards}
    vh = {k: np.zeros_like(wh[k]) for k in wl.shards}
    diffs = 0
    for t in range(1, wl.steps + 1):
        gh = [make.normal_grad(wl, r, t, n) for r in range(p)]
        gd = [g.to(DEV) for g in gh]
        gb = [u16(g) for g in gh]
        for k in wl.shards:
            say(f"tiny_p4 step {t} shard {k}")
            z.zs_fused_shard_step(n, p, k, gd, wd[k], md[k], vd[k], param_d, hp(t))
            oracle.shard_step(n, p, k, gb, "f16", 0, wh[k], mh[k], vh[k], param_h, "f16", 0,
                              LR, B1, B2, EPS, t)
        torch.cuda.synchronize()
        tol = 1e-6 if t == 1 else 2e-6
        for k in wl.shards:
            diffs += check_f32(f32(wd[k]), wh[k], tol, f"w k={k} t={t}")
            diffs += check_f32(f32(md[k]), mh[k], tol, f"m k={k} t={t}")
            diffs += check_f32(f32(vd[k]), vh[k], tol, f"v k={k} t={t}")
        diffs += check_param(u16(param_d), param_h, "f16", f"param t={t}")
    say(f"tiny_p4: {diffs} elements differ in bits")
    assert not np.any(u16(param_d) == SENTINEL)   # every shard wrote its slice


@pytest.mark.parametrize("gdt,pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
                                     ("bf16", "f16")])
@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_dtypes_and_forms_from_mid_training_state(gdt, pdt, form):
    n, p, k, T = 70_001, 5, 2, 4
    M, s, e = oracle.plan_shards(n, p)
    L = e[k] - s[k]
    w0 = normal(L, 0.02, seed_for(11, k)).numpy()
    m0, v0 = (x.numpy() for x in make.random_state(L, 5))
    wd, md, vd = (torch.from_numpy(x.copy()).to(DEV) for x in (w0, m0, v0))
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    param_d = torch.empty(n, dtype=TD[pdt], device=DEV)
    param_d.view(torch.int16).fill_(SENTINEL)
    param_h = np.full(n, SENTINEL, np.uint16)
    for t in range(1, T + 1):
        gb = [_rand_bits(n, gdt, 1e-2, seed_for(12, r, t)) for r in range(p)]
        gd = [to_dev_u16(b, TD[gdt]) for b in gb]
        z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, hp(t, form))
        oracle.shard_step(n, p, k, gb, gdt, 0, wh, mh, vh, param_h, pdt, 0, LR, B1, B2, EPS, t,
                          form)
        torch.cuda.synchronize()
        tol = 1e-6 if t == 1 else 2e-6
        check_f32(f32(wd), wh, tol, "w")
        check_f32(f32(md), mh, tol, "m")
        check_f32(f32(vd), vh, tol, "v")
        check_param(u16(param_d), param_h, pdt, "param")


def test_canary_outside_the_shard_untouched():
    n, p, k = 100_003, 3, 1
    M, s, e = oracle.plan_shards(n, p)
    L = e[k] - s[k]
    gb = [_rand_bits(n, "f16", 1e-2, seed_for(13, r)) for r in range(p)]
    gd = [to_dev_u16(b, torch.float16) for b in gb]
    w0 = normal(L, 0.02, seed_for(14)).numpy()
    wd = torch.from_numpy(w0.copy()).to(DEV)
    md, vd = torch.zeros_like(wd), torch.zeros_like(wd)
    # the param buffer has guard zones before and after the N elements
    guard = 4096
    buf = torch.empty(n + 2 * guard, dtype=torch.float16, device=DEV)
    buf.view(torch.int16).fill_(SENTINEL)
    param_d = buf[guard:guard + n]
    # the state arrays too
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, hp(1))
    torch.cuda.synchronize()
    out = u16(buf)
    inside = np.zeros(out.size, bool)
    inside[guard + s[k]:guard + e[k]] = True
    assert np.all(out[~inside] == SENTINEL)
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    ph = np.full(n, SENTINEL, np.uint16)
    oracle.shard_step(n, p, k, gb, "f16", 0, wh, mh, vh, ph, "f16", 0, LR, B1, B2, EPS, 1)
    assert np.array_equal(out[inside], ph[s[k]:e[k]])
    check_f32(f32(wd), wh, 1e-6, "w")


def _offset_view(length, off, dtype):
    buf = torch.empty(length + 16, dtype=dtype, device=DEV)
    return buf[off:off + length]


@pytest.mark.parametrize("case", range(16))
def test_alignment_sweep(case):
    """Every array at its own element offset (slice layout): the vector path
    must give the same bits whichever streams are 16-byte aligned."""
    rng = np.random.default_rng(case)
    n, p, k = 50_021, 4, 1
    M, s, e = oracle.plan_shards(n, p)
    L = e[k] - s[k]
    if case == 0:
        go, wo, mo, vo, po = [0] * p, 0, 0, 0, 0
    elif case < 8:
        go, wo, mo, vo, po = [case] * p, case % 4, case % 4, case % 4, case
    else:
        go = [int(x) for x in rng.integers(0, 8, p)]
        wo, mo, vo = (int(x) for x in rng.integers(0, 4, 3))
        po = int(rng.integers(0, 8))
    gb = [_rand_bits(L, "bf16", 1e-2, seed_for(15, case, r)) for r in range(p)]
    gd = []
    for r in range(p):
        t = _offset_view(L, go[r], torch.bfloat16)
        t.copy_(to_dev_u16(gb[r], torch.bfloat16))
        gd.append(t)
    w0 = normal(L, 0.02, seed_for(16, case)).numpy()
    m0, v0 = (x.numpy() for x in make.random_state(L, case))
    wd, md, vd = (_offset_view(L, o, torch.float32) for o in (wo, mo, vo))
    wd.copy_(torch.from_numpy(w0))
    md.copy_(torch.from_numpy(m0))
    vd.copy_(torch.from_numpy(v0))
    param_d = _offset_view(L, po, torch.bfloat16)
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, hp(3), grad_base=s[k],
                          param_base=s[k])
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    ph = oracle_step_threaded("bf16", gb, wh, mh, vh, "bf16", 3)
    assert check_f32(f32(wd), wh, 1e-6, "w") == 0
    assert check_f32(f32(md), mh, 1e-6, "m") == 0
    assert check_f32(f32(vd), vh, 1e-6, "v") == 0
    assert check_param(u16(param_d), ph, "bf16", "param") == 0


@pytest.mark.parametrize("p", [1, 2, 3, 7, 8, 9, 15, 16, 17, 63, 64, 65, 128, 200, 256])
def test_rank_count_sweep(p):
    L = 3_001 + 8 * p
    n = L * p - 5 if p > 1 else L
    M, s, e = oracle.plan_shards(n, p)
    k = p // 2
    L = e[k] - s[k]
    gb = [_rand_bits(L, "f16", 1e-2, seed_for(17, p, r)) for r in range(p)]
    gd = [to_dev_u16(b, torch.float16) for b in gb]
    w0 = normal(L, 0.02, seed_for(18, p)).numpy()
    wd = torch.from_numpy(w0.copy()).to(DEV)
    md, vd = torch.zeros_like(wd), torch.zeros_like(wd)
    param_d = torch.empty(L, dtype=torch.float16, device=DEV)
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, hp(1), grad_base=s[k],
                          param_base=s[k])
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    ph = oracle_step_threaded("f16", gb, wh, mh, vh, "f16", 1)
    assert check_f32(f32(wd), wh, 1e-6, "w") == 0
    assert check_f32(f32(vd), vh, 1e-6, "v") == 0
    assert check_param(u16(param_d), ph, "f16", "param") == 0


@pytest.mark.parametrize("n,p,k", [(9, 4, 3), (0, 1, 0), (5, 8, 7)])
def test_empty_shard_is_a_no_op(n, p, k):
    M, s, e = oracle.plan_shards(n, p)
    assert s[k] == e[k]
    g = [torch.ones(max(n, 1), dtype=torch.float16, device=DEV) for _ in range(p)]
    w = torch.full((4,), 3.0, device=DEV)
    st = z.zs_fused_shard_step(n, p, k, g, w, w.clone(), w.clone(),
                               torch.zeros(max(n, 1), dtype=torch.float16, device=DEV), hp(1))
    assert st == z.ZS_OK
    torch.cuda.synchronize()
    assert torch.all(w == 3.0)


@pytest.mark.parametrize("L", [1, 2, 7, 8, 9, 15, 16, 17, 255, 2048 + 3])
def test_short_shards_and_ragged_tails(L):
    p = 3
    n = L * p
    k = 1
    M, s, e = oracle.plan_shards(n, p)
    gb = [_rand_bits(n, "f16", 1e-2, seed_for(19, L, r)) for r in range(p)]
    gd = [to_dev_u16(b, torch.float16) for b in gb]
    # misalign the full buffers by one element so head and tail both occur
    w0 = normal(L, 0.02, seed_for(20, L)).numpy()
    wd = _offset_view(L, 1, torch.float32)
    wd.copy_(torch.from_numpy(w0))
    md = torch.zeros(L, device=DEV)
    vd = torch.zeros(L, device=DEV)
    param_d = torch.empty(n, dtype=torch.float16, device=DEV)
    param_d.view(torch.int16).fill_(SENTINEL)
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, hp(1))
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    ph = np.full(n, SENTINEL, np.uint16)
    oracle.shard_step(n, p, k, gb, "f16", 0, wh, mh, vh, ph, "f16", 0, LR, B1, B2, EPS, 1)
    assert check_f32(f32(wd), wh, 1e-6, "w") == 0
    assert np.array_equal(u16(param_d), ph)


def test_determinism_and_resume():
    n, p, k = 200_003, 8, 5
    M, s, e = oracle.plan_shards(n, p)
    L = e[k] - s[k]
    w0 = normal(L, 0.02, seed_for(21)).to(DEV)
    grads = {t: [normal(n, 1e-3, seed_for(22, r, t), torch.bfloat16, "cpu").to(DEV)
                 for r in range(p)] for t in range(1, 11)}

    def run(ts, w, m, v, par):
        for t in ts:
            z.zs_fused_shard_step(n, p, k, grads[t], w, m, v, par, hp(t))

    a = [w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0)]
    pa = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    run(range(1, 11), *a, pa)
    b = [w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0)]
    pb = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    run(range(1, 11), *b, pb)
    # resume: 5 steps, state to the host and back into fresh buffers, 5 more
    c = [w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0)]
    pc = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    run(range(1, 6), *c, pc)
    host = [x.cpu() for x in c] + [pc.cpu()]
    c2 = [x.to(DEV) for x in host[:3]]
    pc2 = host[3].to(DEV)
    run(range(6, 11), *c2, pc2)
    torch.cuda.synchronize()
    for x, y, yy in zip(a, b, c2):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(x.view(torch.int32), yy.view(torch.int32))
    assert torch.equal(pa.view(torch.int16), pb.view(torch.int16))
    assert torch.equal(pa.view(torch.int16), pc2.view(torch.int16))


def test_special_gradient_values():
    """inf, NaN, max-finite, subnormal and signed-zero gradients propagate by
    IEEE rules exactly as in the oracle."""
    n, p, k = 4_099, 3, 0
    M, s, e = oracle.plan_shards(n, p)
    L = e[k] - s[k]
    rng = np.random.default_rng(23)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00,
                         0x7E00, 0x3C00, 0x0400], np.uint16)
    gb = []
    for r in range(p):
        b = _rand_bits(n, "f16", 1e-2, seed_for(24, r))
        idx = rng.integers(0, n, 300)
        b[idx] = rng.choice(specials, 300)
        gb.append(b)
    gd = [to_dev_u16(b, torch.float16) for b in gb]
    w0 = normal(L, 0.02, seed_for(25)).numpy()
    wd = torch.from_numpy(w0.copy()).to(DEV)
    md, vd = torch.zeros_like(wd), torch.zeros_like(wd)
    param_d = torch.empty(n, dtype=torch.float16, device=DEV)
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, hp(1))
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    ph = np.zeros(n, np.uint16)
    oracle.shard_step(n, p, k, gb, "f16", 0, wh, mh, vh, ph, "f16", 0, LR, B1, B2, EPS, 1)
    assert np.isnan(wh).any() and np.isinf(mh).any()
    check_f32(f32(wd), wh, 1e-6, "w")
    check_f32(f32(md), mh, 1e-6, "m")
    check_f32(f32(vd), vh, 1e-6, "v")
    check_param(u16(param_d)[:L], ph[:L], "f16", "param")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_downcast_exhaustive_via_zero_gradient(dt):
    """With g = 0 and m = v = 0 the update is exactly 0, so the working copy is
    the 16-bit rounding of w itself: feed every interesting fp32 pattern."""
    vals = []
    h = np.arange(0, 0x7C00 if dt == "f16" else 0x7F80, dtype=np.uint16)
    wide = oracle.widen(dt, h).astype(np.float64)
    mid = ((wide[:-1] + wide[1:]) / 2).astype(np.float32)
    vals += [wide.astype(np.float32), mid, np.nextafter(mid, np.float32(0)),
             np.nextafter(mid, np.float32(np.inf))]
    rng = np.random.default_rng(26)
    vals.append(rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
                .view(np.float32))
    vals.append(np.array([np.inf, np.nan, 65520.0, 65519.996, 3.3961776e38, 1e-45, 1e-40],
                         np.float32))
    w = np.concatenate(vals)
    w = np.concatenate([w, -w])
    L = w.size
    wd = torch.from_numpy(w.copy()).to(DEV)
    g = torch.zeros(L, device=DEV)
    md, vd = torch.zeros_like(g), torch.zeros_like(g)
    param = torch.empty(L, dtype=TD[dt], device=DEV)
    z.zs_adam_step(g, wd, md, vd, param, L, hp(1))
    torch.cuda.synchronize()
    out_w = f32(wd)
    fin = ~np.isnan(w)
    assert np.array_equal(out_w[fin].view(np.uint32), w[fin].view(np.uint32))
    assert np.all(np.isnan(out_w[~fin]))
    want = oracle.narrow(dt, w)
    got = u16(param)
    nan_w = np.isnan(w)
    assert np.array_equal(got[~nan_w], want[~nan_w])
    from gpu_util import nan16

    assert np.all(nan16(got[nan_w], dt))
