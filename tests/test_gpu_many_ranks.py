"""GPU parity for more ranks than fit in one launch's kernel arguments
(257..1024), and for the 16-bit stored mean.

Above 256 ranks the fused step reads its rank pointers from a device
workspace that one small launch per 256 ranks fills first; the stored mean
runs in passes of 256 ranks, each continuing the fp32 sums the previous pass
left behind.  Both must give the oracle's result bit for bit: the same left
fold in rank order 0..P-1 (page "深度学习专题：模型训练的数据并行（三）"
§(四) step 2; the mean of page "高效AI 第19讲" 通信原语 All-Reduce).

The 16-bit mean (the gradient the GPU hands to the CPU in the offload of
page "ZeRO 技术原理：进阶与 Offload" §2.2) must equal the oracle's fp32 mean
rounded to nearest even.

Shards with whole chunks for at least half the CUs take the chunked kernels;
there the oracle runs on a sample of positions (every regime edge plus
random ones), gathered on the device.
"""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for
from zs_synth.gen import normal
from gpu_util import (DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, check_f32, check_param,
                      oracle_step_threaded)

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
GROUP = 256 * 8
CHUNK = 28 * GROUP


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _grads_dev(p, L, dt, seed, std=1e-2):
    return [normal(L, std, seed_for(seed, r), TD[dt], DEV) for r in range(p)]


def _sample(L, n_rand, seed):
    rng = np.random.default_rng(seed)
    pts = set(range(min(L, 64))) | set(range(max(0, L - 64), L))
    for h in (0, 4):
        nvec = (L - h) // 8
        nfull = nvec // (CHUNK // 8)
        for b in (h, h + CHUNK, h + nfull * CHUNK - CHUNK, h + nfull * CHUNK, h + nvec * 8):
            pts |= set(range(max(0, b - 8), min(L, b + 8)))
    pts |= set(int(x) for x in rng.integers(0, L, n_rand))
    return np.array(sorted(pts), np.int64)


@pytest.mark.parametrize("p", [257, 512, 1024])
@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_fused_step_beyond_kernel_arguments_every_element(p, form):
    # small shards (the small-shard kernel), every element against the oracle
    L = 20_011 + 3 * p
    n = L * p - 7
    M, s, e = oracle.plan_shards(n, p)
    k = p // 3
    L = e[k] - s[k]
    gd = _grads_dev(p, L, "f16", 60 + p)
    gb = [u16(g) for g in gd]
    w0 = normal(L, 0.02, seed_for(61, p)).numpy()
    wd = torch.from_numpy(w0.copy()).to(DEV)
    md, vd = torch.zeros_like(wd), torch.zeros_like(wd)
    param_d = torch.empty(L, dtype=torch.float16, device=DEV)
    ws = torch.empty(z.zs_shard_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    wh, mh, vh = w0.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in (1, 2):
        say(f"{p} ranks, shard {k} ({L} elements), step {t}, {form}")
        z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, z.hparams(LR, B1, B2, EPS, t, form),
                              grad_base=s[k], param_base=s[k], workspace=ws)
        ph = oracle_step_threaded("f16", gb, wh, mh, vh, "f16", t, form)
        torch.cuda.synchronize()
        tol = 1e-6 if t == 1 else 2e-6
        d = check_f32(f32(wd), wh, tol, "w") + check_f32(f32(md), mh, tol, "m")
        d += check_f32(f32(vd), vh, tol, "v") + check_param(u16(param_d), ph, "f16", "param")
        assert d == 0, f"{d} elements differ in bits"


def test_fused_step_512_ranks_whole_chunks_sampled():
    # a shard with whole chunks for every CU: the one-workgroup-per-CU kernel
    p, k = 512, 511
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    L = CHUNK * ncu + 3 * GROUP + 13
    n = L * p
    M, s, e = oracle.plan_shards(n, p)
    assert e[k] - s[k] == L
    say(f"512 ranks, shard {k}: {L} elements")
    gd = _grads_dev(p, L, "bf16", 62, std=1e-3)
    w0 = normal(L, 0.02, seed_for(63)).to(DEV)
    wd = w0.clone()
    md, vd = torch.zeros_like(wd), torch.zeros_like(wd)
    param_d = torch.empty(L, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(z.zs_shard_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, z.hparams(LR, B1, B2, EPS, 1),
                          grad_base=s[k], param_base=s[k], workspace=ws)
    idx = _sample(L, 20_000, 64)
    idev = torch.from_numpy(idx).to(DEV)
    gs = [u16(g[idev]) for g in gd]
    wh = f32(w0[idev]).copy()
    mh, vh = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    ph = oracle.step_elems("bf16", gs, wh, mh, vh, "bf16", LR, B1, B2, EPS, 1)
    torch.cuda.synchronize()
    d = check_f32(f32(wd[idev]), wh, 1e-6, "w") + check_f32(f32(md[idev]), mh, 1e-6, "m")
    d += check_f32(f32(vd[idev]), vh, 1e-6, "v")
    d += check_param(u16(param_d[idev]), ph, "bf16", "param")
    assert d == 0, f"{d} sampled values differ in bits"
    assert torch.equal(param_d.view(torch.int16), wd.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("p", [257, 300, 512, 1024])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_mean_in_passes_bit_exact(p, dt):
    L = 30_001 + p
    n = L * p
    M, s, e = oracle.plan_shards(n, p)
    k = p - 1
    gd = _grads_dev(p, L, dt, 65 + p)
    out = torch.full((L,), float("nan"), device=DEV)
    z.zs_reduce_scatter_mean_local(gd, n, p, k, out, grad_base=s[k])
    want = oracle.grad_mean(dt, [u16(g) for g in gd])
    torch.cuda.synchronize()
    assert np.array_equal(f32(out).view(np.uint32), want.view(np.uint32))


def test_mean_in_passes_whole_chunks_sampled():
    p, k = 300, 299
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    L = CHUNK * ncu + 2 * GROUP + 5
    n = L * p
    M, s, e = oracle.plan_shards(n, p)
    gd = _grads_dev(p, L, "f16", 66)
    out = torch.empty(L, device=DEV)
    out16 = torch.empty(L, dtype=torch.bfloat16, device=DEV)
    part = torch.empty(L, device=DEV)
    z.zs_reduce_scatter_mean_local(gd, n, p, k, out, grad_base=s[k])
    z.zs_reduce_scatter_mean_local16(gd, n, p, k, out16, grad_base=s[k], partial=part)
    idx = _sample(L, 20_000, 67)
    idev = torch.from_numpy(idx).to(DEV)
    want = oracle.grad_mean("f16", [u16(g[idev]) for g in gd])
    torch.cuda.synchronize()
    assert np.array_equal(f32(out[idev]).view(np.uint32), want.view(np.uint32))
    assert np.array_equal(u16(out16[idev]), oracle.narrow("bf16", want))
    # every element: the 16-bit mean is the fp32 mean rounded to nearest even
    assert torch.equal(out16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("p", [1, 4, 64, 256, 300])
@pytest.mark.parametrize("gdt,odt", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "f16")])
def test_mean16_matches_rounded_oracle_mean(p, gdt, odt):
    L = 50_003 + 5 * p
    n = L * p + 3
    M, s, e = oracle.plan_shards(n, p)
    k = 0
    L = e[k] - s[k]
    gd = _grads_dev(p, L, gdt, 68 + p)
    out = torch.empty(L, dtype=TD[odt], device=DEV)
    part = torch.empty(L, device=DEV) if p > 256 else None
    z.zs_reduce_scatter_mean_local16(gd, n, p, k, out, grad_base=s[k], partial=part)
    want = oracle.narrow(odt, oracle.grad_mean(gdt, [u16(g) for g in gd]))
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), want)


def test_mean16_whole_chunks_bit_exact():
    p, k = 8, 3
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    L = CHUNK * ncu + 7 * GROUP + 3
    n = L * p
    M, s, e = oracle.plan_shards(n, p)
    gd = _grads_dev(p, L, "bf16", 69, std=1e-3)
    out = torch.empty(L, dtype=torch.bfloat16, device=DEV)
    z.zs_reduce_scatter_mean_local16(gd, n, p, k, out, grad_base=s[k])
    want = oracle.narrow("bf16", oracle.grad_mean("bf16", [u16(g) for g in gd]))
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), want)


def test_fused_step_1024_ranks_across_soft_barriers_sampled():
    # 1024 ranks (pointers from the device workspace), seven rounds of whole
    # chunks on every CU (soft barriers before rounds 3 and 6), then pieces
    # and a ragged tail.  Rank r reads buffer r % 16 (inputs may share
    # memory), which keeps 16 x L values instead of 1024 x L.
    p, k, nbuf = 1024, 1023, 16
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    L = 7 * ncu * CHUNK + 5 * GROUP + 11
    n = L * p
    M, s, e = oracle.plan_shards(n, p)
    assert e[k] - s[k] == L
    say(f"1024 ranks over {nbuf} buffers, shard {k}: {L} elements")
    bufs = _grads_dev(nbuf, L, "f16", 68, std=1e-3)
    gd = [bufs[r % nbuf] for r in range(p)]
    w0 = normal(L, 0.02, seed_for(69)).to(DEV)
    wd = w0.clone()
    md, vd = torch.zeros_like(wd), torch.zeros_like(wd)
    param_d = torch.empty(L, dtype=torch.float16, device=DEV)
    ws = torch.empty(z.zs_shard_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    z.zs_fused_shard_step(n, p, k, gd, wd, md, vd, param_d, z.hparams(LR, B1, B2, EPS, 1),
                          grad_base=s[k], param_base=s[k], workspace=ws)
    idx = np.unique(np.concatenate([
        _sample(L, 6_000, 70),
        np.arange(3 * ncu * CHUNK - 64, 3 * ncu * CHUNK + 64),      # around the first barrier
        np.arange(6 * ncu * CHUNK - 64, 6 * ncu * CHUNK + 64)]))    # and the second
    idev = torch.from_numpy(idx).to(DEV)
    bs = [u16(b[idev]) for b in bufs]
    gs = [bs[r % nbuf] for r in range(p)]
    wh = f32(w0[idev]).copy()
    mh, vh = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    ph = oracle.step_elems("f16", gs, wh, mh, vh, "f16", LR, B1, B2, EPS, 1)
    torch.cuda.synchronize()
    d = check_f32(f32(wd[idev]), wh, 1e-6, "w") + check_f32(f32(md[idev]), mh, 1e-6, "m")
    d += check_f32(f32(vd[idev]), vh, 1e-6, "v")
    d += check_param(u16(param_d[idev]), ph, "f16", "param")
    assert d == 0, f"{d} sampled values differ in bits"
    assert torch.equal(param_d.view(torch.int16), wd.to(torch.float16).view(torch.int16))


def test_mean_in_passes_across_soft_barriers_sampled():
    # 300 ranks: two passes (256 + 44 ranks), each over five rounds of whole
    # chunks (soft barriers before rounds 2 and 4); rank r reads buffer r % 12
    p, k, nbuf = 300, 299, 12
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    L = 5 * ncu * CHUNK + 3 * GROUP + 7
    n = L * p
    M, s, e = oracle.plan_shards(n, p)
    say(f"300-rank mean over {nbuf} buffers: {L} elements")
    bufs = _grads_dev(nbuf, L, "bf16", 71)
    gd = [bufs[r % nbuf] for r in range(p)]
    out = torch.empty(L, device=DEV)
    z.zs_reduce_scatter_mean_local(gd, n, p, k, out, grad_base=s[k])
    idx = np.unique(np.concatenate([
        _sample(L, 6_000, 72),
        np.arange(2 * ncu * CHUNK - 64, 2 * ncu * CHUNK + 64),
        np.arange(4 * ncu * CHUNK - 64, 4 * ncu * CHUNK + 64)]))
    idev = torch.from_numpy(idx).to(DEV)
    bs = [u16(b[idev]) for b in bufs]
    want = oracle.grad_mean("bf16", [bs[r % nbuf] for r in range(p)])
    torch.cuda.synchronize()
    assert np.array_equal(f32(out[idev]).view(np.uint32), want.view(np.uint32))
