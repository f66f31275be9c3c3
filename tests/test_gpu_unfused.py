"""GPU parity of the unfused pair: zs_reduce_scatter_mean_local (fp32 mean,
bit-exact; small shards by a grid-stride kernel, shards with whole chunks
for at least half the CUs by the chunked kernel) and zs_adam_step, and their
composition against the fused step."""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for
from zs_synth.gen import normal
from zs_synth import make
from gpu_util import DEV, LR, B1, B2, EPS, need_gpu, u16, f32, to_dev_u16, check_f32, check_param

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _bits(n, dt, std, seed):
    return normal(n, std, seed, TD[dt]).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("p", [1, 4, 13, 64, 256])
@pytest.mark.parametrize("layout", ["full", "slice"])
def test_mean_bit_exact(dt, p, layout):
    n = 40_000 + 37 * p
    M, s, e = oracle.plan_shards(n, p)
    k = (p - 1) // 2
    L = e[k] - s[k]
    if layout == "full":
        gb = [_bits(n, dt, 1e-2, seed_for(30, p, r)) for r in range(p)]
        base = 0
        host = [b[s[k]:e[k]] for b in gb]
    else:
        gb = [_bits(L, dt, 1e-2, seed_for(31, p, r)) for r in range(p)]
        base = s[k]
        host = gb
    gd = [to_dev_u16(b, TD[dt]) for b in gb]
    out = torch.full((L,), float("nan"), device=DEV)
    z.zs_reduce_scatter_mean_local(gd, n, p, k, out, grad_base=base)
    torch.cuda.synchronize()
    want = oracle.grad_mean(dt, host)
    assert np.array_equal(f32(out).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("pdt", ["f16", "bf16", None])
@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_adam_step_matches_oracle(pdt, form):
    L = 123_457
    g = normal(L, 1e-2, seed_for(32)).numpy()
    w0 = normal(L, 0.02, seed_for(33)).numpy()
    m0, v0 = (x.numpy() for x in make.random_state(L, 34))
    gd, wd, md, vd = (torch.from_numpy(x.copy()).to(DEV) for x in (g, w0, m0, v0))
    par = torch.empty(L, dtype=TD[pdt], device=DEV) if pdt else None
    for t in (1, 2, 3):
        z.zs_adam_step(gd, wd, md, vd, par, L, z.hparams(LR, B1, B2, EPS, t, form))
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    for t in (1, 2, 3):
        ph = oracle.adam_apply(g, wh, mh, vh, pdt or "f16", LR, B1, B2, EPS, t, form)
    assert check_f32(f32(wd), wh, 2e-6, "w") == 0
    assert check_f32(f32(md), mh, 2e-6, "m") == 0
    assert check_f32(f32(vd), vh, 2e-6, "v") == 0
    if pdt:
        assert check_param(u16(par), ph, pdt, "param") == 0


@pytest.mark.parametrize("gdt", ["f16", "bf16"])
def test_unfused_pair_equals_fused(gdt):
    n, p, k = 300_007, 6, 4
    M, s, e = oracle.plan_shards(n, p)
    L = e[k] - s[k]
    gd = [normal(n, 1e-3, seed_for(35, r), TD[gdt], "cpu").to(DEV) for r in range(p)]
    w0 = normal(L, 0.02, seed_for(36)).to(DEV)
    a = [w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0)]
    b = [w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0)]
    pa = torch.zeros(n, dtype=TD[gdt], device=DEV)
    pb = torch.zeros(L, dtype=TD[gdt], device=DEV)
    g = torch.empty(L, device=DEV)
    for t in (1, 2):
        h = z.hparams(LR, B1, B2, EPS, t)
        z.zs_fused_shard_step(n, p, k, gd, *a, pa, h)
        z.zs_reduce_scatter_mean_local(gd, n, p, k, g)
        z.zs_adam_step(g, *b, pb, L, h)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(pa[s[k]:e[k]].view(torch.int16), pb.view(torch.int16))


@pytest.mark.parametrize("p,dt,regime", [(3, "f16", "rounds_plus_pieces"),
                                         (32, "bf16", "half_round"),
                                         (17, "f16", "all_whole"),
                                         (100, "bf16", "half_round")])
def test_mean_whole_chunk_path(p, dt, regime):
    # shards with whole chunks for at least half the CUs take the chunked mean
    # kernel (one workgroup per CU, the fused kernel's read phase); shard 1
    # starts at an element that is not a multiple of 8, so a head is peeled
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    chunk = 28 * 256 * 8
    chunks = {"rounds_plus_pieces": cu + cu // 4, "half_round": cu // 2,
              "all_whole": cu + (3 * cu) // 4}[regime]
    L = chunks * chunk + 8 * 333 + 5
    n, k = L * p, 1
    M, s, e = oracle.plan_shards(n, p)
    assert e[k] - s[k] == L and s[k] % 8 != 0
    gb = [_bits(L, dt, 1e-2, seed_for(37, p, r)) for r in range(p)]
    gd = [to_dev_u16(b, TD[dt]) for b in gb]
    out = torch.full((L + 16,), float("nan"), device=DEV)
    z.zs_reduce_scatter_mean_local(gd, n, p, k, out[:L], grad_base=s[k])
    torch.cuda.synchronize()
    want = oracle.grad_mean(dt, gb)
    got = f32(out)
    assert np.array_equal(got[:L].view(np.uint32), want.view(np.uint32))
    assert np.isnan(got[L:]).all(), "write past the shard"


@pytest.mark.parametrize("L", [7, 4096, 4096 * 3 + 8 * 5 + 3, 1_000_003])
def test_adam_step_pairs_and_tails(L):
    # the Adam kernel takes two vectors per lane; lengths around that pairing
    g = normal(L, 1e-2, seed_for(38, L)).numpy()
    w0 = normal(L, 0.02, seed_for(39, L)).numpy()
    m0, v0 = (x.numpy() for x in make.random_state(L, 40))
    gd, wd, md, vd = (torch.from_numpy(x.copy()).to(DEV) for x in (g, w0, m0, v0))
    pbuf = torch.zeros(L + 8, dtype=torch.float16, device=DEV)
    z.zs_adam_step(gd, wd, md, vd, pbuf[:L], L, z.hparams(LR, B1, B2, EPS, 2))
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    ph = oracle.adam_apply(g, wh, mh, vh, "f16", LR, B1, B2, EPS, 2)
    assert check_f32(f32(wd), wh, 2e-6, "w") + check_f32(f32(md), mh, 2e-6, "m") == 0
    assert check_f32(f32(vd), vh, 2e-6, "v") == 0
    assert check_param(u16(pbuf[:L]), ph, "f16", "param") == 0
    assert not u16(pbuf[L:]).any(), "write past the shard"


@pytest.mark.parametrize("with_param,off", [(True, 3), (False, 0)])
def test_adam_step_whole_chunk_path(with_param, off):
    # shards with whole chunks for at least half the CUs take the chunked Adam
    # kernel; the arrays start `off` elements into their buffers (a head of
    # scalar elements when the start is not 8-aligned)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    L = (cu + cu // 4) * 28 * 256 * 8 + 8 * 333 + 5
    g = normal(L, 1e-2, seed_for(41, off)).numpy()
    w0 = normal(L, 0.02, seed_for(42, off)).numpy()
    m0, v0 = (x.numpy() for x in make.random_state(L, 43))

    def dev(x):
        buf = torch.zeros(L + off, dtype=torch.float32, device=DEV)
        buf[off:].copy_(torch.from_numpy(x))
        return buf[off:]

    gd, wd, md, vd = dev(g), dev(w0), dev(m0), dev(v0)
    pbuf = torch.zeros(L + off + 8, dtype=torch.bfloat16, device=DEV)
    par = pbuf[off:off + L] if with_param else None
    for t in (1, 2):
        z.zs_adam_step(gd, wd, md, vd, par, L, z.hparams(LR, B1, B2, EPS, t, "page1_literal"),
                       param_dtype=None if with_param else "bf16")
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    for t in (1, 2):
        ph = oracle.adam_apply(g, wh, mh, vh, "bf16", LR, B1, B2, EPS, t, "page1_literal")
    d = check_f32(f32(wd), wh, 2e-6, "w") + check_f32(f32(md), mh, 2e-6, "m")
    d += check_f32(f32(vd), vh, 2e-6, "v")
    if with_param:
        d += check_param(u16(par), ph, "bf16", "param")
        canary = u16(pbuf)
        assert not canary[:off].any() and not canary[off + L:].any(), "write outside the shard"
    assert d == 0


@pytest.mark.parametrize("case", range(12))
def test_adam_step_alignment_sweep(case):
    # every array at its own element offset within a 128-byte line (fp32:
    # 0-31 elements, the 16-bit working copy: 0-63): the head (0-7 scalar
    # elements) follows the alignment; every element must match the oracle.
    # Cases 8-11 take the whole-chunk kernel with the state on whole lines
    # and the working copy 40 / 8 / 2 / 4 bytes into one (rank 63's slice of
    # the 7.5B-parameter working copy sits 40 bytes in; the copy is staged in
    # LDS and written out on whole lines, 2- and 4-byte offsets through the
    # element-wise flush).
    rng = np.random.default_rng(100 + case)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if case < 8:
        L = 50_021 + case * 997
        go, wo, mo, vo = (int(x) for x in rng.integers(0, 32, 4))
        po = int(rng.integers(0, 64))
    else:
        L = (cu // 2 + 3) * 28 * 256 * 8 + 8 * 29 + 3
        go = wo = mo = vo = 0
        po = {8: 20, 9: 4, 10: 1, 11: 2}[case]
    g = normal(L, 1e-2, seed_for(44, case)).numpy()
    w0 = normal(L, 0.02, seed_for(45, case)).numpy()
    m0, v0 = (x.numpy() for x in make.random_state(L, 46 + case))

    def dev(x, off):
        buf = torch.zeros(L + 32, dtype=torch.float32, device=DEV)
        assert buf.data_ptr() % 128 == 0
        buf[off:off + L].copy_(torch.from_numpy(x))
        return buf[off:off + L]

    gd, wd, md, vd = dev(g, go), dev(w0, wo), dev(m0, mo), dev(v0, vo)
    pbuf = torch.zeros(L + 64, dtype=torch.float16, device=DEV)
    par = pbuf[po:po + L]
    z.zs_adam_step(gd, wd, md, vd, par, L, z.hparams(LR, B1, B2, EPS, 3))
    torch.cuda.synchronize()
    wh, mh, vh = w0.copy(), m0.copy(), v0.copy()
    ph = oracle.adam_apply(g, wh, mh, vh, "f16", LR, B1, B2, EPS, 3)
    d = check_f32(f32(wd), wh, 2e-6, "w") + check_f32(f32(md), mh, 2e-6, "m")
    d += check_f32(f32(vd), vh, 2e-6, "v") + check_param(u16(par), ph, "f16", "param")
    assert d == 0
    canary = u16(pbuf)
    assert not canary[:po].any() and not canary[po + L:].any(), "write outside the slice"
