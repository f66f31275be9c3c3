"""The allocation-free fused step (zs_fused_shard_step_static) against the
workspace one (zs_fused_shard_step), bit for bit, through the C ABI.

Above 256 ranks the fused step needs a device table of the rank pointers:
the workspace entry point takes it in caller memory, the allocation-free one
keeps it in a static device array of the library that every call on the GPU
shares.  Two calls in a row, the second with fewer ranks and a smaller
shard, must each give the workspace entry point's bits (so the second call
does not see the first one's table), and a third call with few ranks (no
table at all) too.
"""

import pytest
import torch

from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for
from zs_synth.gen import normal
from gpu_util import DEV, LR, B1, B2, EPS, need_gpu, say

pytestmark = pytest.mark.gpu

CHUNK = 28 * 256 * 8


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _case(p, L, k, seed, form):
    n = L * p
    M, s, e = z.zs_plan_shards(n, p)
    assert e[k] - s[k] == L
    grads = [normal(L, 1e-2, seed_for(seed, r), torch.float16, DEV) for r in range(p)]
    w0 = normal(L, 0.02, seed_for(seed, -1), torch.float32, DEV)
    m0 = normal(L, 1e-3, seed_for(seed, -2), torch.float32, DEV)
    v0 = normal(L, 1e-3, seed_for(seed, -3), torch.float32, DEV).abs_()
    return n, s[k], grads, (w0, m0, v0)


def _run(static, n, p, k, sk, grads, state, t, form):
    w, m, v = (x.clone() for x in state)
    par = torch.zeros(e_minus_s(n, p, k), dtype=torch.float16, device=DEV)
    ws = None if static else torch.empty(max(z.zs_shard_workspace_bytes(p), 16),
                                         dtype=torch.uint8, device=DEV)
    z.zs_fused_shard_step(n, p, k, grads, w, m, v, par, z.hparams(LR, B1, B2, EPS, t, form),
                          grad_base=sk, param_base=sk, workspace=ws, static=static)
    return w, m, v, par


def e_minus_s(n, p, k):
    M, s, e = z.zs_plan_shards(n, p)
    return e[k] - s[k]


def _same(a, b):
    return all(torch.equal(x.view(torch.int32 if x.dtype == torch.float32 else torch.int16),
                           y.view(torch.int32 if y.dtype == torch.float32 else torch.int16))
               for x, y in zip(a, b))


def test_static_scratch_matches_workspace_on_successive_calls():
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    calls = [
        # (ranks, shard length, shard, form): whole chunks, then a smaller
        # shard with fewer ranks (small-shard kernel), then no table at all
        (600, CHUNK * ncu + 5 * 2048 + 3, 599, "standard"),
        (300, 40_009, 7, "page1_literal"),
        (64, 30_011, 3, "standard"),
    ]
    for i, (p, L, k, form) in enumerate(calls):
        say(f"call {i}: {p} ranks, shard {k} of {L} elements, {form}")
        n, sk, grads, state = _case(p, L, k, seed_for(95, i), form)
        got = _run(True, n, p, k, sk, grads, state, 3, form)
        want = _run(False, n, p, k, sk, grads, state, 3, form)
        torch.cuda.synchronize()
        assert _same(got, want), f"call {i}: static-scratch step differs from the workspace step"
        del grads


def test_static_scratch_rejects_too_many_ranks():
    n, p = 2000, z.ZS_MAX_P + 1
    grads = [torch.empty(2, dtype=torch.float16, device=DEV)] * p
    w = torch.zeros(1, device=DEV)
    st = z.zs_fused_shard_step(n, p, 0, grads, w, w, w, torch.zeros(2, dtype=torch.float16,
                                                                    device=DEV),
                               z.hparams(LR, B1, B2, EPS, 1), static=True, check=False)
    assert st == z.ZS_ERR_ARG
