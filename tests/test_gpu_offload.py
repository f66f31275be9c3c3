"""GPU parity of the optimizer offload pipeline (zs_offload_step) against the
oracle, bit for bit.

Page "ZeRO 技术原理：进阶与 Offload" §2.2 Offload 策略: the GPU sends the
shard's 16-bit gradient to host memory bucket by bucket, the CPU updates the
fp32 master weights and moments and converts to 16 bits, and the 16-bit
parameters go back.  §2.3 扩展性, delayed parameter update: steps 1..N-1
update normally, step N only receives, and from step N+1 the CPU applies the
gradient received the step before.

The oracle replays the same schedule: the gradient of step t is the
rank-order fp32 mean of that step's rank gradients rounded to 16 bits
(oracle grad_mean, then narrow); an update applies the widened 16-bit
gradient with the canonical Adam sequence (oracle adam_apply), its step
count being the number of updates applied so far plus one.
"""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for
from zs_synth.gen import normal
from gpu_util import DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, check_f32, check_param

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
SENTINEL = 0x3C3C


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


class Offload:
    """Device rank gradients and working copy, pinned host state and staging
    for rank k's shard, and the oracle's copy of the host state."""

    def __init__(self, n, p, k, dt, bucket, form, seed, threads=4):
        self.n, self.p, self.k, self.dt, self.bucket, self.form = n, p, k, dt, bucket, form
        M, s, e = oracle.plan_shards(n, p)
        self.s, self.e = s[k], e[k]
        self.L = L = e[k] - s[k]
        self.seed = seed
        self.threads = threads
        self.grads = [torch.empty(L, dtype=TD[dt], device=DEV) for _ in range(p)]
        self.param = torch.empty(n, dtype=TD[dt], device=DEV)
        self.param.view(torch.int16).fill_(SENTINEL)
        self.g16_dev = torch.empty(L, dtype=TD[dt], device=DEV)
        self.partial = torch.empty(L, device=DEV) if p > z.ZS_KERNARG_P else None
        pin = dict(pin_memory=True)
        self.g16_host = [torch.empty(L, dtype=TD[dt], **pin) for _ in range(2)]
        w0 = normal(L, 0.02, seed_for(seed, 1))
        self.w = torch.empty(L, **pin)
        self.w.copy_(w0)
        self.m = torch.zeros(L, **pin)
        self.v = torch.zeros(L, **pin)
        self.param_host = torch.empty(L, dtype=TD[dt], **pin)
        self.d2h = torch.cuda.Stream()
        self.h2d = torch.cuda.Stream()
        # oracle state
        self.wh = w0.numpy().copy()
        self.mh = np.zeros(L, np.float32)
        self.vh = np.zeros(L, np.float32)
        self.ph = None
        self.recv = {}

    def make_grads(self, t):
        bits = []
        for r in range(self.p):
            self.grads[r].copy_(normal(self.L, 1e-2, seed_for(self.seed, 2, r, t), TD[self.dt],
                                       DEV))
            bits.append(u16(self.grads[r]))
        # the 16-bit gradient of step t: the fp32 rank-order mean, rounded
        self.recv[t] = oracle.narrow(self.dt, oracle.grad_mean(self.dt, bits))

    def run(self, t, mode, slot, update_count):
        hp = z.hparams(LR, B1, B2, EPS, update_count, self.form)
        z.zs_offload_step(self.n, self.p, self.k, self.grads, self.param, self.g16_dev,
                          self.g16_host, self.w, self.m, self.v, self.param_host, hp, mode, slot,
                          grad_base=self.s, partial=self.partial, bucket_elems=self.bucket,
                          threads=self.threads, d2h_stream=self.d2h, h2d_stream=self.h2d)

    def oracle_update(self, g_bits, update_count):
        g = oracle.widen(self.dt, g_bits)
        self.ph = oracle.adam_apply(g, self.wh, self.mh, self.vh, self.dt, LR, B1, B2, EPS,
                                    update_count, self.form)

    def check(self, what, received_t=None, slot=None):
        torch.cuda.synchronize()
        d = check_f32(self.w.numpy(), self.wh, 2e-6, f"w {what}")
        d += check_f32(self.m.numpy(), self.mh, 2e-6, f"m {what}")
        d += check_f32(self.v.numpy(), self.vh, 2e-6, f"v {what}")
        par = u16(self.param)
        if self.ph is None:
            assert np.all(par == SENTINEL), f"working copy written before any update ({what})"
        else:
            d += check_param(par[self.s:self.e], self.ph, self.dt, f"param {what}")
        assert np.all(par[:self.s] == SENTINEL) and np.all(par[self.e:] == SENTINEL), \
            f"working copy outside the shard written ({what})"
        if received_t is not None:
            got = self.g16_host[slot].view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(got, self.recv[received_t]), f"received gradient {what}"
        assert d == 0, f"{d} elements differ in bits ({what})"


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("bucket", [0, 65_536, 100_003])
def test_plain_offload_steps_match_oracle(dt, bucket):
    o = Offload(1_000_003, 4, 1, dt, bucket, "standard", seed_for(90, bucket))
    for t in (1, 2, 3):
        o.make_grads(t)
        o.run(t, z.ZS_OFFLOAD_PLAIN, 0, t)
        o.oracle_update(o.recv[t], t)
        o.check(f"t={t}", received_t=t, slot=0)


@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_delayed_parameter_update_ten_steps(form):
    # N = 4: steps 1..3 plain, step 4 receives only, steps 5..10 apply the
    # gradient of the step before while receiving their own
    N, T = 4, 10
    o = Offload(2_000_029, 8, 5, "bf16", 131_072, form, seed_for(91))
    say(f"delayed update, N={N}, {T} steps, shard of {o.L} elements, {form}")
    applied = 0
    for t in range(1, T + 1):
        o.make_grads(t)
        if t < N:
            slot = 0
            o.run(t, z.ZS_OFFLOAD_PLAIN, slot, applied + 1)
            applied += 1
            o.oracle_update(o.recv[t], applied)
        elif t == N:
            slot = 0
            o.run(t, z.ZS_OFFLOAD_RECEIVE, slot, applied + 1)
        else:
            slot = (t - N) % 2           # receive alternately into slots 1, 0, 1, ...
            o.run(t, z.ZS_OFFLOAD_DELAYED, slot, applied + 1)
            applied += 1
            o.oracle_update(o.recv[t - 1], applied)   # the stale gradient of step t-1
        o.check(f"t={t}", received_t=t, slot=slot)
    assert applied == T - 1


def test_offload_beyond_kernel_argument_ranks():
    o = Offload(300 * 4_001, 300, 299, "f16", 1_000, "standard", seed_for(92))
    for t in (1, 2):
        o.make_grads(t)
        o.run(t, z.ZS_OFFLOAD_PLAIN, t % 2, t)
        o.oracle_update(o.recv[t], t)
        o.check(f"t={t}", received_t=t, slot=t % 2)


def test_receive_only_changes_nothing_but_the_received_gradient():
    o = Offload(500_009, 2, 0, "f16", 0, "standard", seed_for(93))
    o.make_grads(1)
    o.run(1, z.ZS_OFFLOAD_RECEIVE, 1, 1)
    o.check("receive", received_t=1, slot=1)   # state, copy untouched; gradient received
