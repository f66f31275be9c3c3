"""GPU parity across the single-tensor kernel's work-split regimes, every
element checked against the oracle.

The kernel runs whole chunks (28 vectors of 8 elements per lane, 57,344
elements per block) in balanced rounds over its blocks (one per CU), keeps a
last partial round only when it fills at least half of the blocks, and
deals the rest out as two-vector pieces.  A shard under half a whole chunk
per CU goes to the small-shard kernel instead (pieces only, three
workgroups per CU).  The shard lengths below are chosen
from the device's CU count to land in each regime: a last round under half
full (whole rounds + pieces), one over half full (whole chunks only, plus a
short tail), a shard smaller than one round (pieces only), and lengths that
leave every head / scalar-tail combination.
"""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for
from zs_synth.gen import normal
from gpu_util import DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, check_f32, check_param, \
    oracle_step_threaded

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
CHUNK = 28 * 256 * 8


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _run(L, p, gdt, steps, seed, offset=0):
    """Shard k = 0 of n = L * p with slice-layout gradients; the working copy
    is written at `offset` elements into a larger buffer (alignment)."""
    n = L * p
    M, s, e = z.zs_plan_shards(n, p)
    assert e[0] - s[0] == L
    w0 = normal(L, 0.02, seed_for(seed, 1))
    w, m, v = w0.to(DEV), torch.zeros(L, device=DEV), torch.zeros(L, device=DEV)
    parbuf = torch.zeros(L + 16, dtype=TD[gdt], device=DEV)
    par = parbuf[offset:offset + L]
    wh, mh, vh = w0.numpy().copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in range(1, steps + 1):
        gh = [normal(L, 1e-3, seed_for(seed, 2, r, t), TD[gdt]) for r in range(p)]
        gd = [g.to(DEV) for g in gh]
        z.zs_fused_shard_step(n, p, 0, gd, w, m, v, par, z.hparams(LR, B1, B2, EPS, t),
                              grad_base=0, param_base=0)
        bits = [g.view(torch.int16).numpy().view(np.uint16) for g in gh]
        ph = oracle_step_threaded(gdt, bits, wh, mh, vh, gdt, t)
    torch.cuda.synchronize()
    d = check_f32(f32(w), wh, 2e-6, "w") + check_f32(f32(m), mh, 2e-6, "m")
    d += check_f32(f32(v), vh, 2e-6, "v") + check_param(u16(par), ph, gdt, "param")
    assert d == 0, f"{d} elements differ in bits"
    canary = u16(parbuf)
    assert not canary[:offset].any() and not canary[offset + L:].any(), "write outside the shard"


@pytest.mark.parametrize("regime", ["rounds_plus_pieces", "all_whole", "pieces_only"])
def test_work_split_regimes(regime):
    cu = _cu()
    rounds_whole = {"rounds_plus_pieces": cu + cu // 4,     # last round a quarter full
                    "all_whole": cu + (3 * cu) // 4,       # last round three quarters full
                    "pieces_only": cu // 3}[regime]
    L = rounds_whole * CHUNK + 8 * 333 + 5
    say(f"{regime}: {rounds_whole} whole chunks' worth on {cu} CUs, L={L}")
    _run(L, 2, "f16", 2, seed_for(60, len(regime)))


@pytest.mark.parametrize("tail,offset", [(0, 0), (1, 3), (7, 1), (3, 4), (6, 6)])
def test_work_split_heads_and_tails(tail, offset):
    cu = _cu()
    L = (cu // 2) * CHUNK + 8 * 511 + tail
    _run(L, 3, "bf16", 1, seed_for(61, tail, offset), offset=offset)


@pytest.mark.parametrize("p", [1, 5, 19])
def test_small_shard_kernel(p):
    # just under half a whole chunk per CU: the small-shard kernel (three
    # workgroups per CU, ranks in batches of 4: 19 = 4 + 4 + 4 + 4 + 3)
    cu = _cu()
    L = (cu // 2 - 1) * CHUNK + 8 * 77 + 3
    say(f"small-shard kernel: L={L}, p={p} on {cu} CUs")
    _run(L, p, "bf16", 2, seed_for(62, p), offset=p % 4)


@pytest.mark.parametrize("p", [65, 128])
def test_whole_chunks_beyond_64_ranks(p):
    # more than 64 ranks takes the kernel instance with room for 256 gradient
    # pointers; a shard with whole chunks for half the CUs and one more runs
    # its whole-chunk rank loop, then the pieces and a ragged tail
    cu = _cu()
    L = (cu // 2 + 1) * CHUNK + 8 * 21 + 3
    say(f"whole chunks at {p} ranks: L={L} on {cu} CUs")
    _run(L, p, "f16", 1, seed_for(63, p), offset=1)


def test_rounds_across_soft_barriers():
    # four rounds of whole chunks (the last half full) take one soft barrier,
    # after the third round; every element against the oracle
    cu = _cu()
    L = (3 * cu + cu // 2) * CHUNK + 8 * 37 + 6
    say(f"rounds across a soft barrier: L={L} on {cu} CUs")
    _run(L, 2, "f16", 1, seed_for(64, 1), offset=2)


def test_concurrent_steps_share_soft_barriers():
    # Two shards stepped at once on two streams share the soft-barrier
    # counters (they only pace the workgroups): each result must equal the
    # same step run alone.
    cu = _cu()
    L = 7 * cu * CHUNK + 8 * 3 + 1          # seven rounds: two barriers
    n, p = 2 * L, 2
    say(f"two concurrent shard steps: L={L} on {cu} CUs")
    runs = []
    for i in range(2):
        g = [normal(L, 1e-3, seed_for(65, i, r), torch.float16).to(DEV) for r in range(p)]
        w0 = normal(L, 0.02, seed_for(65, i, 9)).to(DEV)
        runs.append([g, w0])
    def state(w0):
        return [w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0),
                torch.zeros(L, dtype=torch.float16, device=DEV)]
    hp = z.hparams(LR, B1, B2, EPS, 1)
    alone = []
    for g, w0 in runs:
        st = state(w0)
        z.zs_fused_shard_step(n, p, 0, g, *st, hp, grad_base=0, param_base=0)
        torch.cuda.synchronize()
        alone.append(st)
    together = [state(w0) for _, w0 in runs]
    streams = [torch.cuda.Stream() for _ in runs]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for (g, _), st, s_ in zip(runs, together, streams):
        z.zs_fused_shard_step(n, p, 0, g, *st, hp, grad_base=0, param_base=0,
                              stream=s_.cuda_stream)
    torch.cuda.synchronize()
    for a, b in zip(alone, together):
        for x, y in zip(a[:3], b[:3]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(a[3].view(torch.int16), b[3].view(torch.int16))
