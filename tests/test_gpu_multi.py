"""GPU parity of the multi-tensor chunk-table step (zs_plan_chunks +
zs_mt_upload + zs_fused_shard_step_multi) against the oracle, whose map from
shard index to (tensor, offset) comes from prefix sums over the tensor list,
not from the chunk table."""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import seed_for, gpt2_small_tensors, WORKLOADS
from zs_synth.gen import normal
from zs_synth import make
from gpu_util import (DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, check_f32, check_param,
                      oracle_step_threaded)

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
SENTINEL = 0x4B4B


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


class MtCase:
    """Device buffers of one rank's shard over a flattened tensor list:
    rank slices of the shard (gradients), flat shard-local w/m/v, and one
    16-bit working-copy tensor per parameter tensor the shard touches."""

    def __init__(self, numel, p, k, gdt, pdt, chunk, seed):
        self.numel, self.p, self.k, self.gdt, self.pdt = numel, p, k, gdt, pdt
        n = sum(numel)
        self.n = n
        M, s, e = oracle.plan_shards(n, p)
        self.s, self.e = s[k], e[k]
        self.L = L = e[k] - s[k]
        self.pieces, self.nchunks = z.zs_plan_chunks(numel, p, k, chunk)
        assert self.pieces == oracle.shard_pieces(numel, s[k], e[k])
        self.w0 = normal(L, 0.02, seed_for(seed, 1))
        self.w = self.w0.to(DEV)
        self.m = torch.zeros_like(self.w)
        self.v = torch.zeros_like(self.w)
        self.params = {}
        for (t, to, so, ln) in self.pieces:
            if t not in self.params:
                buf = torch.empty(numel[t], dtype=TD[pdt], device=DEV)
                buf.view(torch.int16).fill_(SENTINEL)
                self.params[t] = buf
        self.grads = [torch.empty(max(L, 1), dtype=TD[gdt], device=DEV) for _ in range(p)]
        ptrs = []
        esz = 2
        for (t, to, so, ln) in self.pieces:
            ptrs.append(dict(w=self.w.data_ptr() + 4 * so, m=self.m.data_ptr() + 4 * so,
                             v=self.v.data_ptr() + 4 * so,
                             param=self.params[t].data_ptr() + esz * to,
                             grads=[g.data_ptr() + esz * so for g in self.grads]))
        nb = z.zs_mt_workspace_bytes(len(self.pieces), self.nchunks, p)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        self.table = z.zs_mt_upload(self.pieces, ptrs, p, gdt, pdt, chunk, self.ws, nb)
        assert self.table.nchunks == self.nchunks

    def set_grads(self, step, seed):
        self.gbits = []
        for r in range(self.p):
            g = normal(self.L, 1e-3, seed_for(seed, 2, r, step), TD[self.gdt])
            self.grads[r][:self.L].copy_(g.to(DEV))
            self.gbits.append(g.view(torch.int16).numpy().view(np.uint16))

    def step(self, t, form="standard"):
        z.zs_fused_shard_step_multi(self.table, z.hparams(LR, B1, B2, EPS, t, form))


def _scatter(case, flat_bits):
    """Per-tensor expected working copies from a shard-flat result, using the
    oracle's prefix-sum map (pieces)."""
    out = {t: np.full(case.numel[t], SENTINEL, np.uint16) for t in case.params}
    for (t, to, so, ln) in oracle.shard_pieces(case.numel, case.s, case.e):
        out[t][to:to + ln] = flat_bits[so:so + ln]
    return out


def _run_and_check(case, steps, seed, form="standard", check_every=True):
    wh = case.w0.numpy().copy()
    mh = np.zeros_like(wh)
    vh = np.zeros_like(wh)
    for t in range(1, steps + 1):
        case.set_grads(t, seed)
        case.step(t, form)
        ph = oracle_step_threaded(case.gdt, case.gbits, wh, mh, vh, case.pdt, t, form)
        if check_every or t == steps:
            torch.cuda.synchronize()
            tol = 1e-6 if t == 1 else 2e-6
            d = check_f32(f32(case.w), wh, tol, f"w t={t}")
            d += check_f32(f32(case.m), mh, tol, f"m t={t}")
            d += check_f32(f32(case.v), vh, tol, f"v t={t}")
            exp = _scatter(case, ph)
            for tt, buf in case.params.items():
                d += check_param(u16(buf), exp[tt], case.pdt, f"param tensor {tt} t={t}")
            assert d == 0, f"{d} elements differ in bits at t={t}"


@pytest.mark.parametrize("seed", range(4))
def test_random_tensor_lists_all_shards(seed):
    rng = np.random.default_rng(seed)
    numel = [int(x) for x in rng.integers(0, 3000, 40)]
    numel[5] = 0
    numel[7] = 1
    numel += [50_001, 7, 123_457]
    p = [2, 3, 5, 8][seed]
    for k in range(p):
        case = MtCase(numel, p, k, ["f16", "bf16"][seed % 2], ["f16", "bf16"][seed % 2],
                      [64, 1024, 4096, 65536][seed], seed_for(40, seed, k))
        _run_and_check(case, 2, seed_for(41, seed, k))


def _bench_chunk(numel, p, k):
    """The chunk length bench.py uses for rank k's shard (zs_mt_chunk_elems)."""
    M, s, e = oracle.plan_shards(sum(numel), p)
    npieces = len(z.zs_plan_chunks(numel, p, k, 8)[0])
    return z.zs_mt_chunk_elems(e[k] - s[k], npieces)


@pytest.mark.parametrize("chunk_rule", ["bench", "65536"])
def test_gpt2_small_shapes_shard0_ten_steps(chunk_rule):
    wl = WORKLOADS["gpt2_small_p8"]
    numel = [n for _, n in wl.tensors]
    chunk = _bench_chunk(numel, wl.p, 0) if chunk_rule == "bench" else 65536
    if chunk_rule == "bench":
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        assert ncu != 256 or chunk == 61_440
    case = MtCase(numel, wl.p, 0, wl.grad_dtype, wl.param_dtype, chunk, 42)
    assert len(case.pieces) == 1
    say(f"gpt2 shard 0: 10 steps, chunk {chunk}")
    _run_and_check(case, wl.steps, 43, check_every=False)


@pytest.mark.parametrize("chunk_rule", ["bench", "65536"])
@pytest.mark.parametrize("k", [2, 7])
def test_gpt2_small_shapes_many_pieces(k, chunk_rule):
    wl = WORKLOADS["gpt2_small_p8"]
    numel = [n for _, n in wl.tensors]
    chunk = _bench_chunk(numel, wl.p, k) if chunk_rule == "bench" else 65536
    case = MtCase(numel, wl.p, k, wl.grad_dtype, wl.param_dtype, chunk, 44 + k)
    assert len(case.pieces) in (15, 35)
    say(f"gpt2 shard {k}: {len(case.pieces)} pieces, chunk {chunk}, 2 steps")
    _run_and_check(case, 2, 46 + k)


def test_table_at_1024_ranks():
    # the chunk table stages up to ZS_MAX_P gradient pointers per entry in LDS
    numel = [30_011, 7, 52_001]
    p, k = 1024, 370           # M = 81: the shard crosses all three tensors
    case = MtCase(numel, p, k, "bf16", "bf16", 2048, 50)
    assert [pc[3] for pc in case.pieces] == [41, 7, 33]
    say(f"1024 ranks: shard {k}, pieces {[pc[3] for pc in case.pieces]}")
    _run_and_check(case, 2, 51)


def test_multi_equals_single_tensor_step():
    # one tensor, one piece: the table path and the single-shard path agree bit for bit
    n, p, k = 500_009, 4, 2
    case = MtCase([n], p, k, "bf16", "bf16", 8192, 47)
    case.set_grads(1, 48)
    case.step(1)
    w = case.w0.to(DEV)
    m, v = torch.zeros_like(w), torch.zeros_like(w)
    par = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    par.view(torch.int16).fill_(SENTINEL)
    z.zs_fused_shard_step(n, p, k, case.grads, w, m, v, par, z.hparams(LR, B1, B2, EPS, 1),
                          grad_base=case.s)
    torch.cuda.synchronize()
    assert torch.equal(w.view(torch.int32), case.w.view(torch.int32))
    assert torch.equal(par.view(torch.int16), case.params[0].view(torch.int16))


def test_two_hundred_ranks_with_whole_chunks():
    # 200 ranks (table entries stage 200 gradient pointers each) and a shard
    # that crosses a 7-element tensor: whole kernel chunks in the large pieces,
    # then their remainders and the tiny piece
    numel = [1_000_003, 35_999_997, 7, 22_999_993]
    p, k = 200, 123
    case = MtCase(numel, p, k, "f16", "f16", 28 * 256 * 8, 48)
    assert [pc[3] for pc in case.pieces] == [100_000, 7, 199_993]
    say(f"200 ranks: shard {k}, pieces {[pc[3] for pc in case.pieces]}, {case.nchunks} chunks")
    _run_and_check(case, 2, 49)


@pytest.mark.parametrize("k,npieces", [(1, 1), (3, 25), (4, 27), (5, 25), (6, 26)])
def test_gpt2_small_shapes_remaining_shards(k, npieces):
    # the other ranks of the 8-way GPT-2 sharding, at the chunk length bench.py
    # uses (short entries for the many-piece shards)
    wl = WORKLOADS["gpt2_small_p8"]
    numel = [n for _, n in wl.tensors]
    chunk = _bench_chunk(numel, wl.p, k)
    case = MtCase(numel, wl.p, k, wl.grad_dtype, wl.param_dtype, chunk, 60 + k)
    assert len(case.pieces) == npieces
    say(f"gpt2 shard {k}: {npieces} pieces, chunk {chunk}, 2 steps")
    _run_and_check(case, 2, 70 + k)


def test_table_across_soft_barriers_by_value_and_step_table():
    # A table of 24 rounds of whole chunks (one 57,344-element entry per CU
    # and round) passes three soft barriers per launch.  Launched with its
    # constants by value and through a step table, from the same inputs and
    # state, the two must agree bit for bit, and sampled elements (every
    # round's first and last chunks, around the barriers) must match the
    # oracle.
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    chunk = 28 * 256 * 8
    p = 2
    L = 24 * ncu * chunk + 12_345            # 24 full rounds and a ragged tail
    numel = [L * p]
    say(f"soft-barrier table: {L} elements per shard, {24 * ncu} whole chunks")
    cases = [MtCase(numel, p, 1, "bf16", "bf16", chunk, 81) for _ in range(2)]
    assert cases[0].nchunks >= 24 * ncu
    for c in cases:
        c.set_grads(1, 82)
    hp = z.hparams(LR, B1, B2, EPS, 1)
    z.zs_fused_shard_step_multi(cases[0].table, hp)
    nb = z.zs_step_table_bytes(1)
    stdev = torch.empty(nb, dtype=torch.uint8, device=DEV)
    steps = z.zs_step_table_init(hp, p, 1, stdev, nb)
    z.zs_fused_shard_step_multi_dev(cases[1].table, steps)
    torch.cuda.synchronize()
    for name in ("w", "m", "v"):
        a, b = getattr(cases[0], name), getattr(cases[1], name)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    pa, pb = cases[0].params[0], cases[1].params[0]
    assert torch.equal(pa.view(torch.int16), pb.view(torch.int16))
    # oracle on sampled elements of the shard: the first and last chunks of
    # the first round, rounds 5-7 around the first barrier, the last round and
    # the tail
    c0 = cases[0]
    idx = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(chunk - 64, chunk + 64),
        np.arange((ncu - 1) * chunk, ncu * chunk, 997),
        np.arange(5 * ncu * chunk, 8 * ncu * chunk, 7919),
        np.arange(23 * ncu * chunk, 23 * ncu * chunk + 4096, 13),
        np.arange(L - 12_345, L)]))
    gb = [g[idx] for g in c0.gbits]
    wh = c0.w0.numpy()[idx].copy()
    mh = np.zeros_like(wh)
    vh = np.zeros_like(wh)
    ph = oracle_step_threaded("bf16", gb, wh, mh, vh, "bf16", 1, "standard")
    d = check_f32(f32(c0.w)[idx], wh, 1e-6, "w")
    d += check_f32(f32(c0.m)[idx], mh, 1e-6, "m")
    d += check_f32(f32(c0.v)[idx], vh, 1e-6, "v")
    d += check_param(u16(pa)[c0.s + idx], ph, "bf16", "param")
    assert d == 0


def test_long_table_graph_replays_equal_eager_launches():
    # The same 24-round table with its constants by value, captured in a HIP
    # graph: its soft-barrier counters need no clearing between launches, so
    # two replays must equal two eager launches of the same step on a copy
    # with the same state.
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    chunk = 28 * 256 * 8
    p = 2
    L = 24 * ncu * chunk + 777
    numel = [L * p]
    say(f"captured long table: {L} elements per shard")
    eager, graphed = (MtCase(numel, p, 1, "bf16", "bf16", chunk, 83) for _ in range(2))
    for c in (eager, graphed):
        c.set_grads(1, 84)
    hp = z.hparams(LR, B1, B2, EPS, 1)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            z.zs_fused_shard_step_multi(graphed.table, hp,
                                        stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(graphed.w, graphed.w0.to(DEV))  # capture ran nothing
    for rep in range(2):
        z.zs_fused_shard_step_multi(eager.table, hp)
        g.replay()
        torch.cuda.synchronize()
        for name in ("w", "m", "v"):
            a, b = getattr(eager, name), getattr(graphed, name)
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (rep, name)
        assert torch.equal(eager.params[0].view(torch.int16), graphed.params[0].view(torch.int16)), rep


def test_concurrent_tables_share_soft_barriers():
    # Two 12-round tables (two soft barriers each) stepped at once on two
    # streams share the soft-barrier counters, which only pace the
    # workgroups: each result must equal the same table stepped alone.
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    chunk = 28 * 256 * 8
    p = 2
    L = 12 * ncu * chunk + 4321
    say(f"two concurrent tables: {L} elements per shard")
    alone = [MtCase([L * p], p, 1, "bf16", "bf16", chunk, 85 + i) for i in range(2)]
    together = [MtCase([L * p], p, 1, "bf16", "bf16", chunk, 85 + i) for i in range(2)]
    for i, c in enumerate(alone + together):
        c.set_grads(1, 90 + i % 2)
    hp = z.hparams(LR, B1, B2, EPS, 1)
    for c in alone:
        z.zs_fused_shard_step_multi(c.table, hp)
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in together]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for c, s_ in zip(together, streams):
        z.zs_fused_shard_step_multi(c.table, hp, stream=s_.cuda_stream)
    torch.cuda.synchronize()
    for a, b in zip(alone, together):
        for name in ("w", "m", "v"):
            assert torch.equal(getattr(a, name).view(torch.int32), getattr(b, name).view(torch.int32)), name
        assert torch.equal(a.params[0].view(torch.int16), b.params[0].view(torch.int16))
