"""Bucketed updates: one shard updated bucket by bucket, and HIP-graph replay.

Page "ZeRO 技术原理：进阶与 Offload" §1.5 (bucket strategy): gradients are
reduced in fixed-size buckets as they become ready, so the update of a shard
can run bucket by bucket instead of in one launch.  A bucket here is a run of
consecutive pieces of the shard's tensor list (at least `bucket_elems`
elements), uploaded as its own chunk table.  Checked: the bucketed launches of
a step give the same bits as one launch over the whole shard, and launches
captured once in a HIP graph and replayed (with eager work between replays)
give the same bits as eager launches.  Graph replay reuses the captured
kernel arguments, so it is valid where they do not change between steps: the
SGD forms (Adam's bias corrections depend on the step).
"""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import WORKLOADS, seed_for
from zs_synth.gen import normal
from gpu_util import DEV, LR, B1, B2, EPS, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def group_buckets(pieces, bucket_elems):
    """Consecutive pieces, each group holding at least bucket_elems elements
    (the last group may hold fewer)."""
    out, cur, size = [], [], 0
    for i, pc in enumerate(pieces):
        cur.append(i)
        size += pc[3]
        if size >= bucket_elems:
            out.append(cur)
            cur, size = [], 0
    if cur:
        out.append(cur)
    return out


class Shard:
    """State of one shard of the GPT-2 parameter list (bf16, P = 8)."""

    def __init__(self, k, seed):
        wl = WORKLOADS["gpt2_small_p8"]
        self.numel = [n for _, n in wl.tensors]
        self.p = wl.p
        M, s, e = oracle.plan_shards(wl.n, wl.p)
        self.L = e[k] - s[k]
        self.k = k
        self.w = normal(self.L, 0.02, seed_for(seed, 1)).to(DEV)
        self.m = torch.zeros_like(self.w)
        self.v = torch.zeros_like(self.w)
        self.params = {}
        self.grads = [torch.empty(self.L, dtype=torch.bfloat16, device=DEV) for _ in range(self.p)]
        self.keep = []

    def tables(self, chunk, bucket_elems=None):
        pieces, _ = z.zs_plan_chunks(self.numel, self.p, self.k, chunk)
        for (t, _, _, _) in pieces:
            if t not in self.params:
                self.params[t] = torch.zeros(self.numel[t], dtype=torch.bfloat16, device=DEV)
        groups = [list(range(len(pieces)))] if bucket_elems is None else \
            group_buckets(pieces, bucket_elems)
        out = []
        for g in groups:
            sub = [pieces[i] for i in g]
            ptrs = [dict(w=self.w.data_ptr() + 4 * so, m=self.m.data_ptr() + 4 * so,
                         v=self.v.data_ptr() + 4 * so,
                         param=self.params[t].data_ptr() + 2 * to,
                         grads=[gr.data_ptr() + 2 * so for gr in self.grads])
                    for (t, to, so, ln) in sub]
            nch = sum((ln + chunk - 1) // chunk for (_, _, _, ln) in sub)
            nb = z.zs_mt_workspace_bytes(len(sub), nch, self.p)
            ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
            self.keep.append(ws)
            out.append(z.zs_mt_upload(sub, ptrs, self.p, "bf16", "bf16", chunk, ws, nb))
        return out

    def set_grads(self, t, seed):
        for r in range(self.p):
            self.grads[r].copy_(normal(self.L, 1e-3, seed_for(seed, r, t), torch.bfloat16, DEV))

    def same_as(self, other):
        ok = torch.equal(self.w.view(torch.int32), other.w.view(torch.int32))
        ok = ok and torch.equal(self.m.view(torch.int32), other.m.view(torch.int32))
        ok = ok and torch.equal(self.v.view(torch.int32), other.v.view(torch.int32))
        for t, buf in self.params.items():
            ok = ok and torch.equal(buf.view(torch.int16), other.params[t].view(torch.int16))
        return ok


@pytest.mark.parametrize("form", ["standard", "sgd_momentum"])
def test_bucketed_launches_equal_one_launch(form):
    k = 7
    a, b = Shard(k, 80), Shard(k, 80)
    whole = a.tables(65536)
    buckets = b.tables(65536, bucket_elems=500_000)
    say(f"shard {k}: {len(buckets)} buckets")
    assert len(buckets) >= 8
    for t in (1, 2, 3):
        a.set_grads(t, 81)
        b.set_grads(t, 81)
        hp = z.hparams(LR, B1, B2, EPS, t, form)
        for tb in whole:
            z.zs_fused_shard_step_multi(tb, hp)
        for tb in buckets:
            z.zs_fused_shard_step_multi(tb, hp)
        torch.cuda.synchronize()
        assert a.same_as(b), f"bucketed step differs at t={t}"


def test_graph_replay_of_bucketed_sgd_momentum():
    k = 5
    eager, graphed = Shard(k, 82), Shard(k, 82)
    te = eager.tables(65536, bucket_elems=400_000)
    tg = graphed.tables(65536, bucket_elems=400_000)
    hp = z.hparams(LR, B1, B2, EPS, 1, "sgd_momentum")  # constants do not change with t
    # one eager launch first (the library caches the CU count outside capture)
    graphed.set_grads(0, 83)
    eager.set_grads(0, 83)
    for tb in te:
        z.zs_fused_shard_step_multi(tb, hp)
    for tb in tg:
        z.zs_fused_shard_step_multi(tb, hp)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream().cuda_stream
            for tb in tg:
                z.zs_fused_shard_step_multi(tb, hp, stream=st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert eager.same_as(graphed)  # capture itself ran nothing
    for t in (1, 2, 3, 4):
        eager.set_grads(t, 84)      # eager work between replays
        graphed.set_grads(t, 84)
        for tb in te:
            z.zs_fused_shard_step_multi(tb, hp)
        g.replay()
        torch.cuda.synchronize()
        assert eager.same_as(graphed), f"replay {t} differs from eager launches"
