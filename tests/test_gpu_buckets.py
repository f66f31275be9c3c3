"""Bucketed updates: one shard updated bucket by bucket, and HIP-graph replay.

Page "ZeRO 技术原理：进阶与 Offload" §1.5 (bucket strategy): gradients are
reduced in fixed-size buckets as they become ready, so the update of a shard
can run bucket by bucket instead of in one launch.  A bucket here is a run of
consecutive pieces of the shard's tensor list (zs_plan_buckets), uploaded as
its own chunk table with the chunk length zs_mt_chunk_elems gives for the
bucket on its own: the rule bench.py --bucket-elems times.

Checked against the oracle element by element: bucketed standard and
page-1-literal Adam steps; the same launches captured once in a HIP graph
(with the step constants read from a device step table and advanced by a
one-thread kernel inside the graph) and replayed; the step table's
exhausted flag.  Checked HIP against HIP: bucketed launches give the bits of
one launch over the whole shard, and momentum-SGD launches (constants that do
not change with the step) replay from by-value arguments.
"""

import numpy as np
import pytest
import torch

from adam_zs_shard_amd import zshard as z
from zs_synth import WORKLOADS, seed_for
from zs_synth.gen import normal
import oracle
from gpu_util import (DEV, LR, B1, B2, EPS, need_gpu, say, u16, f32, check_f32, check_param,
                      oracle_step_threaded)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


class Shard:
    """State of one shard of the GPT-2 parameter list (bf16, P = 8)."""

    def __init__(self, k, seed):
        wl = WORKLOADS["gpt2_small_p8"]
        self.numel = [n for _, n in wl.tensors]
        self.p = wl.p
        M, s, e = oracle.plan_shards(wl.n, wl.p)
        self.L = e[k] - s[k]
        self.k = k
        self.w0 = normal(self.L, 0.02, seed_for(seed, 1))
        self.w = self.w0.to(DEV)
        self.m = torch.zeros_like(self.w)
        self.v = torch.zeros_like(self.w)
        self.params = {}
        self.grads = [torch.empty(self.L, dtype=torch.bfloat16, device=DEV) for _ in range(self.p)]
        self.keep = []
        self.pieces = None

    def tables(self, bucket_elems=None, chunk=None):
        """One chunk table for the whole shard, or one per bucket; chunk
        lengths by zs_mt_chunk_elems unless given."""
        probe, _ = z.zs_plan_chunks(self.numel, self.p, self.k, 8)
        self.pieces = probe
        for (t, _, _, _) in probe:
            if t not in self.params:
                self.params[t] = torch.zeros(self.numel[t], dtype=torch.bfloat16, device=DEV)
        if bucket_elems is None:
            groups = [list(range(len(probe)))]
        else:
            of, nb = z.zs_plan_buckets(probe, bucket_elems)
            groups = [[i for i in range(len(probe)) if of[i] == b] for b in range(nb)]
        out = []
        for g in groups:
            sub = [probe[i] for i in g]
            lb = sum(pc[3] for pc in sub)
            ce = chunk or z.zs_mt_chunk_elems(lb, 1 if bucket_elems else len(sub))
            ptrs = [dict(w=self.w.data_ptr() + 4 * so, m=self.m.data_ptr() + 4 * so,
                         v=self.v.data_ptr() + 4 * so,
                         param=self.params[t].data_ptr() + 2 * to,
                         grads=[gr.data_ptr() + 2 * so for gr in self.grads])
                    for (t, to, so, ln) in sub]
            nch = sum((ln + ce - 1) // ce for (_, _, _, ln) in sub)
            nb_ = z.zs_mt_workspace_bytes(len(sub), nch, self.p)
            ws = torch.empty(nb_, dtype=torch.uint8, device=DEV)
            self.keep.append(ws)
            out.append(z.zs_mt_upload(sub, ptrs, self.p, "bf16", "bf16", ce, ws, nb_))
        return out

    def set_grads(self, t, seed):
        self.gbits = []
        for r in range(self.p):
            g = normal(self.L, 1e-3, seed_for(seed, r, t), torch.bfloat16)
            self.grads[r].copy_(g.to(DEV))
            self.gbits.append(g.view(torch.int16).numpy().view(np.uint16))

    def same_as(self, other):
        ok = torch.equal(self.w.view(torch.int32), other.w.view(torch.int32))
        ok = ok and torch.equal(self.m.view(torch.int32), other.m.view(torch.int32))
        ok = ok and torch.equal(self.v.view(torch.int32), other.v.view(torch.int32))
        for t, buf in self.params.items():
            ok = ok and torch.equal(buf.view(torch.int16), other.params[t].view(torch.int16))
        return ok


class Ref:
    """The oracle's copy of a shard's state, stepped on the host."""

    def __init__(self, sh):
        self.sh = sh
        self.w = sh.w0.numpy().copy()
        self.m = np.zeros_like(self.w)
        self.v = np.zeros_like(self.w)

    def step(self, t, form):
        self.param = oracle_step_threaded("bf16", self.sh.gbits, self.w, self.m, self.v, "bf16",
                                          t, form)

    def check(self, what, tol=2e-6):
        sh = self.sh
        torch.cuda.synchronize()
        d = check_f32(f32(sh.w), self.w, tol, f"w {what}")
        d += check_f32(f32(sh.m), self.m, tol, f"m {what}")
        d += check_f32(f32(sh.v), self.v, tol, f"v {what}")
        for (t, to, so, ln) in oracle.shard_pieces(sh.numel, *self._bounds()):
            d += check_param(u16(sh.params[t][to:to + ln]), self.param[so:so + ln], "bf16",
                             f"param tensor {t} {what}")
        assert d == 0, f"{d} elements differ in bits ({what})"

    def _bounds(self):
        M, s, e = oracle.plan_shards(sum(self.sh.numel), self.sh.p)
        return s[self.sh.k], e[self.sh.k]


@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_bucketed_adam_matches_oracle(form):
    k = 7
    sh = Shard(k, 80)
    buckets = sh.tables(bucket_elems=500_000)
    say(f"shard {k}: {len(sh.pieces)} pieces in {len(buckets)} buckets, {form}")
    assert len(buckets) >= 8
    ref = Ref(sh)
    for t in (1, 2, 3):
        sh.set_grads(t, 81)
        hp = z.hparams(LR, B1, B2, EPS, t, form)
        for tb in buckets:
            z.zs_fused_shard_step_multi(tb, hp)
        ref.step(t, form)
        ref.check(f"t={t}")


@pytest.mark.parametrize("form", ["standard", "sgd_momentum"])
def test_bucketed_launches_equal_one_launch(form):
    k = 7
    a, b = Shard(k, 80), Shard(k, 80)
    whole = a.tables()
    buckets = b.tables(bucket_elems=2_000_000)
    assert len(buckets) >= 4
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


def _capture(launch):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("form", ["standard", "page1_literal"])
def test_graph_replay_of_bucketed_adam_matches_oracle(form):
    k = 5
    sh = Shard(k, 82)
    tables = sh.tables(bucket_elems=400_000)
    say(f"shard {k}: {len(tables)} buckets captured once, replayed 4 times, {form}")
    nsteps = 4
    nbytes = z.zs_step_table_bytes(nsteps)
    st_buf = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    steps = z.zs_step_table_init(z.hparams(LR, B1, B2, EPS, 1, form), sh.p, nsteps, st_buf,
                                 nbytes)
    assert (steps.first_step, steps.nsteps, steps.form) == (1, 4, z.FORMS[form])

    def launch(s):
        for tb in tables:
            z.zs_fused_shard_step_multi_dev(tb, steps, stream=s)
        z.zs_step_table_advance(steps, stream=s)

    g = _capture(launch)
    assert z.zs_step_table_status(steps) == (0, 0)   # capture itself ran nothing
    ref = Ref(sh)
    for t in range(1, nsteps + 1):
        sh.set_grads(t, 83)      # eager work between replays
        g.replay()
        ref.step(t, form)
        ref.check(f"replay {t}")
        assert z.zs_step_table_status(steps) == (t, 0)


def test_step_table_exhausted_leaves_state_alone():
    k = 5
    sh = Shard(k, 84)
    tables = sh.tables(bucket_elems=2_000_000)
    nbytes = z.zs_step_table_bytes(2)
    st_buf = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    steps = z.zs_step_table_init(z.hparams(LR, B1, B2, EPS, 3, "standard"), sh.p, 2, st_buf,
                                 nbytes)
    ref = Ref(sh)
    for t in (3, 4, 5):       # the table holds steps 3 and 4 only
        sh.set_grads(t, 85)
        for tb in tables:
            z.zs_fused_shard_step_multi_dev(tb, steps)
        z.zs_step_table_advance(steps)
        if t < 5:
            ref.step(t, "standard")
        ref.check(f"t={t}")
    assert z.zs_step_table_status(steps) == (3, 1)


def test_graph_replay_of_bucketed_sgd_momentum():
    k = 5
    eager, graphed = Shard(k, 82), Shard(k, 82)
    te = eager.tables(bucket_elems=400_000)
    tg = graphed.tables(bucket_elems=400_000)
    hp = z.hparams(LR, B1, B2, EPS, 1, "sgd_momentum")  # constants do not change with t
    # one eager launch first (the library caches the CU count outside capture)
    graphed.set_grads(0, 83)
    eager.set_grads(0, 83)
    for tb in te:
        z.zs_fused_shard_step_multi(tb, hp)
    for tb in tg:
        z.zs_fused_shard_step_multi(tb, hp)
    torch.cuda.synchronize()

    def launch(s):
        for tb in tg:
            z.zs_fused_shard_step_multi(tb, hp, stream=s)

    g = _capture(launch)
    assert eager.same_as(graphed)  # capture itself ran nothing
    for t in (1, 2, 3, 4):
        eager.set_grads(t, 84)      # eager work between replays
        graphed.set_grads(t, 84)
        for tb in te:
            z.zs_fused_shard_step_multi(tb, hp)
        g.replay()
        torch.cuda.synchronize()
        assert eager.same_as(graphed), f"replay {t} differs from eager launches"
