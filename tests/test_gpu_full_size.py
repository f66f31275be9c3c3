"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times (one call per shard and step, and for the chunk table the chunk
length zs_mt_chunk_elems gives, as bench.py makes them).

The step is elementwise once the shard map is fixed, so the oracle runs on
the gathered inputs of a sample of elements (random positions plus every
boundary the kernels treat specially: the first and last elements, whole-
chunk and leftover-piece edges, the scalar tail, tensor-piece edges) and
the GPU result must match it bit for bit at those positions.  Properties
that hold at any size are checked on every element: the 16-bit working copy
is the round-to-nearest-even downcast of the fp32 master weight, positions
whose gradient is zero on every rank keep their weight exactly, and memory
outside the shard keeps its canary pattern.
"""

import numpy as np
import pytest
import torch

import oracle
from adam_zs_shard_amd import zshard as z
from zs_synth import WORKLOADS, make
from zs_synth.gen import fill_pattern
from gpu_util import DEV, need_gpu, say, u16, f32, check_f32, check_param

pytestmark = pytest.mark.gpu
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
SENTINEL = 0x4B4B
GROUP = 256 * 8            # elements of one lane-group across a workgroup
CHUNK = 28 * GROUP         # elements of one whole chunk of the single-tensor kernel


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _sample(L, edges, n_rand, seed):
    """Sorted unique sample of [0, L): random positions plus +-8 around each edge."""
    rng = np.random.default_rng(seed)
    pts = set(range(min(L, 64))) | set(range(max(0, L - 64), L))
    for b in edges:
        pts |= set(range(max(0, b - 8), min(L, b + 8)))
    pts |= set(int(x) for x in rng.integers(0, L, n_rand))
    return np.array(sorted(pts), np.int64)


def _single_tensor_edges(L):
    """Element offsets where the single-tensor kernel changes regime, for any
    head in 0..7: whole chunks, the first leftover piece edges, the tail."""
    edges = []
    for h in (0, 4):
        nvec = (L - h) // 8
        nfull = nvec // (CHUNK // 8)
        left0 = h + nfull * CHUNK
        edges += [h, h + CHUNK, h + 2 * CHUNK, left0 - CHUNK, left0, h + nvec * 8]
        edges += [left0 + i * GROUP for i in range(1, 18)]
    return [e for e in edges if 0 <= e <= L]


def _downcast_bits(w: torch.Tensor, dt: str) -> torch.Tensor:
    return w.to(TD[dt]).view(torch.int16)


def _gather_grads(grads, base, idx_dev):
    return [u16(g[base + idx_dev]) for g in grads]


def test_zero_7p5b_p64_shard63_five_steps():
    wl = WORKLOADS["zero_7p5b_p64"]
    k = wl.shards[-1]
    M, s, e = z.zs_plan_shards(wl.n, wl.p)
    assert (M, s, e) == oracle.plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    assert L == 117_187_500
    say(f"7.5B/P=64 shard {k}: {L} elements, {wl.steps} steps")
    w = make.initial_w(wl, k, L, DEV)
    m = torch.zeros_like(w)
    v = torch.zeros_like(w)
    param = torch.empty(wl.n, dtype=TD[wl.param_dtype], device=DEV)
    fill_pattern(param, SENTINEL)
    idx = _sample(L, _single_tensor_edges(L), 6000, 11)
    idx_dev = torch.from_numpy(idx).to(DEV)
    ws, ms, vs = f32(w[idx_dev]).copy(), np.zeros(idx.size, np.float32), np.zeros(idx.size,
                                                                                 np.float32)
    for t in range(1, wl.steps + 1):
        grads = [make.normal_grad(wl, r, t, L, DEV, stream=k) for r in range(wl.p)]
        z.zs_fused_shard_step(wl.n, wl.p, k, grads, w, m, v, param,
                              z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, t, wl.form),
                              grad_base=s[k], param_base=0)
        gs = _gather_grads(grads, 0, idx_dev)
        del grads
        ph = oracle.step_elems(wl.grad_dtype, gs, ws, ms, vs, wl.param_dtype, wl.lr, wl.beta1,
                               wl.beta2, wl.eps, t, wl.form)
        torch.cuda.synchronize()
        d = check_f32(f32(w[idx_dev]), ws, 1e-6 if t == 1 else 2e-6, f"w t={t}")
        d += check_f32(f32(m[idx_dev]), ms, 2e-6, f"m t={t}")
        d += check_f32(f32(v[idx_dev]), vs, 2e-6, f"v t={t}")
        d += check_param(u16(param[s[k] + idx_dev]), ph, wl.param_dtype, f"param t={t}")
        assert d == 0, f"{d} sampled values differ in bits at t={t}"
        say(f"  step {t}: {idx.size} sampled elements bit-identical")
    # every element: the working copy is the RNE downcast of the master weight
    assert torch.equal(param[s[k]:e[k]].view(torch.int16), _downcast_bits(w, wl.param_dtype))
    # outside the shard: untouched
    sent = torch.full((4096,), SENTINEL, dtype=torch.int16, device=DEV)
    assert torch.equal(param[s[k] - 4096:s[k]].view(torch.int16), sent)
    assert torch.equal(param[:4096].view(torch.int16), sent)
    assert torch.equal(param[s[k] // 2:s[k] // 2 + 4096].view(torch.int16), sent)


@pytest.mark.parametrize("chunk_rule", ["bench", "1Mi"])
def test_llama3_8b_p8_shard3_multi_tensor_five_steps(chunk_rule):
    # "bench": the chunk length bench.py times (zs_mt_chunk_elems: the kernel's
    # whole chunk, 57,344 elements, one whole chunk per table entry)
    wl = WORKLOADS["llama3_8b_p8"]
    k = wl.shards[0]
    numel = [n for _, n in wl.tensors]
    assert sum(numel) == wl.n
    M, s, e = oracle.plan_shards(wl.n, wl.p)
    L = e[k] - s[k]
    if chunk_rule == "bench":
        npieces = len(z.zs_plan_chunks(numel, wl.p, k, 8)[0])
        chunk = z.zs_mt_chunk_elems(L, npieces)
        assert chunk == 28 * 256 * 8
    else:
        chunk = 1 << 20
    pieces, nchunks = z.zs_plan_chunks(numel, wl.p, k, chunk)
    ref_pieces = oracle.shard_pieces(numel, s[k], e[k])
    assert pieces == ref_pieces and len(pieces) == 42
    say(f"Llama-3-8B/P=8 shard {k}: {L} elements, {len(pieces)} pieces, {nchunks} chunks")
    esz = 2
    w = make.initial_w(wl, k, L, DEV)
    m = torch.zeros_like(w)
    v = torch.zeros_like(w)
    params = {}
    for (t_, to, so, ln) in pieces:
        if t_ not in params:
            params[t_] = fill_pattern(torch.empty(numel[t_], dtype=TD[wl.param_dtype], device=DEV),
                                      SENTINEL)
    grads = [torch.empty(L, dtype=TD[wl.grad_dtype], device=DEV) for _ in range(wl.p)]
    ptrs = [dict(w=w.data_ptr() + 4 * so, m=m.data_ptr() + 4 * so, v=v.data_ptr() + 4 * so,
                 param=params[t_].data_ptr() + esz * to,
                 grads=[g.data_ptr() + esz * so for g in grads])
            for (t_, to, so, ln) in pieces]
    nb = z.zs_mt_workspace_bytes(len(pieces), nchunks, wl.p)
    ws_buf = torch.empty(nb, dtype=torch.uint8, device=DEV)
    table = z.zs_mt_upload(pieces, ptrs, wl.p, wl.grad_dtype, wl.param_dtype, chunk, ws_buf, nb)

    starts = np.array([so for (_, _, so, _) in ref_pieces], np.int64)
    edges = [int(x) for x in starts] + [L] + list(range(0, L, chunk))[:4] + [L - L % chunk]
    idx = _sample(L, edges, 6000, 12)
    idx_dev = torch.from_numpy(idx).to(DEV)
    which = np.searchsorted(starts, idx, side="right") - 1
    ws, ms, vs = f32(w[idx_dev]).copy(), np.zeros(idx.size, np.float32), np.zeros(idx.size,
                                                                                 np.float32)
    for t in range(1, wl.steps + 1):
        for r in range(wl.p):
            grads[r].copy_(make.normal_grad(wl, r, t, L, DEV, stream=k))
        z.zs_fused_shard_step_multi(table, z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, t,
                                                     wl.form))
        gs = _gather_grads(grads, 0, idx_dev)
        ph = oracle.step_elems(wl.grad_dtype, gs, ws, ms, vs, wl.param_dtype, wl.lr, wl.beta1,
                               wl.beta2, wl.eps, t, wl.form)
        torch.cuda.synchronize()
        d = check_f32(f32(w[idx_dev]), ws, 1e-6 if t == 1 else 2e-6, f"w t={t}")
        d += check_f32(f32(m[idx_dev]), ms, 2e-6, f"m t={t}")
        d += check_f32(f32(v[idx_dev]), vs, 2e-6, f"v t={t}")
        got = np.empty(idx.size, np.uint16)
        for pi, (t_, to, so, ln) in enumerate(ref_pieces):
            sel = np.nonzero(which == pi)[0]
            if sel.size:
                off = torch.from_numpy(to + (idx[sel] - so)).to(DEV)
                got[sel] = u16(params[t_][off])
        d += check_param(got, ph, wl.param_dtype, f"param t={t}")
        assert d == 0, f"{d} sampled values differ in bits at t={t}"
        say(f"  step {t}: {idx.size} sampled elements bit-identical")
    sent = torch.full((64,), SENTINEL, dtype=torch.int16, device=DEV)
    for (t_, to, so, ln) in ref_pieces:
        pt = params[t_]
        assert torch.equal(pt[to:to + ln].view(torch.int16),
                           _downcast_bits(w[so:so + ln], wl.param_dtype)), f"piece of tensor {t_}"
        if to >= 64:
            assert torch.equal(pt[to - 64:to].view(torch.int16), sent), f"before tensor {t_}"
        if to + ln + 64 <= numel[t_]:
            assert torch.equal(pt[to + ln:to + ln + 64].view(torch.int16), sent), \
                f"after tensor {t_}"


def test_edge_p16_literal_all_shards_twenty_steps():
    wl = WORKLOADS["edge_p16_literal"]
    M, s, e = oracle.plan_shards(wl.n, wl.p)
    assert wl.n % wl.p != 0
    say(f"edge N={wl.n} P={wl.p}: all shards, {wl.steps} steps, {wl.form}")
    zero = make.edge_zero_mask(wl, wl.n, DEV)
    param = torch.empty(wl.n, dtype=TD[wl.param_dtype], device=DEV)
    fill_pattern(param, SENTINEL)
    st, idxs, idev, host = [], [], [], []
    for k in range(wl.p):
        L = e[k] - s[k]
        w = make.initial_w(wl, k, L, DEV)
        st.append((w, torch.zeros_like(w), torch.zeros_like(w), w.clone()))
        edges = _single_tensor_edges(L) + [wl.const_block]
        idx = _sample(L, edges, 400, 100 + k)
        idxs.append(idx)
        idev.append(torch.from_numpy(idx).to(DEV))
        host.append([f32(w[idev[-1]]).copy(), np.zeros(idx.size, np.float32),
                     np.zeros(idx.size, np.float32)])
    for t in range(1, wl.steps + 1):
        grads = [make.edge_grad(wl, r, t, wl.n, zero, s, e, DEV) for r in range(wl.p)]
        hp = z.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, t, wl.form)
        for k in range(wl.p):
            w, m, v, _ = st[k]
            z.zs_fused_shard_step(wl.n, wl.p, k, grads, w, m, v, param, hp)
        d = 0
        for k in range(wl.p):
            w, m, v, _ = st[k]
            gs = _gather_grads(grads, s[k], idev[k])
            ws, ms, vs = host[k]
            ph = oracle.step_elems(wl.grad_dtype, gs, ws, ms, vs, wl.param_dtype, wl.lr, wl.beta1,
                                   wl.beta2, wl.eps, t, wl.form)
            torch.cuda.synchronize()
            d += check_f32(f32(w[idev[k]]), ws, 2e-6, f"w k={k} t={t}")
            d += check_f32(f32(m[idev[k]]), ms, 2e-6, f"m k={k} t={t}")
            d += check_f32(f32(v[idev[k]]), vs, 2e-6, f"v k={k} t={t}")
            d += check_param(u16(param[s[k] + idev[k]]), ph, wl.param_dtype, f"param k={k} t={t}")
        assert d == 0, f"{d} sampled values differ in bits at t={t}"
        del grads
        if t % 5 == 0:
            say(f"  step {t}: all 16 shards' samples bit-identical")
    for k in range(wl.p):
        w, m, v, w0 = st[k]
        assert torch.equal(param[s[k]:e[k]].view(torch.int16), _downcast_bits(w, wl.param_dtype))
        zk = zero[s[k]:e[k]].clone()
        zk[:min(wl.const_block, e[k] - s[k])] = False   # the constant block is never zero
        assert torch.equal(w[zk].view(torch.int32), w0[zk].view(torch.int32)), f"shard {k}"
        assert not torch.any(m[zk] != 0) and not torch.any(v[zk] != 0)
