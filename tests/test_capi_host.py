"""Host-side tests of libzshard's C ABI (no GPU needed, no kernel launched).

The library loads and exports every symbol include/zshard.h declares; the
host planners match the oracle exactly; every argument error is reported
before anything reaches the device (fake device addresses are safe here
because the calls return before any launch).
"""

import re
import os

import numpy as np
import pytest

import oracle
from adam_zs_shard_amd import zshard as z

try:
    import torch

    _HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _HAVE_GPU = False
from zs_synth import gpt2_small_tensors, llama3_8b_tensors

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "zshard.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zs_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) == 23 and sorted(names) == sorted(z.EXPORTS)
    L = z.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(z.EXPORTS) == names
    assert z.zs_version() == 2
    for st in range(10):
        assert z.zs_status_string(st).startswith("ZS_")
        assert z.zs_status_string(st) != "ZS_ERR_UNKNOWN"
    assert z.zs_status_string(z.ZS_ERR_RESOURCE) == "ZS_ERR_RESOURCE"
    assert z.zs_status_string(99) == "ZS_ERR_UNKNOWN"


@pytest.mark.parametrize("n,p", [(0, 1), (1, 1), (9, 4), (1_000_003, 4), (124_439_808, 8),
                                 (7_500_000_000, 64), (8_030_261_248, 8), (100_000_007, 16),
                                 (5, 256), (2**40 + 3, 256)])
def test_plan_matches_oracle(n, p):
    assert z.zs_plan_shards(n, p) == oracle.plan_shards(n, p)


def test_plan_brute_force_small():
    for n in range(0, 40):
        for p in range(1, 12):
            assert z.zs_plan_shards(n, p) == oracle.plan_shards(n, p)


def test_plan_rejects():
    for n, p in ((-1, 2), (5, 0), (5, -3)):
        with pytest.raises(z.ZsError) as ei:
            z.zs_plan_shards(n, p)
        assert ei.value.status == z.ZS_ERR_ARG
    with pytest.raises(z.ZsError) as ei:
        z.zs_plan_shards(2**61, 4)
    assert ei.value.status == z.ZS_ERR_RANGE


@pytest.mark.parametrize("tensors", ["gpt2", "llama", "random"])
def test_plan_chunks_matches_oracle_pieces(tensors):
    if tensors == "gpt2":
        numel = [n for _, n in gpt2_small_tensors()]
    elif tensors == "llama":
        numel = [n for _, n in llama3_8b_tensors()]
    else:
        numel = [int(x) for x in np.random.default_rng(0).integers(0, 50, 40)]
    for p in (1, 3, 8, 16):
        _, s, e = oracle.plan_shards(sum(numel), p)
        for k in range(p):
            got, nchunks = z.zs_plan_chunks(numel, p, k, 4096)
            want = oracle.shard_pieces(numel, s[k], e[k])
            assert got == want
            assert nchunks == sum(-(-ln // 4096) for *_, ln in want)


def test_plan_chunks_capacity():
    import ctypes as C

    numel = (C.c_int64 * 4)(5, 5, 5, 5)
    arr = (z.zs_piece * 1)()
    npieces = C.c_int32()
    st = z.lib().zs_plan_chunks(numel, 4, 1, 0, 8, arr, 1, C.byref(npieces), None)
    assert st == z.ZS_ERR_CAPACITY and npieces.value == 4


HP = z.hparams(1e-3, 0.9, 0.999, 1e-8, 1)
FAKE = 1 << 40  # a device-looking address; never dereferenced on these paths

# Every call below with FAKE addresses must be rejected before any launch.
# They run only where no GPU exists, so a mistake here cannot reach a device.
no_device = pytest.mark.skipif(_HAVE_GPU, reason="fake device addresses: CPU-only test")


def _fused(n=1000, p=4, k=1, grads=None, w=FAKE, m=FAKE + (1 << 30), v=FAKE + (2 << 30),
           param=FAKE + (3 << 30), hp=HP, gdt=z.ZS_F16, pdt=z.ZS_F16, grad_base=0, param_base=0,
           workspace=None, workspace_bytes=0):
    if grads is None:
        grads = [FAKE + ((4 + r) << 30) for r in range(p)]
    return z.zs_fused_shard_step(n, p, k, grads, w, m, v, param, hp, grad_base=grad_base,
                                 param_base=param_base, grad_dtype=gdt, param_dtype=pdt,
                                 workspace=workspace, workspace_bytes=workspace_bytes,
                                 check=False)


@no_device
def test_fused_argument_errors():
    assert _fused(p=0) == z.ZS_ERR_ARG
    assert _fused(p=1025, grads=[FAKE + (8 << 30) + (r << 20) for r in range(1025)]) == \
        z.ZS_ERR_ARG
    assert _fused(k=4) == z.ZS_ERR_ARG
    assert _fused(k=-1) == z.ZS_ERR_ARG
    assert _fused(n=-5) == z.ZS_ERR_ARG
    assert _fused(gdt=3) == z.ZS_ERR_DTYPE
    assert _fused(pdt=0) == z.ZS_ERR_DTYPE
    assert _fused(hp=z.hparams(1e-3, 0.9, 0.999, 1e-8, 0)) == z.ZS_ERR_ARG
    assert _fused(hp=z.hparams(1e-3, 1.0, 0.999, 1e-8, 1)) == z.ZS_ERR_ARG
    assert _fused(hp=z.hparams(float("nan"), 0.9, 0.999, 1e-8, 1)) == z.ZS_ERR_ARG
    assert _fused(hp=z.hparams(1e-3, 0.9, 0.999, float("inf"), 1)) == z.ZS_ERR_ARG
    assert _fused(hp=z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, form=4)) == z.ZS_ERR_ARG
    assert _fused(hp=z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, form=-1)) == z.ZS_ERR_ARG
    assert _fused(w=None) == z.ZS_ERR_NULL
    assert _fused(param=None) == z.ZS_ERR_NULL
    assert _fused(grads=[FAKE, None, FAKE, FAKE]) == z.ZS_ERR_NULL
    # shard 1 of 1000 over 4 starts at 250: bases beyond it are out of range
    assert _fused(grad_base=251) == z.ZS_ERR_RANGE
    assert _fused(param_base=-1) == z.ZS_ERR_RANGE
    assert _fused(n=2**61) == z.ZS_ERR_RANGE


@no_device
def test_fused_alias_detection():
    L = 250  # shard 1 of n=1000 over p=4 is [250, 500)
    assert _fused(m=FAKE + 4 * L - 4) == z.ZS_ERR_ALIAS          # w and m overlap by one
    g = [FAKE + ((4 + r) << 30) for r in range(4)]
    # rank 2 reads [g2 + 500, g2 + 1000) bytes; param's slice starts at param + 500
    assert _fused(grads=g, param=g[2]) == z.ZS_ERR_ALIAS
    assert _fused(grads=g, param=g[2] + 498) == z.ZS_ERR_ALIAS   # last byte pair shared
    # w overlaps a gradient slice
    assert _fused(grads=g, w=g[0] + 2 * 250) == z.ZS_ERR_ALIAS


@no_device
def test_empty_shard_returns_ok_without_device():
    # n=9, p=4: shard 3 is empty; nothing may be launched or dereferenced
    assert _fused(n=9, p=4, k=3, w=None, m=None, v=None, param=None) == z.ZS_OK
    assert _fused(n=0, p=1, k=0) == z.ZS_OK


@no_device
def test_mean_and_adam_argument_errors():
    g = [FAKE + (r << 30) for r in range(4)]
    f = z.zs_reduce_scatter_mean_local
    assert f(g, 1000, 4, 4, FAKE + (8 << 30), grad_dtype="f16", check=False) == z.ZS_ERR_ARG
    assert f(g, 1000, 4, 1, None, grad_dtype="f16", check=False) == z.ZS_ERR_NULL
    assert f(g, 1000, 4, 1, FAKE + (8 << 30), grad_dtype=7, check=False) == z.ZS_ERR_DTYPE
    assert f(g, 1000, 4, 1, g[1] + 500, grad_dtype="f16", check=False) == z.ZS_ERR_ALIAS
    assert f(g, 1000, 4, 1, FAKE + (8 << 30), grad_base=300, grad_dtype="f16",
             check=False) == z.ZS_ERR_RANGE
    a = z.zs_adam_step
    base = FAKE
    assert a(base, base + 4096, base + 8192, base + 12288, None, -1, HP,
             check=False) == z.ZS_ERR_ARG
    assert a(base, base + 4096, base + 8192, base + 12288, None, 0, HP, check=False) == z.ZS_OK
    # 1025 floats from base run one float into w's range
    assert a(base, base + 4096, base + 8192, base + 12288, None, 1025, HP,
             check=False) == z.ZS_ERR_ALIAS
    assert a(None, base + 4096, base + 8192, base + 12288, None, 8, HP,
             check=False) == z.ZS_ERR_NULL
    assert a(base, base + 4096, base + 8192, base + 12288, base + 16384, 8, HP, param_dtype=9,
             check=False) == z.ZS_ERR_DTYPE


@no_device
def test_mt_upload_argument_errors():
    assert z.zs_mt_workspace_bytes(3, 10, 8) > 0
    assert z.zs_mt_workspace_bytes(3, 10, 0) == 0
    assert z.zs_mt_workspace_bytes(-1, 10, 4) == 0
    pieces = [(0, 0, 0, 100), (1, 0, 100, 50)]
    ptrs = [dict(w=FAKE, m=FAKE + (1 << 30), v=FAKE + (2 << 30), param=FAKE + (3 << 30),
                 grads=[FAKE + (4 << 30), FAKE + (5 << 30)]),
            dict(w=FAKE + 400, m=FAKE + (1 << 30) + 400, v=FAKE + (2 << 30) + 400,
                 param=FAKE + (6 << 30), grads=[FAKE + (4 << 30) + 200, FAKE + (5 << 30) + 200])]
    ws = FAKE + (10 << 30)
    nb = z.zs_mt_workspace_bytes(2, 2, 2)

    def up(pieces=pieces, ptrs=ptrs, p=2, gdt="f16", pdt="f16", ce=64, ws=ws, nb=nb):
        try:
            z.zs_mt_upload(pieces, ptrs, p, gdt, pdt, ce, ws, nb)
        except z.ZsError as e:
            return e.status
        return z.ZS_OK

    assert up(ce=12) == z.ZS_ERR_ARG          # not a multiple of 8
    assert up(ce=0) == z.ZS_ERR_ARG
    assert up(p=0) == z.ZS_ERR_ARG
    assert up(pdt=5) == z.ZS_ERR_DTYPE
    assert up(nb=nb - 1) == z.ZS_ERR_CAPACITY
    assert up(ws=ws + 8) == z.ZS_ERR_CAPACITY
    bad = [dict(ptrs[0]), dict(ptrs[1])]
    bad[1]["w"] = FAKE + 396                     # overlaps piece 0's w by one float
    assert up(ptrs=bad) == z.ZS_ERR_ALIAS
    bad = [dict(ptrs[0]), dict(ptrs[1])]
    bad[1]["param"] = FAKE + (4 << 30) + 100     # param on top of a gradient
    assert up(ptrs=bad) == z.ZS_ERR_ALIAS
    bad = [dict(ptrs[0]), dict(ptrs[1])]
    bad[0]["w"] = None
    assert up(ptrs=bad) == z.ZS_ERR_NULL
    # m and v are optional at upload (the step checks the form against the
    # table's state mask); passing the checks means reaching the copy, which
    # fails with ZS_ERR_HIP on a host without a device
    nov = [dict(ptrs[0]), dict(ptrs[1])]
    nov[0]["v"] = None
    assert up(ptrs=nov) == z.ZS_ERR_HIP


@no_device
def test_multi_step_argument_errors():
    t = z.zs_mt_table(workspace=FAKE, nchunks=0, chunk_elems=64, npieces=0, p=2, grad_dtype=1,
                      param_dtype=1)
    assert z.zs_fused_shard_step_multi(t, HP, check=False) == z.ZS_OK     # nothing to do
    t.nchunks = 3
    t.p = 0
    assert z.zs_fused_shard_step_multi(t, HP, check=False) == z.ZS_ERR_ARG
    t.p = 2
    t.grad_dtype = 9
    assert z.zs_fused_shard_step_multi(t, HP, check=False) == z.ZS_ERR_DTYPE
    t.grad_dtype = 1
    assert z.zs_fused_shard_step_multi(t, z.hparams(1e-3, 0.9, 0.999, 1e-8, 0),
                                       check=False) == z.ZS_ERR_ARG


@no_device
def test_state_pointers_required_by_form():
    # Adam needs m and v, momentum SGD only m, plain SGD neither.  On a host
    # with no device, ZS_ERR_HIP means every check before the launch passed.
    adam = z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, "standard")
    lit = z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, "page1_literal")
    sgd = z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, "sgd")
    mom = z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, "sgd_momentum")
    for hp in (adam, lit):
        assert _fused(hp=hp, m=None) == z.ZS_ERR_NULL
        assert _fused(hp=hp, v=None) == z.ZS_ERR_NULL
    assert _fused(hp=mom, m=None) == z.ZS_ERR_NULL
    assert _fused(hp=mom, v=None) == z.ZS_ERR_HIP
    assert _fused(hp=sgd, m=None, v=None) == z.ZS_ERR_HIP
    # state a form does not use is not written, so it may even alias w
    assert _fused(hp=sgd, m=FAKE, v=FAKE) == z.ZS_ERR_HIP
    assert _fused(hp=mom, m=FAKE) == z.ZS_ERR_ALIAS
    assert z.zs_adam_step(FAKE, FAKE + (1 << 30), None, None, None, 100, sgd,
                          check=False) == z.ZS_ERR_HIP
    assert z.zs_adam_step(FAKE, FAKE + (1 << 30), None, None, None, 100, mom,
                          check=False) == z.ZS_ERR_NULL


@no_device
def test_multi_step_checks_state_mask():
    def step(state, form):
        t = z.zs_mt_table(workspace=FAKE, nchunks=4, chunk_elems=64, npieces=1, p=2,
                          grad_dtype=1, param_dtype=1, state=state)
        return z.zs_fused_shard_step_multi(t, z.hparams(1e-3, 0.9, 0.999, 1e-8, 1, form),
                                           check=False)
    both = z.ZS_STATE_M | z.ZS_STATE_V
    assert step(both, "standard") == z.ZS_ERR_HIP          # checks passed
    assert step(z.ZS_STATE_M, "standard") == z.ZS_ERR_NULL
    assert step(z.ZS_STATE_M, "page1_literal") == z.ZS_ERR_NULL
    assert step(z.ZS_STATE_M, "sgd_momentum") == z.ZS_ERR_HIP
    assert step(0, "sgd_momentum") == z.ZS_ERR_NULL
    assert step(0, "sgd") == z.ZS_ERR_HIP


def test_workspace_bytes_for_many_ranks():
    assert z.ZS_MAX_P == 1024 and z.ZS_KERNARG_P == 256
    for p in (1, 64, 256):
        assert z.zs_shard_workspace_bytes(p) == 0
    assert z.zs_shard_workspace_bytes(257) == 2304       # 8 * 257 rounded up to 256
    assert z.zs_shard_workspace_bytes(512) == 4096
    assert z.zs_shard_workspace_bytes(1024) == 8192
    assert z.zs_shard_workspace_bytes(1025) == 0
    assert z.zs_shard_workspace_bytes(0) == 0


@no_device
def test_many_ranks_need_a_workspace():
    # 512 ranks: the rank pointers go through a device workspace
    n, p, k = 100_000, 512, 7
    g = [FAKE + (8 << 30) + (r << 24) for r in range(p)]   # clear of w, m, v and param
    ws = FAKE + (3 << 30) + (1 << 20)     # clear of the working copy's used slice
    assert _fused(n=n, p=p, k=k, grads=g) == z.ZS_ERR_CAPACITY               # none given
    assert _fused(n=n, p=p, k=k, grads=g, workspace=ws, workspace_bytes=4095) == \
        z.ZS_ERR_CAPACITY                                                      # too small
    assert _fused(n=n, p=p, k=k, grads=g, workspace=ws + 8, workspace_bytes=4096) == \
        z.ZS_ERR_CAPACITY                                                      # misaligned
    assert _fused(n=n, p=p, k=k, grads=g, workspace=FAKE + 16, workspace_bytes=4096) == \
        z.ZS_ERR_ALIAS                                                         # inside w
    assert _fused(n=n, p=p, k=k, grads=g, workspace=g[3] + 2 * 7 * 196 + 8,
                  workspace_bytes=4096) == z.ZS_ERR_ALIAS                      # on a gradient
    # every check passed: the launch itself fails on a host without a device
    assert _fused(n=n, p=p, k=k, grads=g, workspace=ws, workspace_bytes=4096) == z.ZS_ERR_HIP
    # 256 ranks still travel as kernel arguments: no workspace needed
    g256 = g[:256]
    assert _fused(n=n, p=256, k=7, grads=g256) == z.ZS_ERR_HIP


@no_device
def test_mean_many_ranks_and_16bit_output_errors():
    n, p = 100_000, 1024
    g = [FAKE + (8 << 30) + (r << 24) for r in range(p)]
    out = FAKE + (1 << 20)
    f = z.zs_reduce_scatter_mean_local
    assert f(g, n, p, 3, out, grad_dtype="f16", check=False) == z.ZS_ERR_HIP   # passes of 256
    assert f(g + [FAKE], n, 1025, 3, out, grad_dtype="f16", check=False) == z.ZS_ERR_ARG
    f16 = z.zs_reduce_scatter_mean_local16
    g4 = g[:4]
    assert f16(g4, n, 4, 1, out, "bf16", grad_dtype="f16", check=False) == z.ZS_ERR_HIP
    assert f16(g4, n, 4, 1, out, 0, grad_dtype="f16", check=False) == z.ZS_ERR_DTYPE
    assert f16(g4, n, 4, 1, out, 3, grad_dtype="f16", check=False) == z.ZS_ERR_DTYPE
    assert f16(g4, n, 4, 1, None, "f16", grad_dtype="f16", check=False) == z.ZS_ERR_NULL
    # a 16-bit output of 25,000 elements is 50,000 bytes: one byte pair onto rank 2's slice
    assert f16(g4, n, 4, 1, g4[2] + 2 * 25_000 - 50_000 + 2, "f16", grad_dtype="f16",
               check=False) == z.ZS_ERR_ALIAS
    # more than 256 ranks: the fp32 sums between passes need `partial`
    assert f16(g, n, p, 3, out, "f16", grad_dtype="f16", check=False) == z.ZS_ERR_NULL
    part = FAKE + (2 << 30)
    assert f16(g, n, p, 3, out, "f16", grad_dtype="f16", partial=part,
               check=False) == z.ZS_ERR_HIP
    assert f16(g, n, p, 3, out, "f16", grad_dtype="f16", partial=out + 64,
               check=False) == z.ZS_ERR_ALIAS


def test_chunk_rule():
    whole = 28 * 256 * 8
    # two whole chunks per CU or more: the kernel's whole chunk
    assert z.zs_mt_chunk_elems(2 * whole * 256, 1, 256) == whole
    assert z.zs_mt_chunk_elems(1_003_782_656, 42, 256) == whole            # Llama-3-8B shard 3
    # less: the per-CU share (a quarter with several pieces), up to 2,048
    assert z.zs_mt_chunk_elems(15_554_976, 1, 256) == 61_440               # GPT-2 shard 0
    assert z.zs_mt_chunk_elems(15_554_976, 35, 256) == 16_384              # GPT-2 shard 7
    assert z.zs_mt_chunk_elems(2 * whole * 256 - 1, 1, 256) == 2 * whole  # one chunk per CU
    assert z.zs_mt_chunk_elems(1, 1, 256) == 2048
    assert z.zs_mt_chunk_elems(0, 1, 256) == 2048
    assert z.zs_mt_chunk_elems(10_000_000, 1, 80) == whole
    assert z.zs_mt_chunk_elems(-1, 1, 256) == 0
    assert z.zs_mt_chunk_elems(100, 0, 256) == 0
    for L in (3, 999, 123_457, 9_999_999):
        for npc in (1, 2, 40):
            c = z.zs_mt_chunk_elems(L, npc, 256)
            assert c % 2048 == 0 and 2048 <= c <= 2 * whole


@pytest.mark.parametrize("seed", range(6))
def test_buckets_are_minimal_runs(seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(1, 5000, int(rng.integers(1, 60)))]
    pieces = [(i, 0, sum(lens[:i]), ln) for i, ln in enumerate(lens)]
    B = int(rng.integers(1, 20_000))
    of, nb = z.zs_plan_buckets(pieces, B)
    assert of[0] == 0 and of == sorted(of) and nb == of[-1] + 1
    assert all(b - a in (0, 1) for a, b in zip(of, of[1:]))              # consecutive runs
    for b in range(nb):
        run = [lens[i] for i in range(len(lens)) if of[i] == b]
        if b < nb - 1:
            assert sum(run) >= B and sum(run) - run[-1] < B                # closed at B
        else:
            assert sum(run) - run[-1] < B                                  # last may be short
    assert z.zs_plan_buckets(pieces, 0) == ([0] * len(lens), 1)
    assert z.zs_plan_buckets(pieces, 1) == (list(range(len(lens))), len(lens))
    assert z.zs_plan_buckets([], 10) == ([], 0)
    with pytest.raises(z.ZsError):
        z.zs_plan_buckets([(0, 0, 0, 0)], 10)


def test_step_table_layout_and_errors():
    assert z.zs_step_table_bytes(0) == 0
    assert z.zs_step_table_bytes(1) == 256
    assert z.zs_step_table_bytes(5) == 256                 # 48 + 5 * 36 bytes
    assert z.zs_step_table_bytes(6) == 512
    big = z.ZS_MAX_TABLE_STEPS
    assert z.zs_step_table_bytes(big) == (48 + 36 * big + 255) // 256 * 256
    assert z.zs_step_table_bytes(big + 1) == 0
    L = z.lib()
    import ctypes as C

    t = z.zs_step_table()
    assert L.zs_step_table_init(C.byref(HP), 8, 0, FAKE, 256, None, C.byref(t)) == z.ZS_ERR_ARG
    # more entries than one table holds: refused before any host staging
    assert L.zs_step_table_init(C.byref(HP), 8, big + 1, FAKE, 1 << 40, None, C.byref(t)) == \
        z.ZS_ERR_ARG
    assert L.zs_step_table_init(C.byref(HP), 0, 4, FAKE, 256, None, C.byref(t)) == z.ZS_ERR_ARG
    assert L.zs_step_table_init(C.byref(HP), 1025, 4, FAKE, 256, None, C.byref(t)) == \
        z.ZS_ERR_ARG
    assert L.zs_step_table_init(C.byref(HP), 8, 4, None, 256, None, C.byref(t)) == z.ZS_ERR_NULL
    assert L.zs_step_table_init(C.byref(HP), 8, 4, FAKE + 16, 256, None, C.byref(t)) == \
        z.ZS_ERR_CAPACITY
    assert L.zs_step_table_init(C.byref(HP), 8, 4, FAKE, 255, None, C.byref(t)) == \
        z.ZS_ERR_CAPACITY
    bad = z.hparams(1e-3, 0.9, 0.999, 1e-8, 0)
    assert L.zs_step_table_init(C.byref(bad), 8, 4, FAKE, 256, None, C.byref(t)) == z.ZS_ERR_ARG
    # handles are checked before any launch
    st = z.zs_step_table(dev=None, first_step=1, nsteps=4, p=8, form=0)
    assert z.zs_step_table_advance(st, check=False) == z.ZS_ERR_NULL
    st.dev = FAKE
    st.nsteps = 0
    assert z.zs_step_table_advance(st, check=False) == z.ZS_ERR_ARG
    st.nsteps = big + 1
    assert z.zs_step_table_advance(st, check=False) == z.ZS_ERR_ARG
    st.nsteps, st.form = 4, 7
    assert z.zs_step_table_advance(st, check=False) == z.ZS_ERR_ARG
    st.form = 0
    mt = z.zs_mt_table(workspace=FAKE + (1 << 30), nchunks=4, chunk_elems=64, npieces=1, p=4,
                       grad_dtype=1, param_dtype=1, state=3)
    assert z.zs_fused_shard_step_multi_dev(mt, st, check=False) == z.ZS_ERR_ARG   # p differs
    st.form = 1
    mt.state = 1
    mt.p = 8
    assert z.zs_fused_shard_step_multi_dev(mt, st, check=False) == z.ZS_ERR_NULL  # no v


@no_device
def test_step_table_calls_reach_the_device():
    st = z.zs_step_table(dev=FAKE, first_step=1, nsteps=4, p=8, form=0)
    assert z.zs_step_table_advance(st, check=False) == z.ZS_ERR_HIP
    mt = z.zs_mt_table(workspace=FAKE + (1 << 30), nchunks=4, chunk_elems=64, npieces=1, p=8,
                       grad_dtype=1, param_dtype=1, state=3)
    assert z.zs_fused_shard_step_multi_dev(mt, st, check=False) == z.ZS_ERR_HIP


@no_device
def test_offload_argument_errors():
    import numpy as np

    n, p, k = 1000, 4, 1                      # shard [250, 500): 250 elements
    g = [FAKE + (8 << 30) + (r << 24) for r in range(p)]
    host = [np.zeros(250, np.float32) for _ in range(3)]
    g16 = [np.zeros(250, np.uint16) for _ in range(2)]
    ph = np.zeros(250, np.uint16)
    hp = HP

    def off(mode=z.ZS_OFFLOAD_PLAIN, slot=0, p=p, k=k, grads=g, g16_dev=FAKE, param=FAKE + (1 << 30),
            w=host[0], m=host[1], v=host[2], g16_host=g16, bucket=0, partial=None, hp=hp):
        return z.zs_offload_step(n, p, k, grads, param, g16_dev, g16_host, w, m, v, ph, hp, mode,
                                 slot, grad_dtype="f16", param_dtype="f16", partial=partial,
                                 bucket_elems=bucket, check=False)

    assert off(mode=3) == z.ZS_ERR_ARG
    assert off(slot=2) == z.ZS_ERR_ARG
    assert off(k=4) == z.ZS_ERR_ARG
    assert off(bucket=-1) == z.ZS_ERR_ARG
    assert off(bucket=0) == z.ZS_ERR_HIP                     # every check passed
    assert off(hp=z.hparams(1e-3, 0.9, 0.999, 1e-8, 0)) == z.ZS_ERR_ARG
    assert off(g16_dev=None) == z.ZS_ERR_NULL
    assert off(w=None) == z.ZS_ERR_NULL
    assert off(mode=z.ZS_OFFLOAD_RECEIVE, w=None, m=None, v=None) == z.ZS_ERR_HIP  # no update
    assert off(mode=z.ZS_OFFLOAD_DELAYED, g16_host=[g16[0], None]) == z.ZS_ERR_NULL
    # host buffers overlapping: m inside w
    assert off(m=host[0][10:]) == z.ZS_ERR_ALIAS
    # the gradient being received overlaps the one being applied
    assert off(mode=z.ZS_OFFLOAD_DELAYED, g16_host=[g16[0], g16[0][5:]]) == z.ZS_ERR_ALIAS
    # device: the rounded mean on top of rank 2's slice
    assert off(g16_dev=g[2] + 2 * 250 + 64) == z.ZS_ERR_ALIAS
    # more than 256 ranks need the fp32 partial sums
    g300 = [FAKE + (8 << 30) + (r << 24) for r in range(300)]
    assert off(p=300, k=0, grads=g300) == z.ZS_ERR_NULL
    assert off(p=300, k=0, grads=g300, partial=FAKE + (2 << 30)) == z.ZS_ERR_HIP
    assert off(bucket=1) == z.ZS_ERR_HIP                     # 250 buckets of one element


@no_device
def test_static_scratch_entry_checks_like_the_workspace_one():
    n, p, k = 100_000, 512, 7
    g = [FAKE + (8 << 30) + (r << 24) for r in range(p)]

    def st(**kw):
        return z.zs_fused_shard_step(n, p, k, g, FAKE, FAKE + (1 << 30), FAKE + (2 << 30),
                                     FAKE + (3 << 30), kw.pop("hp", HP), grad_dtype="f16",
                                     param_dtype="f16", static=True, check=False, **kw)

    assert st() == z.ZS_ERR_HIP                              # no workspace needed
    assert st(hp=z.hparams(1e-3, 0.9, 0.999, 1e-8, 0)) == z.ZS_ERR_ARG
    assert z.zs_fused_shard_step(n, 1025, k, g + g[:513], FAKE, FAKE + (1 << 30),
                                 FAKE + (2 << 30), FAKE + (3 << 30), HP, grad_dtype="f16",
                                 param_dtype="f16", static=True, check=False) == z.ZS_ERR_ARG
