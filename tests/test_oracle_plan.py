"""Pins of the oracle's shard plan.

[DP-III] = page "深度学习专题：模型训练的数据并行（三）", §(三) ZeRO-1 优化原理,
1. 步骤分析: M = ceil(N/P); GPU k owns s_k = 1+(k-1)M .. e_k = kM.
Pinned by brute-force invariants over all small (N, P), by the page's own
4-layer toy model, by hand-worked bounds of the workload sizes, and by
pieces of flattened tensor lists checked element by element.
"""

import numpy as np
import pytest

import oracle
from zs_synth import gpt2_small_tensors, llama3_8b_tensors


@pytest.mark.parametrize("n", range(0, 17))
@pytest.mark.parametrize("p", range(1, 10))
def test_plan_invariants_brute_force(n, p):
    m, s, e = oracle.plan_shards(n, p)
    # M is the least integer with P*M >= N
    assert p * m >= n
    assert m == 0 or p * (m - 1) < n
    covered = []
    for k in range(p):
        assert 0 <= s[k] <= e[k] <= n
        assert e[k] - s[k] <= m
        covered.extend(range(s[k], e[k]))
        if k > 0:
            assert s[k] == e[k - 1]          # contiguous, in rank order
    assert covered == list(range(n))         # disjoint and complete
    # every shard before the first short one is full
    lens = [e[k] - s[k] for k in range(p)]
    first_short = next((k for k in range(p) if lens[k] < m), p)
    assert all(x == m for x in lens[:first_short])
    assert all(x == 0 for x in lens[first_short + 1:])


def test_plan_page_one_based_formula_small():
    # The page's 1-based inclusive bounds, checked on every N, P <= 8 where
    # the division is exact (so the page's formula needs no clamp).
    for n in range(1, 9):
        for p in range(1, 9):
            if n % p:
                continue
            m, s, e = oracle.plan_shards(n, p)
            for k1 in range(1, p + 1):
                assert s[k1 - 1] + 1 == 1 + (k1 - 1) * m
                assert e[k1 - 1] == k1 * m


def test_plan_toy_model_four_layers():
    # [DP-III] §(四) ZeRO-3 层间流水线优化: 4 layers with parameters (w_m, b_m),
    # 4 GPUs, GPU-m stores layer m.  Flattened (w1,b1,...,w4,b4): N=8, P=4.
    m, s, e = oracle.plan_shards(8, 4)
    assert m == 2
    names = ["w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4"]
    for k in range(4):
        assert names[s[k]:e[k]] == [f"w{k + 1}", f"b{k + 1}"]


def test_plan_empty_shards_count():
    # Over N, P in 1..8 a shard is empty exactly when the ceiling leaves fewer
    # than P non-empty pieces; count by enumerating the element ownership.
    empty_cases = 0
    for n in range(1, 9):
        for p in range(1, 9):
            _, s, e = oracle.plan_shards(n, p)
            owners = set()
            for k in range(p):
                owners.update([k] * (e[k] - s[k]))
            if len(owners) < p:
                empty_cases += 1
                assert any(e[k] == s[k] for k in range(p))
    assert empty_cases == 37


# Bounds worked by hand from M = ceil(N/P) for the five workload sizes.
@pytest.mark.parametrize("n,p,k,m,s,e", [
    (1_000_003, 4, 3, 250_001, 750_003, 1_000_003),
    (1_000_003, 4, 1, 250_001, 250_001, 500_002),
    (124_439_808, 8, 0, 15_554_976, 0, 15_554_976),
    (7_500_000_000, 64, 63, 117_187_500, 7_382_812_500, 7_500_000_000),
    (8_030_261_248, 8, 3, 1_003_782_656, 3_011_347_968, 4_015_130_624),
    (100_000_007, 16, 15, 6_250_001, 93_750_015, 100_000_007),
    (9, 4, 3, 3, 9, 9),
])
def test_plan_workload_bounds(n, p, k, m, s, e):
    mm, ss, ee = oracle.plan_shards(n, p)
    assert (mm, ss[k], ee[k]) == (m, s, e)


def test_plan_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.plan_shards(-1, 4)
    with pytest.raises(ValueError):
        oracle.plan_shards(10, 0)


def _brute_pieces(numel, lo, hi):
    """Element-by-element ownership walk (tiny lists only)."""
    owner = []
    for t, n in enumerate(numel):
        owner += [(t, o) for o in range(n)]
    pieces = []
    for j in range(lo, hi):
        t, o = owner[j]
        if pieces and pieces[-1][0] == t and pieces[-1][1] + pieces[-1][3] == o:
            pieces[-1][3] += 1
        else:
            pieces.append([t, o, j - lo, 1])
    return [tuple(x) for x in pieces]


@pytest.mark.parametrize("seed", range(20))
def test_pieces_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 12))
    numel = [int(x) for x in rng.integers(0, 9, size=T)]
    n = sum(numel)
    for p in range(1, 6):
        _, s, e = oracle.plan_shards(n, p)
        for k in range(p):
            got = oracle.shard_pieces(numel, s[k], e[k])
            assert got == _brute_pieces(numel, s[k], e[k])
            for j in range(s[k], e[k]):
                t, off = oracle.locate(numel, j)
                assert _brute_pieces(numel, j, j + 1)[0][:2] == (t, off)


def test_pieces_gpt2_and_llama_shapes():
    gpt = [n for _, n in gpt2_small_tensors()]
    assert len(gpt) == 148 and sum(gpt) == 124_439_808
    m, s, e = oracle.plan_shards(sum(gpt), 8)
    # shards 0 and 1 lie inside the token embedding (50257*768 values)
    assert oracle.shard_pieces(gpt, s[0], e[0]) == [(0, 0, 0, m)]
    assert len(oracle.shard_pieces(gpt, s[1], e[1])) == 1
    counts = [len(oracle.shard_pieces(gpt, s[k], e[k])) for k in range(8)]
    assert counts == [1, 1, 15, 25, 27, 25, 26, 35]

    lt = llama3_8b_tensors()
    ll = [n for _, n in lt]
    assert len(ll) == 291 and sum(ll) == 8_030_261_248
    m, s, e = oracle.plan_shards(sum(ll), 8)
    pcs = oracle.shard_pieces(ll, s[3], e[3])
    assert len(pcs) == 42
    assert lt[pcs[0][0]][0] == "layers.11.gate" and pcs[0][1] == 44_836_352
    assert lt[pcs[-1][0]][0] == "layers.16.q" and pcs[-1][1] == 0 and pcs[-1][3] == 2_048
    assert sum(x[3] for x in pcs) == m
    assert min(x[3] for x in pcs) == 2_048 and max(x[3] for x in pcs) == 58_720_256
