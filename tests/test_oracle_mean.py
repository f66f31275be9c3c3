"""Pins of the oracle's P-rank gradient mean.

Page "高效AI 第19讲：分布式训练（第一部分）", 通信原语 / All-Reduce: g = (1/N) sum g_i;
page "深度学习专题：模型训练的数据并行（三）" §(四) ZeRO-2 step 2 (reduce-scatter,
then the mean of the rank's slice).  Read as: fp32 sum in rank order 0..P-1
seeded with rank 0's value, then one division by P.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp32exact import round_f32


def _to_bits(x: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f16":
        return x.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy(
    ).view(np.uint16)


def _values(bits: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("p", [1, 2, 3, 4, 7, 8, 16, 64, 256])
def test_identical_ranks_give_that_value(dt, p):
    # P copies of v: every partial sum k*v is exact (<= 11+8 significant bits),
    # so the mean is v itself.  The edge workload's constant block relies on it.
    rng = np.random.default_rng(p)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 4, 4096)).astype(np.float32)
    bits = _to_bits(x, dt)
    got = oracle.grad_mean(dt, [bits] * p)
    assert np.array_equal(got, oracle.widen(dt, bits))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("p", [2, 3, 5, 8, 13, 64])
def test_exact_rational_mean(dt, p):
    # Small dyadic values: every partial sum is exact in fp32, so the fold is
    # the exact sum and the result is the exact rational sum/P rounded once.
    rng = np.random.default_rng(100 + p)
    n = 300
    ints = rng.integers(-255, 256, size=(p, n))
    scale = 2.0 ** rng.integers(-10, 3, size=n)
    x = (ints * scale).astype(np.float32)
    bits = [_to_bits(x[r], dt) for r in range(p)]
    vals = [_values(b, dt) for b in bits]
    got = oracle.grad_mean(dt, bits)
    for i in range(n):
        total = sum(Fraction(float(vals[r][i])) for r in range(p))
        assert got[i] == round_f32(total / p), (i, total)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fold_order_is_rank_order(dt):
    # Random magnitudes make fp32 addition order-dependent; the oracle must
    # equal a left fold in rank order and differ from the reverse order.
    rng = np.random.default_rng(7)
    p, n = 64, 20000
    x = (rng.standard_normal((p, n)) * 10.0 ** rng.integers(-3, 3, (p, n))).astype(np.float32)
    bits = [_to_bits(x[r], dt) for r in range(p)]
    widened = [_values(b, dt).astype(np.float32) for b in bits]
    fwd = widened[0].copy()
    for r in range(1, p):
        fwd = (fwd + widened[r]).astype(np.float32)
    fwd = (fwd / np.float32(p)).astype(np.float32)
    rev = widened[p - 1].copy()
    for r in range(p - 2, -1, -1):
        rev = (rev + widened[r]).astype(np.float32)
    rev = (rev / np.float32(p)).astype(np.float32)
    got = oracle.grad_mean(dt, bits)
    assert np.array_equal(got.view(np.uint32), fwd.view(np.uint32))
    assert not np.array_equal(got.view(np.uint32), rev.view(np.uint32))


def test_mean_of_zeros_is_positive_zero():
    z = np.zeros(16, np.uint16)
    got = oracle.grad_mean("bf16", [z] * 5)
    assert np.all(got.view(np.uint32) == 0)


def test_mean_subnormal_fp16_inputs_widen_exactly():
    # fp16 subnormals (2^-24 .. 2^-14) widen to exact fp32 normals
    h = np.arange(1, 0x400, dtype=np.uint16)
    got = oracle.grad_mean("f16", [h, h])
    assert np.array_equal(got, h.view(np.float16).astype(np.float32))
