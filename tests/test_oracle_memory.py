"""Pins of the oracle's memory model against the numbers the pages print
(tests/golden/memory_model.json, each entry with its page and section)."""

import json
import os

import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "memory_model.json")))


@pytest.mark.parametrize("row", GOLD["per_gpu_gb"], ids=lambda r: r["cite"][:40])
def test_per_gpu_gigabytes(row):
    got = oracle.mp_bytes_per_param(row["stage"], row["ndev"]) * row["params"] / 1e9
    assert abs(got - row["value"]) <= row["tol"] + 1e-9, (got, row)


@pytest.mark.parametrize("row", GOLD["bytes_per_param"], ids=lambda r: r["cite"][:40])
def test_bytes_per_param(row):
    got = oracle.mp_bytes_per_param(row["stage"], row["ndev"])
    assert abs(got - row["value"]) <= row["tol"] + 1e-12, (got, row)


@pytest.mark.parametrize("row", GOLD["limits"], ids=lambda r: r["cite"][:40])
def test_large_n_limits(row):
    got = oracle.mp_bytes_per_param(row["stage"], 1e12) / oracle.mp_bytes_per_param(0, 1)
    assert abs(got - row["value_fraction_of_replicated"]) < 1e-9


def test_adam_share_and_fp16_weights():
    a = GOLD["adam_share"]
    assert oracle.mp_bytes_per_param(0, 1) - 4 == pytest.approx(a["value"] * 16)
    f = GOLD["fp16_weights_gb"]
    assert f["params"] * f["bytes_per_param"] / 1e9 == f["value"]


@pytest.mark.parametrize("row", GOLD["max_params_80gb"], ids=lambda r: r["cite"][:40])
def test_max_params_on_80gb(row):
    got = 80e9 / oracle.mp_bytes_per_param(row["stage"], row["ndev"]) / 1e9
    assert abs(got - row["value_billion"]) <= row["tol"], (got, row)


def test_page_one_float_counts():
    # The page's formulas with M = ceil(N/P), checked on the sizing case and a
    # case where P does not divide N.
    for n, p in ((7_500_000_000, 64), (1_000_003, 4), (9, 4)):
        M = -(-n // p)
        want = {0: 2 * n, 1: 4 * n, 2: 2 * M + 2 * n, 3: 3 * M + n, 4: 4 * M}
        for scheme, val in want.items():
            assert oracle.p1_floats(scheme, n, p) == val
    # 7.5e9 parameters on 64 GPUs
    assert oracle.p1_floats(1, 7_500_000_000, 64) == 3.0e10
    assert abs(oracle.p1_floats(2, 7_500_000_000, 64) / 1.523e10 - 1) < 1e-3
    assert abs(oracle.p1_floats(3, 7_500_000_000, 64) / 7.852e9 - 1) < 1e-3
    assert oracle.p1_floats(4, 7_500_000_000, 64) == 4.6875e8
    # ZeRO stages order the storage as the page says: DP > Z1 > Z2 > Z3
    vals = [oracle.p1_floats(s, 10_000, 8) for s in (1, 2, 3, 4)]
    assert vals == sorted(vals, reverse=True)
