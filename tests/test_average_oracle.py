"""Pins of the oracle's averaged hop-2 output (the optimizer-ready shard).

Page "ZeRO Stage 2: Gradient Partitioning", the numbered steps of the
stage-2 flow, step 2: the reduce-scatter averages the gradients over all GPUs
and GPU i keeps the average of shard i. Reading (in ``oracle/zpp_oracle.c``):
the binary32 hop sum divided by the number of contributing GPUs, correctly
rounded. The sum itself is pinned in ``test_oracle_pins.py``; these tests pin
the division against hand-derived values, exact rational arithmetic and the
exactness of power-of-two divisors.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from test_oracle_pins import _f32_from_hex, _nearest_f32, _pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "average_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_average(oracle_lib, case):
    codes = [_pack(i["codes"], case["bits"]) for i in case["inputs"]]
    scales = [np.asarray(i["scales"], dtype=np.float32) for i in case["inputs"]]
    n = len(case["inputs"][0]["codes"])
    avg = oracle.dequant_average(codes, scales, case["bits"], n, case["block"], case["divisor"])
    if "avg_bits_hex" in case:
        assert avg.view(np.uint32).tolist() == _f32_from_hex(case["avg_bits_hex"]).view(np.uint32).tolist()
    else:
        assert avg.tolist() == case["avg"]


def _random_inputs(bits, n_inputs, numel, block, seed):
    rng = np.random.default_rng([23, bits, n_inputs, seed])
    Q = 127 if bits == 8 else 7
    codes, scales = [], []
    for _ in range(n_inputs):
        q = rng.integers(-Q, Q + 1, numel)
        codes.append(_pack(q.tolist(), bits))
        scales.append((rng.uniform(0.5, 1.0, numel // block) * np.exp2(rng.integers(-30, 10, numel // block)))
                      .astype(np.float32))
    return codes, scales


@pytest.mark.parametrize("divisor", [1, 3, 7, 24, 255, 1000, 65535, 1 << 24])
@pytest.mark.parametrize("bits,n_inputs", [(4, 1), (4, 5), (8, 2), (4, 32)])
def test_average_is_correctly_rounded_quotient_of_sum(oracle_lib, divisor, bits, n_inputs):
    numel, block = 512, 32
    codes, scales = _random_inputs(bits, n_inputs, numel, block, divisor)
    total = oracle.dequant_sum(codes, scales, bits, numel, block)
    avg = oracle.dequant_average(codes, scales, bits, numel, block, divisor)
    for i in range(numel):
        assert _nearest_f32(Fraction(float(total[i])) / divisor, avg[i]), (i, total[i], avg[i])


@pytest.mark.parametrize("k", [0, 1, 3, 8, 15])
def test_power_of_two_divisor_only_shifts_the_exponent(oracle_lib, k):
    numel, block = 1024, 64
    codes, scales = _random_inputs(4, 8, numel, block, 100 + k)
    total = oracle.dequant_sum(codes, scales, 4, numel, block)
    avg = oracle.dequant_average(codes, scales, 4, numel, block, 1 << k)
    assert np.array_equal(avg, total * np.float32(2.0 ** -k))


@pytest.mark.parametrize("divisor", [0, -1, (1 << 24) + 1])
def test_divisor_out_of_range_is_rejected(oracle_lib, divisor):
    codes, scales = _random_inputs(4, 2, 64, 32, 0)
    with pytest.raises(Exception):
        oracle.dequant_average(codes, scales, 4, 64, 32, divisor)
