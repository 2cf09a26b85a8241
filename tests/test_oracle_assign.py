"""Pins for oracle.assign: hand-worked cases (tests/golden/assign_cases.json)
and the tier splits of the two mixed-precision decode workloads."""
import json
import os

import numpy as np
import pytest

from oracle import assign

GOLD = os.path.join(os.path.dirname(__file__), "golden", "assign_cases.json")


def _cases():
    with open(GOLD) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    got = assign.assign_precision(case["stat"], case["tier_frac"], case["tier_prec"])
    assert got == case["expect"]


def test_kda_quarter_bf16_split():
    stat = -np.linspace(0.01, 1.0, 32)[::-1]        # head 31 slowest
    got = assign.assign_precision(stat, [0.25, 0.75], [1, 2])
    assert got.count(1) == 8 and got.count(2) == 24
    assert all(got[h] == 1 for h in range(24, 32))


def test_half_int4_split():
    rng = np.random.default_rng(0)
    stat = -rng.uniform(0, 1, 32)
    got = assign.assign_precision(stat, [0.5, 0.5], [2, 3])
    assert got.count(2) == 16 and got.count(3) == 16
    slow = set(np.argsort(-stat, kind="stable")[:16].tolist())
    assert {h for h in range(32) if got[h] == 2} == slow


def test_decay_stat_closed_forms():
    a = np.full((10, 3), 0.5)
    a[:, 1] = 0.25
    a[:, 2] = 1.0
    np.testing.assert_allclose(assign.decay_stat(a), [np.log(0.5), np.log(0.25), 0.0])
    ch = np.ones((4, 2, 8))
    ch[:, 0, :4] = np.e ** -2          # half the channels at log = -2
    np.testing.assert_allclose(assign.decay_stat(ch), [-1.0, 0.0])
