"""Pins for the alternative mask rules (BSA notes design 2; the top-k budget rule):
hand-worked rows (tests/golden/mask_rules.json), brute force, limits and the
normal-quantile reading."""
import json
import os
from itertools import combinations
from statistics import NormalDist

import numpy as np
import pytest

from oracle.mask_rules import build_mask_rule, stat_threshold_row, topk_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_rules.json")


def test_golden_rows():
    g = json.load(open(GOLDEN))
    for case in g["stat"]:
        kept, _ = stat_threshold_row(np.array(case["row"], np.float32), case["u"])
        assert kept == case["kept"], case
    for case in g["topk"]:
        assert topk_row(np.array(case["row"], np.float32), case["k"]) == case["kept"], case


@pytest.mark.parametrize("nb,seed", [(1, 0), (6, 1), (9, 2)])
def test_topk_brute_force(nb, seed):
    rng = np.random.default_rng(seed)
    row = rng.choice(np.array([0.0, 0.125, 0.25, 0.5, 1.0], np.float32), size=nb)
    for k in range(1, nb + 2):
        kept = topk_row(row, k)
        m = min(k, nb)
        # the kept set is the lexicographically smallest of the size-m sets with the largest sum
        best = max(combinations(range(nb), m), key=lambda c: (sum(float(row[j]) for j in c), [-j for j in c]))
        assert kept == sorted(best)
        if k > 1:
            assert set(topk_row(row, k - 1)) <= set(kept)     # nested in k


def test_stat_limits_and_floor():
    rng = np.random.default_rng(3)
    row = rng.random(40).astype(np.float32)
    assert stat_threshold_row(row, -50.0)[0] == list(range(40))          # p below every score
    top = int(np.argmax(row))
    assert stat_threshold_row(row, 50.0)[0] == [top]                      # only the guaranteed largest block
    kept0, _ = stat_threshold_row(row, 0.0)
    mean = row.astype(np.float64).mean()
    assert kept0 == [j for j in range(40) if row[j] >= mean]              # u = 0 keeps the blocks at or above the mean
    for u in (-1.0, 0.3, 1.2):
        a, _ = stat_threshold_row(row, u)
        b, _ = stat_threshold_row(row, u + 0.4)
        assert set(b) <= set(a)                                           # larger u keeps a subset


def test_stat_keeps_about_k_of_n_for_normal_scores():
    # the quantile U(1 - k/n) makes a normally distributed row keep about k of its n blocks
    rng = np.random.default_rng(4)
    n, k = 4000, 400
    row = np.clip(0.5 + 0.05 * rng.standard_normal(n), 0.0, 1.0).astype(np.float32)
    u = NormalDist().inv_cdf(1.0 - k / n)
    kept, _ = stat_threshold_row(row, u)
    assert abs(len(kept) - k) < 60          # binomial spread sqrt(k) ~ 20


def test_invalid_rows_keep_all():
    row = np.array([0.2, np.nan, 0.1], np.float32)
    assert topk_row(row, 1) == [0, 1, 2]
    assert stat_threshold_row(row, 1.0)[0] == [0, 1, 2]
    cnt, idx, msk, _ = build_mask_rule(np.array([[0.1, 0.9], [0.5, 0.4]], np.float32), "topk", 1)
    assert cnt.tolist() == [1, 1] and idx.tolist() == [[1, -1], [0, -1]]
