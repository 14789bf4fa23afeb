"""Pins for the oracle's cumulative-threshold mask (Video-BLADE, "Step 2.1").

Brute force over every subset confirms the minimal count and the chosen set
(independent integer arithmetic, not the oracle's rational sums); hand-derived
dyadic rows fix the tie and equality readings; nesting and the tau limits give
the rest.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.mask import build_mask, build_mask_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _as_int(x):
    """float32 value as an exact integer multiple of 2**-149."""
    num, den = float(np.float32(x)).as_integer_ratio()
    return num * (2 ** 149) // den


def test_golden_dyadic_rows():
    g = json.load(open(os.path.join(GOLDEN, "mask_dyadic.json")))
    for c in g["cases"]:
        kept, tie = build_mask_row(np.array(c["row"], dtype=np.float32), c["tau"])
        assert kept == c["kept"], c["derivation"]
        assert tie == c["tie"], c["derivation"]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_minimal_and_top_m(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 11))
    kind = seed % 4
    if kind == 0:
        row = rng.random(nb)
    elif kind == 1:
        row = rng.exponential(size=nb) ** 3
    elif kind == 2:                      # many equal values
        row = rng.integers(0, 3, size=nb) / 4.0
    else:
        row = np.exp(-rng.random(nb) * 30)
    row = np.minimum(row / max(row.max(), 1e-30), 1.0).astype(np.float32)
    tau = float(np.float32(rng.choice([0.3, 0.5, 0.9, 0.95, 0.999])))
    kept, _ = build_mask_row(row, tau)
    vals = [_as_int(v) for v in row]
    total = sum(vals)
    tnum, tden = float(np.float32(tau)).as_integer_ratio()
    reaches = lambda s: s * tden >= tnum * total
    m = len(kept)
    assert m >= 1
    assert reaches(sum(vals[j] for j in kept))
    for sub in itertools.combinations(range(nb), m - 1):
        if m - 1 >= 1:
            assert not reaches(sum(vals[j] for j in sub))
    if m == 2 and not reaches(0):
        pass
    # chosen set = the first m of the order (value desc, index asc)
    order = sorted(range(nb), key=lambda j: (-vals[j], j))
    assert kept == sorted(order[:m])


def test_nesting_in_tau():
    rng = np.random.default_rng(5)
    P = rng.random((20, 16)).astype(np.float32) ** 4
    prev = None
    for tau in (0.1, 0.3, 0.5, 0.7, 0.9, 0.95, 0.99, 1.0):
        _, _, msk, _ = build_mask(P, tau)
        if prev is not None:
            assert (msk >= prev).all()
        prev = msk


def test_tau_limits():
    rng = np.random.default_rng(6)
    P = rng.random((8, 12)).astype(np.float32)
    P[3, 4] = P[3, 7] = 1.0                  # tie for the maximum: lowest index wins
    cnt, idx, msk, _ = build_mask(P, 1.0)
    assert (cnt == 12).all() and (msk == 1).all()
    cnt, idx, _, _ = build_mask(P, 1e-7)
    assert (cnt == 1).all()
    assert np.array_equal(idx[:, 0], np.argmax(P, axis=1))
    assert idx[3, 0] == 4


def test_invalid_rows_keep_everything():
    for bad in (np.nan, -0.5, 1.5, np.inf):
        row = np.array([0.5, 0.2, bad, 0.1], dtype=np.float32)
        kept, _ = build_mask_row(row, 0.5)
        assert kept == [0, 1, 2, 3]
    # negative zero is zero
    kept, _ = build_mask_row(np.array([-0.0, 0.5, 0.25], dtype=np.float32), 0.5)
    assert kept == [1]


def test_output_layout():
    P = np.array([[[0.5, 0.25, 0.125, 0.125], [0.0, 0.0, 0.0, 1.0],
                   [0.25, 0.25, 0.25, 0.25], [0.1, 0.2, 0.3, 0.4]]], dtype=np.float32)
    cnt, idx, msk, ties = build_mask(P, 0.7)
    assert cnt.shape == (1, 4) and idx.shape == (1, 4, 4)
    assert cnt[0].tolist() == [2, 1, 3, 2]
    assert idx[0, 0, :2].tolist() == [0, 1] and (idx[0, 0, 2:] == -1).all()
    assert idx[0, 1, :1].tolist() == [3]
    assert idx[0, 2, :3].tolist() == [0, 1, 2]
    assert idx[0, 3, :2].tolist() == [2, 3]
    assert msk[0].sum(axis=1).tolist() == cnt[0].tolist()
