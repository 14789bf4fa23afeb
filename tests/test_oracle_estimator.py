"""Pins for the oracle's block-importance estimator (Video-BLADE, "Step 1").

The pins do not retype the oracle: the k = b case is checked against the
conceptual definition the page states first (the full softmax map, max-pooled
over b x b blocks), computed by a different route (scipy's softmax on the dense
score matrix and a reshape-max); sampled rows are checked against hand-derived
offsets; k < b is checked as the same definition applied to the subsequence of
sampled tokens; normalisation and bounds give the rest.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle.estimator import block_lengths, p_imp, sample_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qk(N, d, seed, shared=True):
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((N, d))
    q = f + 0.3 * rng.standard_normal((N, d)) if shared else rng.standard_normal((N, d))
    k = f + 0.3 * rng.standard_normal((N, d)) if shared else rng.standard_normal((N, d))
    return q, k


def _dense_blockmax(q, k, blocks, scale):
    """Max-pool of softmax(q k^T * scale) over the given blocks of rows/cols."""
    p = softmax((q @ k.T) * scale, axis=1)
    nb = len(blocks)
    out = np.empty((nb, nb))
    for I, ri in enumerate(blocks):
        for J, cj in enumerate(blocks):
            out[I, J] = p[np.ix_(ri, cj)].max()
    return out


def test_sample_rows_golden():
    g = json.load(open(os.path.join(GOLDEN, "sample_rows.json")))
    for c in g["cases"]:
        got = [r.tolist() for r in sample_rows(c["N"], c["b"], c["k"])]
        assert got == c["rows"], c["derivation"]


@pytest.mark.parametrize("N,b", [(64, 16), (50, 16), (37, 8), (130, 32)])
def test_k_equals_b_reproduces_exact_maxpooled_map(N, b):
    d = 8
    q, k = _qk(N, d, seed=N + b)
    scale = 1 / np.sqrt(d)
    got = p_imp(q, k, N, b, b, scale)
    blocks = [np.arange(J * b, min((J + 1) * b, N)) for J in range(-(-N // b))]
    ref = _dense_blockmax(q, k, blocks, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("N,b,k", [(64, 16, 4), (50, 16, 5), (37, 8, 3), (130, 32, 16)])
def test_sampled_map_is_the_definition_on_the_sampled_subsequence(N, b, k):
    d = 8
    q, k_ = _qk(N, d, seed=3 * N + k)
    scale = 1 / np.sqrt(d)
    got = p_imp(q, k_, N, b, k, scale)
    rows = sample_rows(N, b, k)
    flat = np.concatenate(rows)
    sub_blocks, pos = [], 0
    for r in rows:
        sub_blocks.append(np.arange(pos, pos + len(r)))
        pos += len(r)
    ref = _dense_blockmax(q[flat], k_[flat], sub_blocks, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("N,b", [(64, 8), (45, 8)])
def test_k1_rows_sum_to_one(N, b):
    q, k = _qk(N, 4, seed=7, shared=False)
    P = p_imp(q, k, N, b, 1, 0.5)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_bounds(k):
    N, b = 72, 8
    q, k_ = _qk(N, 6, seed=k)
    P = p_imp(q, k_, N, b, k, 1 / np.sqrt(6))
    assert (P > 0).all() and (P <= 1).all()
    s = P.sum(axis=1)
    assert (s >= 1.0 / k - 1e-12).all() and (s <= k + 1e-12).all()


def test_hand_worked_two_blocks():
    # N = 4, b = 2, k = 1, d = 1, scale 1: samples are rows 0 and 2.
    # q0 = 1, q2 = 2; k0 = 0, k2 = ln 3.
    # row 0 scores (0, ln 3) -> softmax (1/4, 3/4); row 2: (0, 2 ln 3) -> (1/10, 9/10).
    q = np.array([[1.0], [9.0], [2.0], [9.0]])
    k = np.array([[0.0], [9.0], [np.log(3.0)], [9.0]])
    P = p_imp(q, k, 4, 2, 1, 1.0)
    np.testing.assert_allclose(P, [[0.25, 0.75], [0.1, 0.9]], rtol=1e-12)


def test_padding_rows_never_sampled():
    N, b = 21, 8
    q, k = _qk(24, 4, seed=2)
    P1 = p_imp(q, k, N, b, 4, 0.5)
    q2, k2 = q.copy(), k.copy()
    q2[N:] = 1e6
    k2[N:] = -1e6
    P2 = p_imp(q2, k2, N, b, 4, 0.5)
    assert np.array_equal(P1, P2)
    assert block_lengths(N, b).tolist() == [8, 8, 5]


def test_query_block_subset_equals_full_rows():
    N, b, k = 90, 16, 4
    q, k_ = _qk(N, 8, seed=11)
    full = p_imp(q, k_, N, b, k, 0.3)
    part = p_imp(q, k_, N, b, k, 0.3, query_blocks=[0, 3, 5])
    for I in range(full.shape[0]):
        if I in (0, 3, 5):
            assert np.array_equal(part[I], full[I])
        else:
            assert np.isnan(part[I]).all()
