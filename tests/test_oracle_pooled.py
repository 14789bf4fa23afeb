"""Pins for the pooled block estimators and the SICS aggregation score (oracle/pooled.py)."""
import math
from itertools import combinations

import numpy as np
import pytest

from oracle.pooled import aggregation_score, choose_scheme, descriptors, pooled_p_imp, sics_blocks


def _piecewise(nb, b, d, seed):
    rng = np.random.default_rng(seed)
    qb, kb = rng.standard_normal((nb, d)), rng.standard_normal((nb, d))
    return np.repeat(qb, b, axis=0), np.repeat(kb, b, axis=0), qb, kb


def test_mean_equals_block_mass_of_full_attention():
    # constant blocks: every query of block I puts mass |J| e^{s_IJ} / sum_J' |J'| e^{s_IJ'} on key
    # block J, which for equal blocks is the softmax of q_I . k_J / sqrt(d) -- the MEAN estimate
    nb, b, d = 5, 4, 6
    q, k, qb, kb = _piecewise(nb, b, d, 0)
    N = nb * b
    s = q @ k.T / math.sqrt(d)
    a = np.exp(s - s.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)
    mass = a.reshape(nb, b, nb, b).sum(axis=3).mean(axis=1)
    np.testing.assert_allclose(pooled_p_imp(q, k, N, b, "mean"), mass, rtol=1e-12, atol=1e-15)


def test_trip_on_constant_blocks_is_sqrt3_sharper():
    # descriptors [q, q, q]: S = 3 q.k / sqrt(3 d) = sqrt(3) q.k / sqrt(d)
    nb, b, d = 4, 3, 5
    q, k, qb, kb = _piecewise(nb, b, d, 1)
    s = math.sqrt(3) * (qb @ kb.T) / math.sqrt(d)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    np.testing.assert_allclose(pooled_p_imp(q, k, nb * b, b, "trip"), e / e.sum(axis=1, keepdims=True), rtol=1e-12)


def test_descriptor_statistics_by_hand_and_ragged_block():
    x = np.array([[1.0, -2.0], [3.0, 0.0], [-1.0, 4.0], [5.0, 5.0], [7.0, -7.0]])
    dm = descriptors(x, 5, 2, "mean")
    np.testing.assert_array_equal(dm, [[2.0, -1.0], [2.0, 4.5], [7.0, -7.0]])     # last block: one token
    dt = descriptors(x, 5, 2, "trip")
    np.testing.assert_array_equal(dt[1], [2.0, 4.5, 5.0, 5.0, -1.0, 4.0])
    np.testing.assert_array_equal(descriptors(np.vstack([x, np.full((3, 2), 99.0)]), 5, 2, "trip"), dt)  # rows >= N ignored


@pytest.mark.parametrize("kind", ["mean", "trip"])
def test_rows_sum_to_one_and_equivariance(kind):
    rng = np.random.default_rng(2)
    N, b, d = 37, 8, 4
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    P = pooled_p_imp(q, k, N, b, kind)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-12)
    assert (P > 0).all()
    # swapping two whole key blocks swaps the two columns
    k2 = k.copy()
    k2[0:8], k2[16:24] = k[16:24], k[0:8]
    P2 = pooled_p_imp(q, k2, N, b, kind)
    np.testing.assert_allclose(P2[:, [2, 1, 0, 3, 4]], P, rtol=1e-12)


def test_sics_closed_form_and_brute_force():
    # the notes' identity: sum_i sum_j q_i^.q_j^ = BS + 2 sum_{i<j} q_i^.q_j^ = || sum_i q_i^ ||^2
    rng = np.random.default_rng(3)
    b, d = 7, 5
    q = rng.standard_normal((2 * b, d))
    u = q / np.linalg.norm(q, axis=1, keepdims=True)
    for I in range(2):
        blk = u[I * b:(I + 1) * b]
        brute = b + 2 * sum(float(blk[i] @ blk[j]) for i, j in combinations(range(b), 2))
        assert abs(sics_blocks(q, 2 * b, b)[I] - brute) < 1e-12
    # identical directions: BS^2; mutually orthogonal: BS; a scaled copy changes nothing
    same = np.tile(rng.standard_normal((1, d)), (b, 1)) * rng.uniform(0.5, 2.0, (b, 1))
    assert abs(sics_blocks(same, b, b)[0] - b * b) < 1e-9
    eye = np.eye(4)
    assert abs(sics_blocks(eye, 4, 4)[0] - 4.0) < 1e-12
    assert abs(aggregation_score(q, 2 * b, b) - sics_blocks(q, 2 * b, b).sum()) < 1e-12
    z = np.zeros((3, d))
    assert sics_blocks(z, 3, 3)[0] == 0.0


def test_scheme_choice_counts_query_and_key():
    # four tokens, blocks of two.  Candidate 0 pairs tokens (0, 1), (2, 3); candidate 1 pairs
    # (0, 2), (1, 3).  SICS of a pair of unit rows is 2 + 2 cos(angle).
    # Q: rows e0, e0, e1, e1 -> AS(Q | 0) = 4 + 4 = 8, AS(Q | 1) = 2 + 2 = 4, so Q alone picks 0.
    # K: rows e0, e1, e0, e1 -> AS(K | 0) = 4, AS(K | 1) = 8; Q + K ties at 12 and the first wins.
    # Scaling K changes nothing.  Q2 = e0, e0, e1, e60 (e60 at 60 degrees to e1, orthogonal to
    # e0): AS(Q2 | 0) = 4 + 3 = 7, AS(Q2 | 1) = 2 + 2 = 4, so Q2 alone picks 0 but Q2 + K picks 1
    # (11 < 12): a choice from Q alone, or a K term with the wrong sign, fails one of these.
    e0, e1 = np.array([1.0, 0.0, 0.0]), np.array([0.0, 1.0, 0.0])
    q = np.stack([e0, e0, e1, e1])
    k = np.stack([e0, e1, e0, e1])
    perms = [np.array([0, 1, 2, 3]), np.array([0, 2, 1, 3])]
    c, sc = choose_scheme(q, None, perms, 2)
    assert c == 0 and np.allclose(sc, [8.0, 4.0])
    c, sc = choose_scheme(q, k, perms, 2)
    assert np.allclose(sc, [12.0, 12.0]) and c == 0          # tie: the first candidate
    c3, sc3 = choose_scheme(q, 3.0 * k, perms, 2)
    assert c3 == 0 and np.allclose(sc3, sc)
    e60 = np.array([0.0, 0.5, math.sqrt(3) / 2])
    q2 = np.stack([e0, e0, e1, e60])
    c, sc = choose_scheme(q2, None, perms, 2)
    # AS(Q2 | 0) = 4 + (2 + 2 * 0.5) = 7; AS(Q2 | 1): pairs (e0, e1) and (e0, e60), both orthogonal: 4
    assert c == 0 and np.allclose(sc, [7.0, 4.0])
    c, sc = choose_scheme(q2, k, perms, 2)
    assert c == 1 and np.allclose(sc, [11.0, 12.0])


def test_scheme_choice_with_k_equal_q_doubles_scores():
    rng = np.random.default_rng(5)
    N, d, b = 24, 4, 6
    q = rng.standard_normal((N, d))
    perms = [rng.permutation(N) for _ in range(3)]
    cq, sq = choose_scheme(q, None, perms, b)
    ck, sk = choose_scheme(q, q, perms, b)
    assert cq == ck and np.allclose(sk, 2 * sq)
    # and the scores are the sums of the per-block values of each reordered tensor
    k = rng.standard_normal((N, d))
    _, s2 = choose_scheme(q, k, perms, b)
    for c, p in enumerate(perms):
        assert abs(s2[c] - sics_blocks(q[p], N, b).sum() - sics_blocks(k[p], N, b).sum()) < 1e-12
