"""Oracle: pooled block-importance estimators and the SICS aggregation score.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Pooled estimators (the SPADE notes' MEAN and DSA summaries; VEDA's TripPool
descriptor, key design 1, without its learned projections): every block of b
reordered tokens is summarised by a descriptor, the mean of its valid tokens
(MEAN), or the concatenation of their mean, channel-wise maximum and
channel-wise minimum (TRIP; the DSA summary is the same three statistics).
The block score is the scaled dot product of a query block's descriptor with a
key block's, S[I, J] = desc_q(I) . desc_k(J) / sqrt(d'), d' the descriptor
length (VEDA's predicted score with the head-specific projections taken as the
identity, the plain reading when they are not trained), and the estimate is
its row softmax over the key blocks, P[I, :] = softmax(S[I, :]), which takes
the place of P_imp on the path.

SICS (the SPADE notes, runtime scheme generation): a block's sum of intra-block
cosine similarities over its unit-normalised tokens, SICS = sum_i sum_j
q_i^ . q_j^ = || sum_i q_i^ ||^2, and a scheme's aggregation score is its sum
over the blocks, AS = sum_I SICS(I).  Zero rows normalise to zero.  The notes
compute the aggregation score of Query and of Key for every candidate scheme
and pick, per head, the scheme with the highest score; read here as the score
AS(Q | scheme) + AS(K | scheme), the first candidate winning a tie.

float64 throughout.
"""
from __future__ import annotations

import math

import numpy as np


def descriptors(x_r: np.ndarray, N: int, b: int, kind: str) -> np.ndarray:
    """x_r [>= N, d] reordered rows -> [nb, d] (MEAN) or [nb, 3d] (TRIP: mean, max, min)."""
    x = np.asarray(x_r, dtype=np.float64)[:N]
    nb = -(-N // b)
    out = []
    for I in range(nb):
        blk = x[I * b:min((I + 1) * b, N)]
        mean = blk.sum(axis=0) / blk.shape[0]
        if kind == "mean":
            out.append(mean)
        elif kind == "trip":
            out.append(np.concatenate([mean, blk.max(axis=0), blk.min(axis=0)]))
        else:
            raise ValueError(kind)
    return np.stack(out)


def pooled_p_imp(q_r: np.ndarray, k_r: np.ndarray, N: int, b: int, kind: str) -> np.ndarray:
    """One (batch, head): P [nb, nb] = row softmax of the scaled descriptor products."""
    dq = descriptors(q_r, N, b, kind)
    dk = descriptors(k_r, N, b, kind)
    s = (dq @ dk.T) / math.sqrt(dq.shape[1])
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def sics_blocks(q_r: np.ndarray, N: int, b: int) -> np.ndarray:
    """SICS of every block of b reordered rows: || sum of the unit-normalised rows ||^2."""
    q = np.asarray(q_r, dtype=np.float64)[:N]
    n = np.sqrt((q * q).sum(axis=1, keepdims=True))
    u = np.divide(q, n, out=np.zeros_like(q), where=n > 0)
    nb = -(-N // b)
    out = np.empty(nb)
    for I in range(nb):
        s = u[I * b:min((I + 1) * b, N)].sum(axis=0)
        out[I] = float(s @ s)
    return out


def aggregation_score(q_r: np.ndarray, N: int, b: int) -> float:
    """AS of one head under the scheme that produced the reordered rows q_r."""
    return float(sics_blocks(q_r, N, b).sum())


def choose_scheme(q: np.ndarray, k, perms, b: int):
    """One head's scheme choice: q, k [N, d] in token order (k may be None: Q alone); perms a list
    of candidate orders (perm[new] = token).  Returns (index of the chosen candidate, the scores
    AS(Q | c) + AS(K | c) of every candidate)."""
    N = q.shape[0]
    scores = []
    for perm in perms:
        p = np.asarray(perm)
        sc = aggregation_score(np.asarray(q)[p], N, b)
        if k is not None:
            sc += aggregation_score(np.asarray(k)[p], N, b)
        scores.append(sc)
    best = 0
    for c in range(1, len(scores)):
        if scores[c] > scores[best]:
            best = c
    return best, np.array(scores)
