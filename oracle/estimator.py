"""Oracle: online block-importance estimation.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

*Video-BLADE*, "Step 1: Efficient block importance estimation" (BLADE notes,
key design 1): conceptually P = softmax(Q K^T / sqrt(d_k)) is cut into b x b
blocks and max-pooled into the block importance map P_imp.  To avoid forming
P, k < b representative tokens are sampled from every block of Q and of K,
a low-resolution map P_approx is computed from the samples, and P_imp is
derived from it.  Defaults b = 128, k = 16 ("Implementation details").

Readings (the pages leave these open):
- which tokens: evenly spaced and deterministic, offsets floor(t * L_J / k_J)
  for t < k_J, with L_J the valid tokens of block J and k_J = min(k, L_J);
  the same positions for Q and K and for every head.  At k = b every token of
  every block is sampled.
- the softmax runs over all sampled keys of that (batch, head), with the
  scale 1/sqrt(d) of the full head dimension.
- P_imp[I, J] is the maximum of P_approx over the (samples of I) x (samples
  of J) tile, the sampled counterpart of the b x b max-pool.
All arithmetic here is float64 on the given (bf16-representable) inputs.
"""
from __future__ import annotations

import numpy as np


def block_lengths(N: int, b: int) -> np.ndarray:
    nb = -(-N // b)
    return np.array([min(b, N - J * b) for J in range(nb)], dtype=np.int64)


def sample_rows(N: int, b: int, k: int) -> list:
    """Per block J, the reordered row indices sampled from it."""
    rows = []
    for J, L in enumerate(block_lengths(N, b)):
        kJ = min(k, int(L))
        rows.append(np.array([J * b + (t * int(L)) // kJ for t in range(kJ)], dtype=np.int64))
    return rows


def p_imp(q_r: np.ndarray, k_r: np.ndarray, N: int, b: int, k: int, scale: float,
          query_blocks=None) -> np.ndarray:
    """P_imp [nb, nb] for one (batch, head); q_r, k_r are [>=N, d] in curve order.

    With query_blocks given, only those rows are computed (the others are NaN);
    each computed row is the same as in the full map, since every sampled
    query's softmax runs over all sampled keys either way.
    """
    rows = sample_rows(N, b, k)
    nb = len(rows)
    if query_blocks is None:
        query_blocks = range(nb)
    query_blocks = list(query_blocks)
    flat = np.concatenate(rows)
    owner = np.concatenate([np.full(len(r), J) for J, r in enumerate(rows)])
    qflat = np.concatenate([rows[I] for I in query_blocks])
    qowner = np.concatenate([np.full(len(rows[I]), I) for I in query_blocks])
    qs = np.asarray(q_r, dtype=np.float64)[qflat]
    ks = np.asarray(k_r, dtype=np.float64)[flat]
    s = (qs @ ks.T) * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)          # P_approx, one row per sampled query
    out = np.full((nb, nb), np.nan, dtype=np.float64)
    for I in query_blocks:
        pi = p[qowner == I]
        for J in range(nb):
            out[I, J] = pi[:, owner == J].max()
    return out


def p_imp_all(q_r: np.ndarray, k_r: np.ndarray, N: int, b: int, k: int, scale: float) -> np.ndarray:
    """P_imp for every (batch, head): q_r, k_r are [B, Hh, Npad, d] -> [B, Hh, nb, nb]."""
    B, Hh = q_r.shape[:2]
    nb = -(-N // b)
    out = np.empty((B, Hh, nb, nb), dtype=np.float64)
    for bi in range(B):
        for h in range(Hh):
            out[bi, h] = p_imp(q_r[bi, h], k_r[bi, h], N, b, k, scale)
    return out
