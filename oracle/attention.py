"""Oracle: block-masked softmax attention, with the ASA_G global tokens.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

*Video-BLADE*, "Step 2.2: Computation":
1) standard ASA: attention restricted by the binary block mask M, every query
   of query block I seeing exactly the key blocks kept for I;
2) ASA_G: K and V are augmented with "global tokens", the mean of each window
   of n consecutive tokens, K_aug = Concat(K, MeanPool_n(K)) (likewise V).  The
   original region is governed by M; every global-token score gets a fixed
   additive ln(n) before the softmax (BLADE notes, key design 2, the
   score_global += ln(n) equation), so that a global token weighs as much as
   the n tokens it summarises.

Readings: pooling runs over consecutive tokens of the reordered sequence; a
last window of r < n tokens uses its own mean and the bias ln(r); the global
tokens are not subject to M (every query sees all of them); tokens at
positions >= N (padding) are never keys and rows >= N are not computed.
This is plain float64 attention: scores for every key, -inf where the mask
forbids, softmax, then the weighted sum.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def meanpool(x_r: np.ndarray, N: int, n: int) -> np.ndarray:
    """Global tokens: [ceil(N/n), d] means of consecutive windows of the first N rows."""
    x = np.asarray(x_r, dtype=np.float64)[:N]
    Ng = -(-N // n)
    out = np.empty((Ng, x.shape[1]), dtype=np.float64)
    for g in range(Ng):
        out[g] = x[g * n: min((g + 1) * n, N)].mean(axis=0)
    return out


def global_bias(N: int, n: int) -> np.ndarray:
    """ln(r_g) for every window: ln(n), or ln(r) for a short last window."""
    Ng = -(-N // n)
    return np.array([math.log(min(n, N - g * n)) for g in range(Ng)], dtype=np.float64)


def masked_attention(q_r: np.ndarray, k_r: np.ndarray, v_r: np.ndarray, N: int, b: int,
                     kept: Sequence[Sequence[int]], scale: float,
                     k_g: Optional[np.ndarray] = None, v_g: Optional[np.ndarray] = None,
                     g_bias: Optional[np.ndarray] = None,
                     query_blocks: Optional[Sequence[int]] = None):
    """One (batch, head).  kept[I] lists the key blocks of query block I.

    Returns (out [N, d] float64 with only the requested query blocks filled,
    lse [N] natural-log sum of exp of the scores of each computed row).
    """
    q = np.asarray(q_r, dtype=np.float64)
    k = np.asarray(k_r, dtype=np.float64)[:N]
    v = np.asarray(v_r, dtype=np.float64)[:N]
    nb = -(-N // b)
    if query_blocks is None:
        query_blocks = range(nb)
    key_block = np.arange(N) // b
    out = np.zeros((N, q.shape[1]), dtype=np.float64)
    lse = np.full(N, np.nan, dtype=np.float64)
    for I in query_blocks:
        r0, r1 = I * b, min((I + 1) * b, N)
        s = (q[r0:r1] @ k.T) * scale
        allowed = np.isin(key_block, np.asarray(list(kept[I]), dtype=np.int64))
        s[:, ~allowed] = -np.inf
        vals = v
        if k_g is not None:
            sg = (q[r0:r1] @ np.asarray(k_g, dtype=np.float64).T) * scale + g_bias[None, :]
            s = np.concatenate([s, sg], axis=1)
            vals = np.concatenate([v, np.asarray(v_g, dtype=np.float64)], axis=0)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        out[r0:r1] = (e / z) @ vals
        lse[r0:r1] = (m + np.log(z))[:, 0]
    return out, lse
