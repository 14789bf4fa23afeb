"""Oracle: sparsity and work accounting.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

*Video-BLADE* "Efficiency analysis" reports an "effective sparsity rate"
without defining it.  The reading taken is the block sparsity over all
(batch, head, query block, key block) pairs; a token-weighted sparsity is also
given.  The BSA notes' worked example combines a query keep ratio with a KV
keep ratio multiplicatively (0.5 x 0.14 -> sparsity 0.93); `combined_sparsity`
is that rule (query pruning itself is not part of this path).
"""
from __future__ import annotations

import numpy as np


def block_sparsity(kv_count: np.ndarray, nb: int) -> float:
    c = np.asarray(kv_count, dtype=np.float64)
    return 1.0 - c.sum() / (c.size * nb)


def kept_pairs_tokens(kv_count: np.ndarray, kv_idx: np.ndarray, N: int, b: int) -> float:
    """sum over kept (I, J) of |I| * |J| (valid tokens), over all rows."""
    nb = -(-N // b)
    L = np.array([min(b, N - J * b) for J in range(nb)], dtype=np.float64)
    cnt = np.asarray(kv_count).reshape(-1, nb)
    idx = np.asarray(kv_idx).reshape(-1, nb, nb)
    tot = 0.0
    for r in range(cnt.shape[0]):
        for I in range(nb):
            js = idx[r, I, :cnt[r, I]]
            tot += L[I] * L[js].sum()
    return tot


def token_sparsity(kv_count, kv_idx, N: int, b: int) -> float:
    rows = np.asarray(kv_count).reshape(-1, -(-N // b)).shape[0]
    return 1.0 - kept_pairs_tokens(kv_count, kv_idx, N, b) / (rows * float(N) ** 2)


def executed_flop(kv_count, kv_idx, N: int, b: int, d: int, heads_total: int, Ng: int = 0) -> float:
    """4 d sum|I||J| over kept pairs, plus 4 d N Ng per (batch, head) for global tokens."""
    return 4.0 * d * kept_pairs_tokens(kv_count, kv_idx, N, b) + 4.0 * d * heads_total * N * Ng


def dense_flop(batch: int, heads: int, N: int, d: int) -> float:
    return 4.0 * batch * heads * float(N) ** 2 * d


def combined_sparsity(query_keep: float, kv_keep: float) -> float:
    return 1.0 - query_keep * kv_keep
