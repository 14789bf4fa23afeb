"""Oracle: gather tokens into curve order and scatter them back.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

*Video-BLADE*, "Preprocessing": Q, K and V are rearranged along the curve
before they are cut into blocks of b tokens.  The layer must hand its output
back in the original token order (the reading taken: the inverse gather, so
that inverse(forward(x)) == x).

Layouts: x is [B, N, Hh, d] (a DiT layout); y is [B, Hh, Npad, d] with rows
N..Npad-1 zero.  perm is [N] (shared by every head) or [Hh, N].
"""
from __future__ import annotations

import numpy as np


def _perm_for(perm: np.ndarray, h: int) -> np.ndarray:
    perm = np.asarray(perm)
    return perm[h] if perm.ndim == 2 else perm


def reorder(x: np.ndarray, perm: np.ndarray, Npad: int) -> np.ndarray:
    B, N, Hh, d = x.shape
    y = np.zeros((B, Hh, Npad, d), dtype=x.dtype)
    for bi in range(B):
        for h in range(Hh):
            p = _perm_for(perm, h)
            for new in range(N):
                y[bi, h, new, :] = x[bi, p[new], h, :]
    return y


def reorder_fast(x: np.ndarray, perm: np.ndarray, Npad: int) -> np.ndarray:
    """Same result as `reorder`, by fancy indexing (used on large inputs)."""
    B, N, Hh, d = x.shape
    y = np.zeros((B, Hh, Npad, d), dtype=x.dtype)
    for h in range(Hh):
        y[:, h, :N, :] = x[:, _perm_for(perm, h), h, :]
    return y


def inverse_reorder(y: np.ndarray, perm: np.ndarray, N: int) -> np.ndarray:
    B, Hh, Npad, d = y.shape
    x = np.zeros((B, N, Hh, d), dtype=y.dtype)
    for h in range(Hh):
        p = _perm_for(perm, h)
        x[:, p, h, :] = y[:, h, :N, :]
    return x
