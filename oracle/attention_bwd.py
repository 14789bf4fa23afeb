"""Oracle: gradients of the block-masked softmax attention (plain ASA), and the
key-to-query (transposed) form of the kept-block lists.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The forward is the attention of *Video-BLADE*, "Step 2.2: Computation": every
query of query block I attends to exactly the key blocks kept for I.  The
pages stop at the forward pass; the training use they describe (ASA inside
DiT training, and the BSA notes' sparse kernels with a backward driven by a
reverse, key-to-query scatter of the block lists) needs its gradient, which
is the ordinary derivative of that definition, written out here:

    S = Q K^T * scale  (-inf outside the kept blocks and for keys >= N)
    P = softmax_rows(S),   O = P V
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D),     D_q = sum_c P_qc dP_qc = sum_d dO_qd O_qd
    dQ = dS K * scale,     dK = dS^T Q * scale

float64 throughout, one query block at a time, no blocking or reordering
beyond the forward's.  Query rows >= N are not part of the problem (their
gradients are zero), and neither are key rows >= N.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def masked_attention_bwd(q_r: np.ndarray, k_r: np.ndarray, v_r: np.ndarray, do: np.ndarray, N: int, b: int,
                         kept: Sequence[Sequence[int]], scale: float):
    """One (batch, head), plain ASA.  q_r, k_r, v_r, do: [>= N, d] (rows >= N ignored);
    kept[I]: the key blocks of query block I (a set: repeats count once).

    Returns (dq, dk, dv), each [N, d] float64.  A query block with no kept block
    has output 0 and contributes no gradient.
    """
    q = np.asarray(q_r, dtype=np.float64)[:N]
    k = np.asarray(k_r, dtype=np.float64)[:N]
    v = np.asarray(v_r, dtype=np.float64)[:N]
    g = np.asarray(do, dtype=np.float64)[:N]
    nb = -(-N // b)
    key_block = np.arange(N) // b
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for I in range(nb):
        blocks = [J for J in set(kept[I]) if 0 <= J < nb]
        if not blocks:
            continue
        r0, r1 = I * b, min((I + 1) * b, N)
        allowed = np.isin(key_block, np.asarray(blocks, dtype=np.int64))
        s = (q[r0:r1] @ k.T) * scale
        s[:, ~allowed] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v
        dv += p.T @ g[r0:r1]
        dp = g[r0:r1] @ v.T
        D = (g[r0:r1] * o).sum(axis=1, keepdims=True)
        ds = p * (dp - D)
        dq[r0:r1] = (ds @ k) * scale
        dk += (ds.T @ q[r0:r1]) * scale
    return dq, dk, dv


def transpose_lists(kv_count: np.ndarray, kv_idx: np.ndarray):
    """Key-to-query lists of one (batch, head) from its query-to-key lists.

    kv_count [nb], kv_idx [nb, nb] (the first kv_count[I] entries of row I are
    the key blocks of query block I; counts are clamped into [0, nb] and entries
    outside [0, nb) skipped, as the attention does).  A row's list is a set of
    blocks, as in masked_attention_bwd: a repeated entry counts once.  Returns
    (kvT_count [nb], kvT_idx [nb, nb]): row J lists, ascending, the query blocks
    I whose list holds J; unused entries are -1.
    """
    nb = kv_count.shape[0]
    holds = [set() for _ in range(nb)]
    for I in range(nb):
        c = min(max(int(kv_count[I]), 0), nb)
        for J in kv_idx[I, :c].tolist():
            if 0 <= J < nb:
                holds[J].add(I)
    cnt = np.array([len(h) for h in holds], dtype=np.int32)
    idx = np.full((nb, nb), -1, dtype=np.int32)
    for J in range(nb):
        idx[J, :cnt[J]] = sorted(holds[J])
    return cnt, idx
