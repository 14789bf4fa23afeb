"""Oracle: BSA query-side pruning and token filling.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The BSA notes, key design 1 ("spatio-temporal query pruning and feature
filling") and "a complete example": inside each 3D block of queries, a token
that is nearly parallel to its local centre token is represented by it; the
block keeps only the fraction r of its tokens that differ most from their
centre (ranked by 1 - cos), attention is computed for those, and every pruned
position receives the output computed for its centre token.  Centres are
taken per small window (w_t, w_h, w_w) inside the block.

Readings taken where the notes leave a step open (each is a plain one):
- Blocks are the b consecutive tokens of the reordered sequence, the query
  blocks of the attention (with cuboid order and cuboids of b tokens, these
  are the 3D blocks).  Windows tile the latent grid from its origin; a window
  cut by the grid's edge keeps its tokens.
- The centre of a window is the token at offset floor((e - 1) / 2) along each
  axis, e the window's extent on that axis (the exact centre for odd extents,
  the lower middle for even ones).  Text-prefix tokens are their own centres.
- A centre's output is needed for filling, so centres are always computed:
  block I of n valid tokens holding c centres keeps m = min(n, max(ceil(r * n),
  c)) tokens: its centres, and the m - c other tokens of largest
  dissimilarity 1 - cos(q_centre, q_i) (ties by smaller reordered index).
  With the notes' example (4 x 4 x 4 blocks, 2 x 2 x 2 windows, r = 0.5) a
  block keeps its 8 centres and the 24 most distinct other tokens: 32 of 64,
  and 23,296 queries become 11,648, the numbers the notes print.
- cos of a zero vector: 1 - cos is 0 when both vectors are zero and 1 when
  one is.
float64 throughout; rows whose m-th and (m+1)-th candidates lie within 1e-5
in dissimilarity are reported as ties, since the GPU ranks float32 values.
"""
from __future__ import annotations

import math

import numpy as np


def window_anchors(T: int, H: int, W: int, win, prefix: int = 0) -> np.ndarray:
    """anchor[token] = the centre token of the token's window (raster indices, prefix tokens first)."""
    wt, wh, ww = (int(x) for x in win)
    if min(T, H, W, wt, wh, ww) < 1:
        raise ValueError("sides must be >= 1")
    anchor = np.empty(prefix + T * H * W, dtype=np.int64)
    anchor[:prefix] = np.arange(prefix)

    def centre(x, w, n):
        x0 = (x // w) * w
        e = min(x0 + w, n) - x0
        return x0 + (e - 1) // 2

    for t in range(T):
        ct = centre(t, wt, T)
        for h in range(H):
            ch = centre(h, wh, H)
            for w in range(W):
                cw = centre(w, ww, W)
                anchor[prefix + (t * H + h) * W + w] = prefix + (ct * H + ch) * W + cw
    return anchor


def anchors_reordered(perm: np.ndarray, anchor_tok: np.ndarray) -> np.ndarray:
    """The same map in reordered indices: anchor_r[i] = new index of the centre of token perm[i]."""
    perm = np.asarray(perm, dtype=np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.shape[0])
    return inv[np.asarray(anchor_tok)[perm]]


def dissimilarity(a: np.ndarray, q: np.ndarray) -> float:
    """1 - cos(a, q) in float64."""
    a = np.asarray(a, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    na, nq = math.sqrt(float(a @ a)), math.sqrt(float(q @ q))
    if na == 0.0 or nq == 0.0:
        return 0.0 if na == nq else 1.0
    return 1.0 - float(a @ q) / (na * nq)


def prune_block(q_r: np.ndarray, anchor_r: np.ndarray, rows, r: float):
    """Kept rows (ascending) of one block and a tie flag.  rows: the block's valid reordered
    rows; q_r: all reordered rows of the head; anchor_r: the reordered centre of each row."""
    rows = list(rows)
    n = len(rows)
    centres = [i for i in rows if anchor_r[i] == i]
    others = [i for i in rows if anchor_r[i] != i]
    m = min(n, max(math.ceil(r * n), len(centres)))
    dis = {i: dissimilarity(q_r[anchor_r[i]], q_r[i]) for i in others}
    ranked = sorted(others, key=lambda i: (-dis[i], i))
    take = m - len(centres)
    kept = sorted(centres + ranked[:take])
    tie = 0 < take < len(ranked) and abs(dis[ranked[take - 1]] - dis[ranked[take]]) <= 1e-5
    return kept, tie


def query_prune(q_r: np.ndarray, anchor_r: np.ndarray, N: int, b: int, r: float):
    """One (batch, head).  Returns (q_count [nb], rowsel [nb, b] kept rows ascending, -1 padded,
    kept [N] bool, ties: the blocks flagged as ties)."""
    nb = -(-N // b)
    q_count = np.zeros(nb, dtype=np.int32)
    rowsel = np.full((nb, b), -1, dtype=np.int32)
    kept = np.zeros(N, dtype=bool)
    ties = []
    for I in range(nb):
        rows = range(I * b, min((I + 1) * b, N))
        ks, tie = prune_block(q_r, anchor_r, rows, r)
        q_count[I] = len(ks)
        rowsel[I, :len(ks)] = ks
        kept[ks] = True
        if tie:
            ties.append(I)
    return q_count, rowsel, kept, ties


def fill(out_r: np.ndarray, kept: np.ndarray, anchor_r: np.ndarray) -> np.ndarray:
    """Token filling: every pruned row takes its centre's output (centres are always kept)."""
    out = np.array(out_r, copy=True)
    for i in np.nonzero(~np.asarray(kept))[0]:
        out[i] = out_r[anchor_r[i]]
    return out
