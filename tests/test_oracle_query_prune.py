"""Pins for the oracle's BSA query pruning and token filling (oracle/query_prune.py)."""
import json
import math
import os

import numpy as np
import pytest

from oracle.attention import masked_attention
from oracle.perm import perm_cuboid, perm_gilbert3d
from oracle.query_prune import (anchors_reordered, dissimilarity, fill, prune_block, query_prune,
                                window_anchors)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_counts():
    # the pages' example: 23,296 queries -> 11,648 at keep ratio 0.5, whatever the values
    g = json.load(open(os.path.join(GOLDEN, "bsa_query_pruning.json")))
    T, H, W = g["latent_grid"]
    assert T * H * W == g["tokens"]
    perm = perm_cuboid(T, H, W, *g["block"])
    anc = anchors_reordered(perm, window_anchors(T, H, W, g["window"]))
    b = int(np.prod(g["block"]))
    N = T * H * W
    rng = np.random.default_rng(0)
    q = rng.standard_normal((N, 4))
    cnt, rowsel, kept, _ = query_prune(q, anc, N, b, g["keep_ratio"])
    assert int(cnt.sum()) == g["queries_kept"] == int(kept.sum())
    centres = anc == np.arange(N)
    assert (centres.reshape(-1, b).sum(axis=1) == 8).all()       # eight 2x2x2 windows per 4x4x4 block
    assert (kept[centres]).all()


def test_anchor_geometry():
    T, H, W, win, prefix = 5, 7, 6, (2, 3, 4), 3
    anc = window_anchors(T, H, W, win, prefix)
    assert (anc[:prefix] == np.arange(prefix)).all()
    coords = lambda x: np.unravel_index(x - prefix, (T, H, W))
    seen = {}
    for tok in range(prefix, prefix + T * H * W):
        t, h, w = coords(tok)
        at, ah, aw = coords(anc[tok])
        key = (t // win[0], h // win[1], w // win[2])
        assert (at // win[0], ah // win[1], aw // win[2]) == key      # the centre lies in the window
        seen.setdefault(key, set()).add(int(anc[tok]))
        assert anc[anc[tok]] == anc[tok]                                # a centre is its own centre
    assert all(len(v) == 1 for v in seen.values())                      # one centre per window
    # odd extent: the exact centre; even: the lower middle; a cut window uses its own extent
    a1 = window_anchors(1, 1, 7, (1, 1, 3))
    assert a1.tolist() == [1, 1, 1, 4, 4, 4, 6]
    a2 = window_anchors(1, 1, 6, (1, 1, 4))
    assert a2.tolist() == [1, 1, 1, 1, 4, 4]


def test_dissimilarity_closed_forms():
    a = np.array([1.0, 2.0, -2.0])
    assert abs(dissimilarity(a, 3.5 * a)) < 1e-15             # parallel
    assert abs(dissimilarity(a, -a) - 2.0) < 1e-15            # antiparallel
    assert abs(dissimilarity(a, np.array([2.0, -1.0, 0.0])) - 1.0) < 1e-15   # orthogonal
    assert abs(dissimilarity(np.array([1.0, 0.0]), np.array([1.0, 1.0])) - (1 - 1 / math.sqrt(2))) < 1e-15
    assert dissimilarity(np.zeros(3), np.zeros(3)) == 0.0
    assert dissimilarity(np.zeros(3), a) == 1.0


@pytest.mark.parametrize("seed", range(6))
def test_block_selection_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 12))
    d = 3
    q = rng.standard_normal((n, d))
    anc = np.arange(n)
    centres = sorted(rng.choice(n, size=int(rng.integers(1, 3)), replace=False).tolist())
    for i in range(n):
        if i not in centres:
            anc[i] = centres[int(rng.integers(0, len(centres)))]
    for r in (0.05, 0.3, 0.5, 0.77, 1.0):
        kept, _ = prune_block(q, anc, range(n), r)
        m = min(n, max(math.ceil(r * n), len(centres)))
        assert len(kept) == m and kept == sorted(kept)
        assert set(centres) <= set(kept)
        dis = {i: dissimilarity(q[anc[i]], q[i]) for i in range(n)}
        ins = [i for i in kept if i not in centres]
        outs = [i for i in range(n) if i not in kept]
        for a in ins:                          # every kept token outranks every pruned one
            for o in outs:
                assert (dis[a], -a) > (dis[o], -o)
    # brute force on the smallest case: among all subsets that hold the centres and have m
    # elements, the kept one has the largest dissimilarity sum (ties aside)
    from itertools import combinations
    kept, tie = prune_block(q, anc, range(n), 0.5)
    if not tie:
        m = len(kept)
        others = [i for i in range(n) if i not in centres]
        best = max(combinations(others, m - len(centres)),
                   key=lambda s: sum(dissimilarity(q[anc[i]], q[i]) for i in s))
        assert sorted(list(best) + centres) == kept


def test_ratio_limits_and_nesting():
    rng = np.random.default_rng(7)
    T, H, W = 3, 8, 8
    perm = perm_gilbert3d(T, H, W)
    anc = anchors_reordered(perm, window_anchors(T, H, W, (1, 2, 2)))
    N, b = T * H * W, 64
    q = rng.standard_normal((N, 8))
    full = query_prune(q, anc, N, b, 1.0)
    assert full[2].all() and (full[0] == [64, 64, 64]).all()
    low = query_prune(q, anc, N, b, 1e-3)
    assert (low[2] == (anc == np.arange(N))).all()                   # only the centres
    prev = None
    for r in (0.2, 0.4, 0.6, 0.8):
        k = query_prune(q, anc, N, b, r)[2]
        if prev is not None:
            assert (prev <= k).all()                                   # nested in r
        prev = k


def test_fill_and_pruned_attention():
    """Kept rows carry the unpruned attention output; a pruned row carries its centre's."""
    rng = np.random.default_rng(3)
    T, H, W, d, b = 2, 8, 8, 8, 64
    perm = perm_cuboid(T, H, W, 1, 8, 8)
    anc = anchors_reordered(perm, window_anchors(T, H, W, (1, 2, 2)))
    N = T * H * W
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    kept_blocks = [[0, 1], [1]]
    full, _ = masked_attention(q, k, v, N, b, kept_blocks, 0.3)
    cnt, rowsel, kept, _ = query_prune(q, anc, N, b, 0.25)
    out = fill(full, kept, anc)
    assert np.array_equal(out[kept], full[kept])
    for i in np.nonzero(~kept)[0]:
        assert np.array_equal(out[i], full[anc[i]])
    assert int(kept.sum()) == int(cnt.sum()) == 2 * 16       # 16 centres per block of 64 (2x2 windows)
    for I in range(2):
        assert rowsel[I, :cnt[I]].tolist() == sorted(np.nonzero(kept[I * b:(I + 1) * b])[0] + I * b)
