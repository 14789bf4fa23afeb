"""Pins for the oracle's permutations (curve and cuboid orders) and reorder.

The pages only name the Gilbert curve (Video-BLADE, "Preprocessing"), so it is
pinned by what any locality-preserving curve order must satisfy: a bijection,
a walk whose every step moves to a grid neighbour, blocks more compact than
raster blocks; plus closed forms for the cuboid order (BSA notes, "overall
framework").
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.perm import gilbert3d_cells, perm_cuboid, perm_gilbert3d, perm_identity, perm_invert
from oracle.reorder import inverse_reorder, reorder, reorder_fast
from workloads.configs import CONFIGS, latent_grid

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _steps(cells):
    a = np.asarray(cells)
    return np.abs(np.diff(a, axis=0))


@pytest.mark.parametrize("T,H,W", list(itertools.product(range(1, 8), repeat=3)))
def test_gilbert_small_boxes_are_unit_step_hamiltonian(T, H, W):
    cells = gilbert3d_cells(T, H, W)
    assert len(cells) == T * H * W
    assert len(set(cells)) == T * H * W
    assert cells[0] == (0, 0, 0)
    for t, h, w in cells:
        assert 0 <= t < T and 0 <= h < H and 0 <= w < W
    if len(cells) > 1:
        assert (_steps(cells).sum(axis=1) == 1).all()


@pytest.mark.parametrize("cfg", [c for c in CONFIGS], ids=lambda c: c.name)
def test_gilbert_workload_grids_unit_steps(cfg):
    cells = gilbert3d_cells(cfg.T, cfg.H, cfg.W)
    assert len(set(cells)) == cfg.n_video
    assert (_steps(cells).sum(axis=1) == 1).all()


def test_gilbert_line_is_identity():
    for W in (1, 2, 7, 64):
        assert np.array_equal(perm_gilbert3d(1, 1, W), np.arange(W))


def test_gilbert_2x2x2_is_a_gray_path():
    cells = gilbert3d_cells(2, 2, 2)
    assert len(set(cells)) == 8
    assert (_steps(cells).sum(axis=1) == 1).all()


def test_gilbert_blocks_more_compact_than_raster():
    # Wan2.1-1.3B latent grid, blocks of 128 tokens: mean squared distance of a
    # block's cells from their centroid.
    T, H, W = 21, 30, 52
    def spread(order):
        coords = np.array([(o // (H * W), (o // W) % H, o % W) for o in order], dtype=np.float64)
        nb = len(order) // 128
        blocks = coords[: nb * 128].reshape(nb, 128, 3)
        return float(((blocks - blocks.mean(axis=1, keepdims=True)) ** 2).sum(-1).mean())
    g = spread(perm_gilbert3d(T, H, W))
    r = spread(np.arange(T * H * W))
    assert g < 0.25 * r, (g, r)


def test_prefix_identity_then_curve():
    p = perm_gilbert3d(2, 3, 4, prefix=5)
    assert np.array_equal(p[:5], np.arange(5))
    assert sorted(p.tolist()) == list(range(5 + 24))
    assert p[5:].min() == 5


@pytest.mark.parametrize("grid,cub", [((4, 8, 16), (4, 4, 8)), ((5, 9, 7), (2, 4, 3)),
                                      ((3, 3, 3), (8, 4, 4)), ((31, 45, 80), (1, 8, 16))])
def test_cuboid_closed_form(grid, cub):
    T, H, W = grid
    ct, ch, cw = cub
    p = perm_cuboid(T, H, W, ct, ch, cw)
    assert sorted(p.tolist()) == list(range(T * H * W))
    # closed form: position of token (t,h,w) = tokens in earlier cuboids + rank inside its cuboid
    nct, nch, ncw = -(-T // ct), -(-H // ch), -(-W // cw)
    def size(i, n, c, L):
        return min(c, L - i * c)
    start = {}
    acc = 0
    for i, j, l in itertools.product(range(nct), range(nch), range(ncw)):
        start[(i, j, l)] = acc
        acc += size(i, nct, ct, T) * size(j, nch, ch, H) * size(l, ncw, cw, W)
    inv = perm_invert(p)
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        i, j, l = t // ct, h // ch, w // cw
        sh, sw = size(j, nch, ch, H), size(l, ncw, cw, W)
        rank = ((t - i * ct) * sh + (h - j * ch)) * sw + (w - l * cw)
        assert inv[(t * H + h) * W + w] == start[(i, j, l)] + rank


def test_cuboid_blocks_are_whole_cuboids_when_they_divide():
    # BSA notes: 3D cuboid blocks of (4,4,4) = 64 tokens; with b = cuboid volume
    # each block is exactly one cuboid.
    T, H, W = 8, 8, 8
    p = perm_cuboid(T, H, W, 4, 4, 4)
    for j in range(8):
        blk = p[j * 64:(j + 1) * 64]
        t, h, w = blk // 64, (blk // 8) % 8, blk % 8
        assert len({(a // 4, b // 4, c // 4) for a, b, c in zip(t, h, w)}) == 1


def test_invert():
    rng = np.random.default_rng(0)
    p = rng.permutation(100)
    inv = perm_invert(p)
    assert np.array_equal(inv[p], np.arange(100))
    with pytest.raises(ValueError):
        perm_invert(np.array([0, 0, 1]))


def test_latent_grids_match_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "latent_grids.json")))
    for c in g["cases"]:
        T, H, W = latent_grid(c["frames"], c["height"], c["width"])
        assert T * H * W == c["tokens"], c["source"]


def test_workload_token_counts():
    n = {c.cid: c.N for c in CONFIGS}
    assert n == {1: 2048, 2: 32760, 3: 17776, 4: 153600, 5: 111600}
    assert latent_grid(81, 480, 832) == (21, 30, 52)        # Wan2.1 480p, 81 frames
    assert latent_grid(121, 720, 1280) == (31, 45, 80)      # 720p, 121 frames


@pytest.mark.parametrize("per_head", [False, True])
def test_reorder_roundtrip_and_padding(per_head):
    rng = np.random.default_rng(1)
    B, N, Hh, d, b = 2, 37, 3, 4, 8
    Npad = -(-N // b) * b
    x = rng.standard_normal((B, N, Hh, d)).astype(np.float32)
    if per_head:
        perm = np.stack([rng.permutation(N) for _ in range(Hh)])
    else:
        perm = rng.permutation(N)
    y = reorder(x, perm, Npad)
    assert np.array_equal(y, reorder_fast(x, perm, Npad))
    assert (y[:, :, N:, :] == 0).all()
    assert np.array_equal(inverse_reorder(y, perm, N), x)
    h = 1
    p = perm[h] if per_head else perm
    assert np.array_equal(y[1, h, 5], x[1, p[5], h])


def test_identity_perm():
    assert np.array_equal(perm_identity(5), np.arange(5))
