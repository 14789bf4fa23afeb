"""Oracle: token permutations (locality-preserving reorder).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module;
only tests, the smoke check and the CPU-baseline leg of the bench use it.

What is computed
----------------
*Video-BLADE* ("Preprocessing: Locality-preserving token rearrangement") and the
BLADE notes (key design 1) reorder the flattened video tokens along a Gilbert
space-filling curve before cutting them into blocks, so that each block holds a
spatially contiguous region.  The pages only name the curve (credited to
SpargeAttention); they do not define it.  The reading taken here is a
generalised Hilbert curve over the whole T x H x W latent box, defined by the
recursion below (the same recursion is written independently, in C++, in the
library; the two must agree bit for bit).

*Bidirectional Sparse Attention* ("overall framework", "a complete example")
instead cuts the latent into 3D cuboids; *VEDA* (key design 2) draws the cuboid
shape per head from the factorisations of the tile size.  `perm_cuboid` gives
that order: cuboids in raster order of (t//ct, h//ch, w//cw), tokens inside a
cuboid in raster order, partial cuboids at the borders holding fewer tokens.

Convention: perm[new] = old, where old = prefix + t*H*W + h*W + w is the raster
index and new is the position after reordering.  Positions < prefix (text
tokens) are left in place.

The curve recursion (one definition, shared with the C++ host code by
specification only)
--------------------------------------------------------------------------
A call walk(o, a, b, c) visits every cell of the box
{o + i*ua + j*ub + k*uc : 0 <= i < |a|, 0 <= j < |b|, 0 <= k < |c|}
exactly once (ua, ub, uc are the unit vectors of the axis-aligned integer
vectors a, b, c).  It starts at o and ends at o + (|a|-1)*ua, the corner next
to o along the major vector a.  With A, B, C = |a|, |b|, |c|, the first rule
that applies is taken:

1. B == C == 1: the straight line along a.
2. A == 1 (start and end would coincide; never reached from the top level):
   the 2D walk of the (b, c) plane (major = the longer, ties b), reversed.
3. C == 1: the 2D walk of (a, b).   B == 1: the 2D walk of (a, c).
4. A >= 4 and 2A > 3B and 2A > 3C (long along a): split a at
   A1 = even_half(A, 2): walk(o, a1, b, c); walk(o + a1, a - a1, b, c).
5. A == B == C == 2: the Gray-code order o, o+uc, o+ub+uc, o+ub, o+ua+ub,
   o+ua+ub+uc, o+ua+uc, o+ua.
6. Otherwise the "U" in the plane of a and the longer minor x (ties: b),
   with the other minor y passive: X1 = even_half(X, 1), A1 = A // 2;
   walk(o, x1, y, a1); walk(o + x1, a, y, x - x1);
   walk(o + (a - ua) + (x1 - ux), -x1, y, -(a - a1)).

The 2D walk2(o, a, b), same contract: B == 1: the line along a; A == 1: the
line along b, reversed; A >= 4 and 2A > 3B: split a at even_half(A, 2);
otherwise the "U": B1 = even_half(B, 1), A1 = A // 2; walk2(o, b1, a1);
walk2(o + b1, a, b - b1); walk2(o + (a - ua) + (b1 - ub), -b1, -(a - a1)).

even_half(L, r) = L // 2, moved up by one when that is odd and L minus it
stays >= r.

Why this keeps every step a unit step.  A walk from a corner to the next
corner along a exists with unit steps only if the major side is even or all
sides are odd (colour the cells by the parity of i+j+k).  Call such a box
good.  Each split above maps a good box to good pieces whose major sides are
>= 2 (the long split gives even halves, or an even and an odd half of an
all-odd box; the "U" gives X1 even to its two side pieces, and the middle
piece keeps the parent's major).  The top level takes as major the longest
even side when one exists, so the root is good: every step of the curve then
moves exactly one cell (the tests check this exhaustively on small grids and
on every workload grid).

Top level: major = the longest side of even length, else the longest side;
then the longer remaining side as b (ties: w before h before t); the curve
starts at (0, 0, 0).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "gilbert3d_cells",
    "perm_gilbert3d",
    "perm_cuboid",
    "perm_invert",
    "perm_identity",
]


def _length(v):
    return abs(v[0]) + abs(v[1]) + abs(v[2])


def _unit(v):
    return ((v[0] > 0) - (v[0] < 0), (v[1] > 0) - (v[1] < 0), (v[2] > 0) - (v[2] < 0))


def _scale(v, n):
    """Vector along v's axis, with v's sign, of length n."""
    u = _unit(v)
    return (u[0] * n, u[1] * n, u[2] * n)


def _add(*vs):
    return (sum(v[0] for v in vs), sum(v[1] for v in vs), sum(v[2] for v in vs))


def _neg(v):
    return (-v[0], -v[1], -v[2])


def _sub(p, q):
    return (p[0] - q[0], p[1] - q[1], p[2] - q[2])


def _even_half(L, rest_min):
    """L // 2, moved up by one when odd and L - h stays >= rest_min."""
    h = L // 2
    if h % 2 == 1 and L - (h + 1) >= rest_min:
        h += 1
    return h


class _Walker:
    def __init__(self):
        self.out = []

    def line(self, o, a):
        u = _unit(a)
        for i in range(_length(a)):
            self.out.append((o[0] + i * u[0], o[1] + i * u[1], o[2] + i * u[2]))

    def reversed_plane(self, o, b, c):
        sub = _Walker()
        if _length(b) >= _length(c):
            sub.walk2(o, b, c)
        else:
            sub.walk2(o, c, b)
        self.out.extend(reversed(sub.out))

    # ---- 2D -------------------------------------------------------------
    def walk2(self, o, a, b):
        A, B = _length(a), _length(b)
        if B == 1:
            self.line(o, a)
            return
        if A == 1:
            self.line(_add(o, _scale(b, B - 1)), _neg(b))
            return
        if A >= 4 and 2 * A > 3 * B:
            a1 = _scale(a, _even_half(A, 2))
            self.walk2(o, a1, b)
            self.walk2(_add(o, a1), _sub(a, a1), b)
            return
        a1, b1 = _scale(a, A // 2), _scale(b, _even_half(B, 1))
        ua, ub = _unit(a), _unit(b)
        self.walk2(o, b1, a1)
        self.walk2(_add(o, b1), a, _sub(b, b1))
        self.walk2(_add(o, _sub(a, ua), _sub(b1, ub)), _neg(b1), _neg(_sub(a, a1)))

    # ---- 3D -------------------------------------------------------------
    def walk3(self, o, a, b, c):
        A, B, C = _length(a), _length(b), _length(c)
        if B == 1 and C == 1:
            self.line(o, a)
            return
        if A == 1:
            self.reversed_plane(o, b, c)
            return
        if C == 1:
            self.walk2(o, a, b)
            return
        if B == 1:
            self.walk2(o, a, c)
            return
        if A >= 4 and 2 * A > 3 * B and 2 * A > 3 * C:
            a1 = _scale(a, _even_half(A, 2))
            self.walk3(o, a1, b, c)
            self.walk3(_add(o, a1), _sub(a, a1), b, c)
            return
        if A == 2 and B == 2 and C == 2:
            ua, ub, uc = _unit(a), _unit(b), _unit(c)
            for p in ((), (uc,), (ub, uc), (ub,), (ua, ub), (ua, ub, uc), (ua, uc), (ua,)):
                self.out.append(_add(o, *p))
            return
        x, y = (b, c) if B >= C else (c, b)
        a1, x1 = _scale(a, A // 2), _scale(x, _even_half(_length(x), 1))
        ua, ux = _unit(a), _unit(x)
        self.walk3(o, x1, y, a1)
        self.walk3(_add(o, x1), a, y, _sub(x, x1))
        self.walk3(_add(o, _sub(a, ua), _sub(x1, ux)), _neg(x1), y, _neg(_sub(a, a1)))


def gilbert3d_cells(T: int, H: int, W: int) -> list:
    """Cells (t, h, w) of the T x H x W box in curve order."""
    if T < 1 or H < 1 or W < 1:
        raise ValueError("grid sides must be >= 1")
    # (length, tie rank, unit vector in (t, h, w) coordinates); w ranks first
    axes = [(W, 0, (0, 0, 1)), (H, 1, (0, 1, 0)), (T, 2, (1, 0, 0))]
    even = [e for e in axes if e[0] % 2 == 0]
    major = min(even or axes, key=lambda e: (-e[0], e[1]))
    rest = sorted((e for e in axes if e is not major), key=lambda e: (-e[0], e[1]))
    vecs = [_scale(u, L) for (L, _, u) in [major] + rest]
    w = _Walker()
    w.walk3((0, 0, 0), vecs[0], vecs[1], vecs[2])
    return w.out


def perm_gilbert3d(T: int, H: int, W: int, prefix: int = 0) -> np.ndarray:
    """perm[new] = old for the Gilbert order of a T x H x W grid after `prefix` fixed tokens."""
    cells = gilbert3d_cells(T, H, W)
    perm = np.empty(prefix + T * H * W, dtype=np.int64)
    perm[:prefix] = np.arange(prefix)
    for i, (t, h, w) in enumerate(cells):
        perm[prefix + i] = prefix + (t * H + h) * W + w
    return perm


def perm_cuboid(T: int, H: int, W: int, ct: int, ch: int, cw: int, prefix: int = 0) -> np.ndarray:
    """Cuboid-major order: cuboids in raster order, tokens raster order inside each cuboid."""
    if min(T, H, W, ct, ch, cw) < 1:
        raise ValueError("sides must be >= 1")
    order = []
    for T0 in range(0, T, ct):
        for H0 in range(0, H, ch):
            for W0 in range(0, W, cw):
                for t in range(T0, min(T0 + ct, T)):
                    for h in range(H0, min(H0 + ch, H)):
                        for w in range(W0, min(W0 + cw, W)):
                            order.append(prefix + (t * H + h) * W + w)
    return np.concatenate([np.arange(prefix, dtype=np.int64), np.asarray(order, dtype=np.int64)])


def perm_identity(n: int) -> np.ndarray:
    return np.arange(n, dtype=np.int64)


def perm_invert(perm: np.ndarray) -> np.ndarray:
    """inv[old] = new."""
    perm = np.asarray(perm)
    inv = np.full(perm.shape[-1], -1, dtype=np.int64)
    for new, old in enumerate(perm.tolist()):
        if old < 0 or old >= inv.size or inv[old] != -1:
            raise ValueError("not a permutation")
        inv[old] = new
    return inv
