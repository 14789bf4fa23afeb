"""GPU parity: build_mask against the oracle's exact mask builder, bit for bit,
on identical P_imp arrays (random, tie-heavy, degenerate and invalid rows)."""
import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, dev, host, say
from oracle.mask import build_mask as o_build_mask

pytestmark = pytest.mark.gpu


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _rows(kind: str, R: int, nb: int, rng) -> np.ndarray:
    if kind == "uniform":
        P = rng.random((R, nb))
    elif kind == "peaked":
        P = np.exp(-30 * rng.random((R, nb)))
    elif kind == "softmaxish":
        s = rng.standard_normal((R, nb)) * 4
        P = np.exp(s - s.max(axis=1, keepdims=True))
    elif kind == "dyadic":                 # many exact ties and exact-threshold cuts
        P = rng.integers(0, 5, size=(R, nb)) / 8.0
    elif kind == "tiny":                   # denormals and zeros
        P = rng.integers(0, 4, size=(R, nb)) * np.float32(1e-45)
        P[:, 0] = 1e-40
    else:
        raise ValueError(kind)
    return np.minimum(P, 1.0).astype(np.float32)


def _compare(P: np.ndarray, tau: float, rows=None):
    ops = _ops()
    B, Hh, nb, _ = P.shape
    g = [Guarded((B, Hh, nb), torch.int32), Guarded((B, Hh, nb, nb), torch.int32),
         Guarded((B, Hh, nb, nb), torch.uint8, fill=171), Guarded((B * Hh * nb,), torch.int32)]
    cnt, idx, msk, order = ops.build_mask(dev(P), tau, kv_count=g[0].view, kv_idx=g[1].view, mask=g[2].view,
                                          order=g[3].view)
    torch.cuda.synchronize()
    assert all(x.intact() for x in g)          # nothing written outside the outputs
    assert np.array_equal(np.sort(host(order)), np.arange(B * Hh * nb))
    cnt, idx, msk = host(cnt), host(idx), host(msk)
    flatP = P.reshape(-1, nb)
    if rows is None:
        rows = range(flatP.shape[0])
    rows = list(rows)
    rc, ri, rm, ties = o_build_mask(flatP[rows], tau)
    fc = cnt.reshape(-1)[rows]
    fi = idx.reshape(-1, nb)[rows]
    fm = msk.reshape(-1, nb)[rows]
    assert np.array_equal(fc, rc), np.nonzero(fc != rc)
    for j in range(len(rows)):
        assert np.array_equal(fi[j, :rc[j]], ri[j, :rc[j]]), rows[j]
    assert np.array_equal(fm, rm)
    return len(ties)


@pytest.mark.parametrize("nb", [1, 5, 64, 139, 256, 1200])
@pytest.mark.parametrize("kind", ["uniform", "peaked", "softmaxish", "dyadic", "tiny"])
@pytest.mark.parametrize("tau", [0.5, 0.9, 0.95, 1.0])
def test_mask_bitexact(nb, kind, tau):
    say("mask", nb, kind, tau)
    rng = np.random.default_rng(nb * 7 + len(kind))
    R = 8 if nb >= 1000 else 32
    U = _rows(kind, R, nb, rng).reshape(2, R // 2, 1, nb)
    P = np.ascontiguousarray(np.broadcast_to(U, (2, R // 2, nb, nb)))   # each head repeats one row
    ops = _ops()
    cnt, idx, _ = ops.build_mask(dev(P), tau)
    torch.cuda.synchronize()
    cnt, idx = host(cnt), host(idx)
    for bi in range(2):                   # every copy of a row got the same answer
        for h in range(R // 2):
            c = cnt[bi, h]
            assert (c == c[0]).all()
            assert (idx[bi, h, :, :c[0]] == idx[bi, h, :1, :c[0]]).all()
    rows = list(range(0, 2 * (R // 2) * nb, nb))
    _compare(P, tau, rows)


def test_mask_tau_limits_and_ties():
    say("mask limits")
    P = np.array([[0.125, 0.5, 0.25, 0.125], [0.0, 0.0, 0.0, 0.0],
                  [0.25, 0.25, 0.25, 0.25], [1.0, 1.0, 0.0, 0.5]], dtype=np.float32)
    P = P.reshape(1, 1, 4, 4)
    for tau in (1e-6, 0.5, 0.75, 0.8, 0.999, 1.0):
        _compare(P, tau)


def test_mask_invalid_rows_keep_all():
    say("mask invalid")
    P = np.full((1, 1, 4, 4), 0.25, dtype=np.float32)
    P[0, 0, 0, 1] = np.nan
    P[0, 0, 1, 2] = -0.5
    P[0, 0, 2, 3] = 1.5
    P[0, 0, 3, 0] = -0.0
    _compare(P, 0.5)
    cnt, _, _ = _ops().build_mask(dev(P), 0.5)
    c = host(cnt)[0, 0]
    assert c[:3].tolist() == [4, 4, 4] and c[3] == 2


def test_mask_max_nb():
    say("mask nb=4096")
    rng = np.random.default_rng(3)
    P = _rows("softmaxish", 3, 4096, rng).reshape(1, 3, 1, 4096)
    P = np.ascontiguousarray(np.broadcast_to(P, (1, 3, 4096, 4096)))
    _compare(P, 0.9, rows=[0, 4096 + 17, 2 * 4096 + 4095])


def test_mask_deterministic():
    rng = np.random.default_rng(4)
    P = dev(_rows("peaked", 256, 256, rng).reshape(1, 1, 256, 256))
    ops = _ops()
    a = [host(t) for t in ops.build_mask(P, 0.9)[:2]]
    b = [host(t) for t in ops.build_mask(P, 0.9)[:2]]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _xcd_ranges(total: int):
    """The eight contiguous row ranges of the work order (first total % 8 one longer)."""
    per, rem = divmod(total, 8)
    out, start = [], 0
    for x in range(8):
        size = per + (1 if x < rem else 0)
        out.append((start, size))
        start += size
    return out


@pytest.mark.parametrize("B,Hh,nb", [(1, 12, 256), (2, 3, 139), (1, 1, 5), (1, 2, 1200)])
def test_mask_work_order(B, Hh, nb):
    """The work order is a permutation of the rows that lists each XCD range
    by kept count descending (the rule stated in include/dbs.h)."""
    say("mask order", B, Hh, nb)
    rng = np.random.default_rng(B * 1000 + Hh * 10 + nb)
    P = _rows("softmaxish", B * Hh * nb, nb, rng).reshape(B, Hh, nb, nb)
    ops = _ops()
    cnt, _, _, order = ops.build_mask(dev(P), 0.9, want_order=True)
    torch.cuda.synchronize()
    c, o = host(cnt).reshape(-1), host(order)
    total = B * Hh * nb
    assert np.array_equal(np.sort(o), np.arange(total))
    for start, size in _xcd_ranges(total):
        seg = o[start:start + size]
        assert ((seg >= start) & (seg < start + size)).all()
        assert (np.diff(c[seg]) <= 0).all()
