"""Pins for the oracle's attention gradients and transposed block lists.

The gradients are checked against things the oracle does not use: central
finite differences of the oracle's forward (each input separately), torch's
autograd through scaled_dot_product_attention in float64 for the dense case,
and two exact identities of softmax attention.
"""
import numpy as np
import pytest
import torch

from oracle.attention import masked_attention
from oracle.attention_bwd import masked_attention_bwd, transpose_lists


def _rand(N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((N, d)) for _ in range(4)]


def _lists(nb, seed, empty_row=True):
    rng = np.random.default_rng(seed)
    kept = []
    for I in range(nb):
        m = int(rng.integers(1, nb + 1))
        kept.append(sorted(rng.choice(nb, size=m, replace=False).tolist()))
    if empty_row and nb > 2:
        kept[1] = []
    return kept


def _loss(q, k, v, w, N, b, kept, scale):
    # a query block without kept blocks has output 0 (the forward oracle leaves
    # NaN there: a softmax over no keys)
    o, _ = masked_attention(q, k, v, N, b, kept, scale)
    return float((np.nan_to_num(o, nan=0.0) * w).sum())


@pytest.mark.parametrize("N,b,d", [(37, 8, 6), (32, 16, 4), (50, 16, 5)])
def test_finite_differences_each_input(N, b, d):
    q, k, v, w = _rand(N, d, N * d)
    nb = -(-N // b)
    kept = _lists(nb, N)
    scale = 0.7
    dq, dk, dv = masked_attention_bwd(q, k, v, w, N, b, kept, scale)
    rng = np.random.default_rng(1)
    h = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        dirn = rng.standard_normal((N, d))
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p = [a + h * dirn if i == which else a for i, a in enumerate(args_p)]
        args_m = [a - h * dirn if i == which else a for i, a in enumerate(args_m)]
        fd = (_loss(*args_p, w, N, b, kept, scale) - _loss(*args_m, w, N, b, kept, scale)) / (2 * h)
        an = float((grad * dirn).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_single_entry_finite_differences():
    # one coordinate at a time on a tiny case, so a transposed or mis-indexed
    # term cannot cancel out in a random direction
    N, b, d = 12, 4, 3
    q, k, v, w = _rand(N, d, 5)
    kept = [[0, 2], [1], [0, 1, 2]]
    scale = 0.9
    dq, dk, dv = masked_attention_bwd(q, k, v, w, N, b, kept, scale)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for r in range(N):
            for c in range(d):
                ap = [a.copy() for a in (q, k, v)]
                am = [a.copy() for a in (q, k, v)]
                ap[which][r, c] += h
                am[which][r, c] -= h
                fd = (_loss(*ap, w, N, b, kept, scale) - _loss(*am, w, N, b, kept, scale)) / (2 * h)
                assert abs(fd - grad[r, c]) <= 1e-6, (which, r, c, fd, grad[r, c])


@pytest.mark.parametrize("N,b", [(64, 16), (45, 16)])
def test_dense_mask_matches_torch_autograd(N, b):
    q, k, v, w = _rand(N, 8, 3 * N)
    nb = -(-N // b)
    kept = [list(range(nb)) for _ in range(nb)]
    scale = 8 ** -0.5
    dq, dk, dv = masked_attention_bwd(q, k, v, w, N, b, kept, scale)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(t[0][None, None], t[1][None, None], t[2][None, None],
                                                         scale=scale)[0, 0]
    (o * torch.from_numpy(w)).sum().backward()
    for got, ref in ((dq, t[0].grad), (dk, t[1].grad), (dv, t[2].grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_softmax_identities(seed):
    # every row of dS sums to zero, so the key gradients sum to zero; the rows of
    # P sum to one, so the value gradients sum to the output gradient of every
    # query that attends to anything
    N, b, d = 70, 16, 7
    q, k, v, w = _rand(N, d, 100 + seed)
    nb = -(-N // b)
    kept = _lists(nb, seed)
    dq, dk, dv = masked_attention_bwd(q, k, v, w, N, b, kept, 0.5)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-10)
    rows = np.concatenate([np.arange(I * b, min((I + 1) * b, N)) for I in range(nb) if kept[I]])
    np.testing.assert_allclose(dv.sum(axis=0), w[rows].sum(axis=0), rtol=1e-10, atol=1e-10)
    # rows of a query block without kept blocks get no gradient
    np.testing.assert_array_equal(dq[b:2 * b], 0.0)


def test_unkept_keys_get_no_gradient():
    N, b, d = 48, 16, 4
    q, k, v, w = _rand(N, d, 9)
    kept = [[0], [0, 1], [1]]          # block 2 is never kept
    dq, dk, dv = masked_attention_bwd(q, k, v, w, N, b, kept, 1.0)
    assert (dk[32:] == 0).all() and (dv[32:] == 0).all()
    assert np.abs(dk[:32]).sum() > 0 and np.abs(dv[:32]).sum() > 0


@pytest.mark.parametrize("nb,seed", [(1, 0), (5, 1), (16, 2), (33, 3)])
def test_transpose_lists_brute_force(nb, seed):
    rng = np.random.default_rng(seed)
    cnt = rng.integers(-2, nb + 3, size=nb).astype(np.int32)
    idx = np.full((nb, nb), -1, dtype=np.int32)
    for I in range(nb):
        c = min(max(int(cnt[I]), 0), nb)
        idx[I, :c] = rng.choice(nb, size=c, replace=False)
        if c and rng.random() < 0.3:
            idx[I, 0] = nb + 4            # an invalid entry is skipped
    tc, ti = transpose_lists(cnt, idx)
    for J in range(nb):
        want = [I for I in range(nb) if J in idx[I, :min(max(int(cnt[I]), 0), nb)].tolist()]
        assert tc[J] == len(want)
        assert ti[J, :tc[J]].tolist() == want          # ascending I
        assert (ti[J, tc[J]:] == -1).all()
    # a repeated entry counts once, as in the attention oracle's sets
    if nb > 1:
        dup = idx.copy()
        c0 = min(max(int(cnt[0]), 0), nb)
        if c0 >= 2:
            dup[0, 1] = dup[0, 0]
            dc, di = transpose_lists(cnt, dup)
            J = int(dup[0, 0])
            if 0 <= J < nb:
                assert di[J, :dc[J]].tolist().count(0) == 1
    # transposing back gives every row's set of valid blocks
    bc, bi = transpose_lists(tc, ti)
    for I in range(nb):
        c = min(max(int(cnt[I]), 0), nb)
        valid = sorted(j for j in idx[I, :c].tolist() if 0 <= j < nb)
        assert sorted(bi[I, :bc[I]].tolist()) == valid
