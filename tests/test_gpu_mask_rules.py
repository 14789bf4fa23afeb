"""GPU parity: the top-k and statistical-threshold rules (dbs_build_mask_rule)
against the oracle's, bit for bit on identical P_imp arrays, for the
one-wavefront rows (nb <= 256) and the LDS rows (nb up to 4096).  The
statistical rule compares against a float64 threshold; rows the oracle flags as
ties (a score within 1e-12 of the threshold) are excluded and counted."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, say
from oracle.mask_rules import build_mask_rule as o_rule

pytestmark = pytest.mark.gpu


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _rows(kind, R, nb, rng):
    if kind == "uniform":
        P = rng.random((R, nb))
    elif kind == "peaked":
        P = np.exp(-30 * rng.random((R, nb)))
    elif kind == "dyadic":                 # many exact ties
        P = rng.integers(0, 5, size=(R, nb)) / 8.0
    elif kind == "normal":
        P = np.clip(0.5 + 0.1 * rng.standard_normal((R, nb)), 0, 1)
    else:
        raise ValueError(kind)
    P = np.minimum(P, 1.0).astype(np.float32)
    if R > 3:
        P[1, nb // 2] = np.nan             # invalid rows keep every block
        P[2, 0] = 1.5
    return P


def _compare(P, rule, param, rows):
    """P [1, 1, nb, nb]; the oracle checks the listed rows."""
    ops = _ops()
    nb = P.shape[-1]
    cnt, idx, msk = ops.build_mask_rule(dev(P), rule, param, want_mask=True)
    torch.cuda.synchronize()
    cnt, idx, msk = host(cnt).reshape(-1), host(idx).reshape(-1, nb), host(msk).reshape(-1, nb)
    rc, ri, rm, ties = o_rule(P.reshape(-1, nb)[rows], rule, param)
    tie = set(ties)
    for k, r in enumerate(rows):
        if k in tie:
            continue
        assert cnt[r] == rc[k], (rule, param, r)
        assert np.array_equal(idx[r, :rc[k]], ri[k, :rc[k]]), (rule, param, r)
        assert np.array_equal(msk[r], rm[k]), (rule, param, r)
    return len(tie)


def _case(nb, kind, seed):
    rng = np.random.default_rng(seed)
    P = _rows(kind, nb, nb, rng)[None, None]
    rows = list(range(nb)) if nb <= 256 else sorted({0, 1, 2, nb - 1} | set(rng.choice(nb, 44, replace=False).tolist()))
    return P, rows


@pytest.mark.parametrize("nb", [1, 7, 64, 100, 256, 300, 1024, 2000])
@pytest.mark.parametrize("kind", ["uniform", "peaked", "dyadic", "normal"])
def test_topk_bit_exact(nb, kind):
    say("mask topk", nb, kind)
    P, rows = _case(nb, kind, nb * 7 + len(kind))
    for k in sorted({1, 3, max(1, nb // 2), nb, nb + 5}):
        _compare(P, "topk", k, rows)


@pytest.mark.parametrize("nb", [1, 7, 64, 100, 256, 300, 1024, 2000])
@pytest.mark.parametrize("kind", ["uniform", "peaked", "dyadic", "normal"])
def test_stat_bit_exact_outside_ties(nb, kind):
    say("mask stat", nb, kind)
    P, rows = _case(nb, kind, nb * 11 + len(kind))
    us = [-1.0, 0.0, 0.5, 2.2]
    if nb > 16:
        us.append(_ops().stat_quantile(16, nb))
    for u in us:
        n_ties = _compare(P, "stat", u, rows)
        if kind != "dyadic":                  # exact ties are rare except on dyadic rows
            assert n_ties <= max(1, len(rows) // 8), (u, n_ties)


def test_cumulative_rule_equals_build_mask():
    ops = _ops()
    rng = np.random.default_rng(5)
    P = dev(_rows("peaked", 2 * 256, 256, rng).reshape(2, 1, 256, 256))
    a = ops.build_mask(P, 0.9, want_mask=True)
    b = ops.build_mask_rule(P, "cumulative", 0.9, want_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])   # counts and masks (entries past a count are unspecified)


@pytest.mark.parametrize("nb", [64, 256, 1200])
def test_stat_k_equals_stat_with_library_quantile(nb):
    """DBS_RULE_STAT_K (the library computes u = U(1 - k/nb) itself) gives exactly the lists of
    DBS_RULE_STAT at that u, and the oracle's rule at scipy's quantile outside ties."""
    from scipy.special import ndtri
    say("mask stat_k", nb)
    ops = _ops()
    P, rows = _case(nb, "normal", nb + 3)
    Pd = dev(P)
    for kk in (1, 16, nb // 3):
        a = ops.build_mask_rule(Pd, "stat_k", kk, want_mask=True)
        b = ops.build_mask_rule(Pd, "stat", ops.stat_quantile(kk, nb), want_mask=True)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
        _compare(P, "stat", float(ndtri(1 - kk / nb)), rows)
