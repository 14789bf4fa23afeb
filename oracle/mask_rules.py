"""Oracle: two alternative block-selection rules on the same importance map.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Both take a P_imp row and return the kept key blocks, in the form the
cumulative rule of oracle/mask.py returns them, so they drop into the same
place on the path (P_imp -> kept-block lists -> attention):

- top-k: the k blocks of largest importance (ties by block index, ascending),
  the fixed-budget rule that the BSA notes argue against and that VEDA uses
  for its oracle masks ("keep the top-k key blocks of each query block").
- statistical threshold (BSA notes, design 2: an adaptive threshold built
  from the block scores' mean and standard deviation and a quantile of the
  normal distribution, p = mean + std * U(1 - k/n), n the number of blocks, k
  the target number of candidates).  The pages then combine p with a
  cumulative-mass test, which mixes a per-score statistic with a mass
  fraction; the reading taken here is the plain one: a row keeps every block
  whose score is at least p (for normally distributed scores, about k of the
  n blocks), and at least its largest block.  mean and std are over the
  row's nb scores, std the population deviation; U(1 - k/n) is passed in as
  the number u.  Scaling a row scales p alike, so the raw P_imp row gives the
  same set as the normalised one.

Rows holding a value outside [0, 1] or NaN keep every block, as in the
cumulative rule.  The statistical rule compares floats against a computed
threshold: rows where some score lies within 1e-12 (relative) of p are
reported as ties.
"""
from __future__ import annotations

import numpy as np


def _row_valid(row: np.ndarray) -> bool:
    r = np.asarray(row, dtype=np.float32)
    return bool(np.all(np.isfinite(r)) and np.all(r >= 0) and np.all(r <= 1))


def _order(row: np.ndarray):
    """Blocks by importance descending, then index ascending."""
    vals = np.asarray(row, dtype=np.float64)
    return sorted(range(vals.shape[0]), key=lambda J: (-vals[J], J))


def topk_row(row: np.ndarray, k: int):
    """Kept blocks (ascending) of one row under the top-k rule (k >= 1)."""
    row = np.asarray(row, dtype=np.float32)
    nb = row.shape[0]
    if not _row_valid(row):
        return list(range(nb))
    return sorted(_order(row)[:min(k, nb)])


def stat_threshold_row(row: np.ndarray, u: float):
    """(kept blocks ascending, tie flag) of one row under the statistical rule with quantile u."""
    row = np.asarray(row, dtype=np.float32)
    nb = row.shape[0]
    if not _row_valid(row):
        return list(range(nb)), False
    x = row.astype(np.float64)
    mean = x.sum() / nb
    std = np.sqrt(((x - mean) ** 2).sum() / nb)
    p = mean + std * u
    kept = {J for J in range(nb) if x[J] >= p}
    kept.add(_order(row)[0])
    tie = bool(np.any(np.abs(x - p) <= 1e-12 * max(1.0, abs(p))))
    return sorted(kept), tie


def build_mask_rule(p_imp: np.ndarray, rule: str, param: float):
    """P_imp [..., nb, nb] -> (kv_count, kv_idx (-1 padded), mask uint8, ties) for rule 'topk' (param = k)
    or 'stat' (param = u)."""
    p = np.asarray(p_imp, dtype=np.float32)
    lead = p.shape[:-1]
    nb = p.shape[-1]
    flat = p.reshape(-1, nb)
    cnt = np.zeros(flat.shape[0], dtype=np.int32)
    idx = np.full((flat.shape[0], nb), -1, dtype=np.int32)
    msk = np.zeros((flat.shape[0], nb), dtype=np.uint8)
    ties = []
    for r in range(flat.shape[0]):
        if rule == "topk":
            kept, tie = topk_row(flat[r], int(param)), False
        elif rule == "stat":
            kept, tie = stat_threshold_row(flat[r], float(param))
        else:
            raise ValueError(rule)
        cnt[r] = len(kept)
        idx[r, :len(kept)] = kept
        msk[r, kept] = 1
        if tie:
            ties.append(r)
    return cnt.reshape(lead), idx.reshape(lead + (nb,)), msk.reshape(lead + (nb,)), ties
