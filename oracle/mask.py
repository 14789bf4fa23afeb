"""Oracle: the cumulative-threshold block mask.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

*Video-BLADE*, "Step 2.1: Sparse mask construction" (BLADE notes, key design
1): each row of P_imp is sorted in descending order and the minimal number of
key blocks is kept whose cumulative score reaches the threshold (e.g. 90%).
The result is a binary mask M, one row per query block ("queries in the same
block share a mask", "A core design ... ASA").

Readings (the pages leave these open):
- the threshold is relative to the row total: keep the fewest blocks whose
  mass reaches tau * sum_J P_imp[I, J] (P_imp rows do not sum to 1; the BSA
  notes' greedy rule normalises the same way);
- "reaches" is >= (BSA's rule is ">= p"; "exceed" differs only at equality);
- ties in value are ordered by block index, ascending;
- the sums are exact: every float32 entry is an exact rational number, and
  the comparison prefix_m >= tau * total is decided in exact arithmetic, with
  tau taken as the float32 the library receives.  The decision is therefore
  independent of summation order;
- at least one block is kept; tau >= 1 keeps every block, zero-mass ones
  included (the dense limit);
- entries a softmax maximum cannot take (NaN, infinite, negative, or above 1)
  make the row keep every block.
Rows whose cut lies within 1e-6 * total of tau * total, or whose cut falls
between equal values, are reported as ties.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _row_valid(row: np.ndarray) -> bool:
    r = np.asarray(row, dtype=np.float32)
    return bool(np.all(np.isfinite(r)) and np.all(r >= 0) and np.all(r <= 1))


def build_mask_row(row: np.ndarray, tau: float):
    """Returns (kept block indices ascending, tie flag) for one P_imp row."""
    row = np.asarray(row, dtype=np.float32)
    nb = row.shape[0]
    t32 = np.float32(tau)
    if t32 >= 1 or not _row_valid(row):
        return list(range(nb)), False
    vals = [Fraction(float(x)) for x in row]      # exact (-0.0 becomes 0)
    total = sum(vals, Fraction(0))
    target = Fraction(float(t32)) * total
    order = sorted(range(nb), key=lambda J: (-vals[J], J))
    run = Fraction(0)
    m = nb
    prev = Fraction(0)
    for i, J in enumerate(order):
        prev = run
        run += vals[J]
        if run >= target:
            m = i + 1
            break
    kept = sorted(order[:m])
    eps = Fraction(1, 10 ** 6) * total
    tie = abs(run - target) < eps or (m > 1 and abs(prev - target) < eps)
    if m < nb and vals[order[m - 1]] == vals[order[m]]:
        tie = True
    return kept, bool(tie)


def build_mask(p_imp: np.ndarray, tau: float):
    """P_imp [..., nb, nb] float32 -> (kv_count [..., nb], kv_idx [..., nb, nb], mask uint8, ties).

    kv_idx rows hold the kept block indices ascending in their first kv_count
    entries and -1 after them; ties lists the flat row numbers flagged as ties.
    """
    p = np.asarray(p_imp, dtype=np.float32)
    lead = p.shape[:-1]
    nb = p.shape[-1]
    flat = p.reshape(-1, nb)
    cnt = np.zeros(flat.shape[0], dtype=np.int32)
    idx = np.full((flat.shape[0], nb), -1, dtype=np.int32)
    msk = np.zeros((flat.shape[0], nb), dtype=np.uint8)
    ties = []
    for r in range(flat.shape[0]):
        kept, tie = build_mask_row(flat[r], tau)
        cnt[r] = len(kept)
        idx[r, :len(kept)] = kept
        msk[r, kept] = 1
        if tie:
            ties.append(r)
    return cnt.reshape(lead), idx.reshape(lead + (nb,)), msk.reshape(lead + (nb,)), ties
