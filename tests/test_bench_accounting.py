"""bench.py's byte count for the mask stage equals the sizes of the buffers dbs_build_mask reads
and writes (P_imp read once; kv_count, the kept entries of kv_idx and the optional work order
written), on a small mask with known kept counts."""
import numpy as np

import bench


def test_mask_stage_bytes_match_buffers():
    B, H, nb = 1, 3, 5
    cnt = np.array([[1, 2, 0, 5, 3], [4, 4, 4, 4, 4], [1, 1, 1, 1, 1]], dtype=np.int32)[None]
    p_imp = np.zeros((B, H, nb, nb), dtype=np.float32)
    kv_count = np.zeros((B, H, nb), dtype=np.int32)
    order = np.zeros((B * H * nb,), dtype=np.int32)
    kept_entries = np.zeros(int(cnt.sum()), dtype=np.int32)      # the written part of kv_idx
    base = p_imp.nbytes + kv_count.nbytes + kept_entries.nbytes
    assert bench.mask_stage_bytes(B * H, nb, float(cnt.sum()), with_order=False) == base
    assert bench.mask_stage_bytes(B * H, nb, float(cnt.sum()), with_order=True) == base + order.nbytes


def test_mask_stage_bytes_kept_counted_once():
    """The kept total already spans every head: doubling the heads at the same total adds only
    the P_imp, count and order bytes of the new heads."""
    a = bench.mask_stage_bytes(24, 1200, 1.728e6, with_order=False)
    b = bench.mask_stage_bytes(48, 1200, 1.728e6, with_order=False)
    assert b - a == 24 * 1200 * (4 * 1200 + 4)
    assert abs(a - (4 * 24 * 1200 * 1200 + 4 * 24 * 1200 + 4 * 1.728e6)) < 1
