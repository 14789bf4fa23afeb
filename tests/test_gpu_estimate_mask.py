"""GPU parity: the fused estimate-and-select calls (dbs_estimate_mask,
dbs_estimate_mask_tok) against the oracle, and against the two-launch path
they replace (dbs_estimate_blocks then dbs_build_mask_rule), bit for bit.

The fused kernels form each P_imp row on chip with the same arithmetic as the
estimator's final launch and hand it to the same selection code, so P_imp (when
written), kv_count, the kept lists and the mask must equal the two-launch
path's exactly; the oracle's float64 estimator checks P_imp (relative 1e-3, the
estimator's bar) and the oracle's exact mask builder checks the selection on
the GPU's own P_imp, as for dbs_build_mask."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, dev_bf16, host, say, smooth_qkv
from oracle.estimator import p_imp as o_p_imp
from oracle.mask import build_mask as o_build_mask
from oracle.mask_rules import build_mask_rule as o_rule
from oracle.perm import perm_gilbert3d
from oracle.reorder import reorder_fast as o_reorder

pytestmark = pytest.mark.gpu


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _same_lists(a, b, nb):
    """(kv_count, kv_idx, mask) of two calls: counts, the kept prefix of each list and masks equal
    (list entries past a count are unspecified)."""
    ca, ia, ma = (host(x) for x in a)
    cb, ib, mb = (host(x) for x in b)
    assert np.array_equal(ca, cb)
    assert np.array_equal(ma, mb)
    ca, ia, ib = ca.reshape(-1), ia.reshape(-1, nb), ib.reshape(-1, nb)
    for r in range(ca.shape[0]):
        assert np.array_equal(ia[r, :ca[r]], ib[r, :ca[r]]), r


def _inputs(seed, N, Hh, d, B=1):
    q, k, _ = smooth_qkv(seed, B, N, Hh, d)
    return q, k


@pytest.mark.parametrize("N,b,kk,d,Hh", [
    (1000, 64, 8, 64, 2),        # nb 16, ragged last block (KPL 1 rows)
    (6000, 64, 16, 128, 1),      # nb 94 (KPL 2), ragged
    (16384, 64, 4, 64, 1),       # nb 256 (KPL 4)
    (16400, 64, 64, 64, 1),      # nb 257: the radix selection (KPL 8), k = b
    (70000, 64, 2, 64, 1),       # nb 1094: the radix selection (KPL 20)
    (2300, 128, 128, 128, 1),    # k = 128: two 64-key cells per block
    (3000, 128, 12, 128, 2),     # k = 12: slots padded to 16
    (40000, 128, 20, 64, 1),     # nb 313 (radix, KPL 8), k = 20: slots padded to 32
    (95990, 64, 4, 64, 1),       # nb 1500 (radix, KPL 32), ragged
    (262139, 64, 2, 64, 1),      # nb 4096, the largest row (radix, KPL 64), ragged
])
@pytest.mark.parametrize("rule,param", [("cumulative", 0.9), ("topk", 5), ("stat", 1.0)])
def test_fused_equals_two_launches_and_oracle(N, b, kk, d, Hh, rule, param):
    say("estimate_mask", N, b, kk, d, Hh, rule, param)
    ops = _ops()
    q, k = _inputs(N + kk, N, Hh, d)
    Npad = -(-N // b) * b
    nb = Npad // b
    scale = 1.0 / np.sqrt(d)
    ident = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), ident, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), ident, Npad, b, "rows")
    P = ops.estimate_blocks(q_r, k_r, N, b, kk, scale)
    two = ops.build_mask_rule(P, rule, param, want_mask=True)
    c, i, m, Pf = ops.estimate_mask(q_r, k_r, N, b, kk, scale, rule, param, want_p_imp=True, want_mask=True)
    c2, i2, m2, none = ops.estimate_mask(q_r, k_r, N, b, kk, scale, rule, param, want_mask=True)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(P, Pf)
    _same_lists(two, (c, i, m), nb)
    _same_lists((c, i, m), (c2, i2, m2), nb)

    # the oracle: P_imp on a few query blocks, the selection on every row of the GPU's P_imp
    Ph = host(Pf)
    qr, kr = o_reorder(q, np.arange(N), Npad), o_reorder(k, np.arange(N), Npad)
    rng = np.random.default_rng(N)
    blocks = sorted({0, nb - 1} | set(rng.choice(nb, min(nb, 6), replace=False).tolist()))
    ref = o_p_imp(qr[0, 0], kr[0, 0], N, b, kk, scale, query_blocks=blocks)
    for I in blocks:
        np.testing.assert_allclose(Ph[0, 0, I], ref[I], rtol=1e-3, atol=1e-7, err_msg=f"I{I}")
    rows = Ph.reshape(-1, nb)
    sel = sorted(set(rng.choice(rows.shape[0], min(rows.shape[0], 64), replace=False).tolist()) | {0})
    if rule == "cumulative":
        rc, ri, rm, _ = o_build_mask(rows[sel], param)
        ties = set()
    else:
        rc, ri, rm, t = o_rule(rows[sel], rule, param)
        ties = set(t)
    hc, hi, hm = host(c).reshape(-1), host(i).reshape(-1, nb), host(m).reshape(-1, nb)
    for j, r in enumerate(sel):
        if j in ties:
            continue
        assert hc[r] == rc[j], r
        assert np.array_equal(hi[r, :rc[j]], ri[j, :rc[j]]), r
        assert np.array_equal(hm[r], rm[j]), r


def test_token_order_and_work_order():
    """dbs_estimate_mask_tok on a Gilbert-ordered 3D grid: equal to dbs_estimate_blocks_tok +
    dbs_build_mask, and the work order is a permutation that lists each XCD range's rows by kept
    count descending, as dbs_build_mask's."""
    say("estimate_mask_tok")
    ops = _ops()
    T, H, W, Hh, d, b, kk = 5, 12, 20, 3, 128, 64, 16
    N = T * H * W
    q, k, _ = smooth_qkv(11, 1, N, Hh, d, grid=(T, H, W))
    perm = dev(perm_gilbert3d(T, H, W).astype(np.int32))
    Npad = -(-N // b) * b
    nb = Npad // b
    scale = 1.0 / np.sqrt(d)
    qd = dev_bf16(q)
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    P = ops.estimate_blocks_tok(qd, perm, k_r, N, b, kk, scale)
    two = ops.build_mask(P, 0.9, want_mask=True, want_order=True)
    order = torch.empty(Hh * nb, dtype=torch.int32, device="cuda")
    c, i, m, Pf = ops.estimate_mask(qd, k_r, N, b, kk, scale, "cumulative", 0.9, q_perm=perm, want_p_imp=True,
                                    want_mask=True, order=order)
    torch.cuda.synchronize()
    assert torch.equal(P, Pf)
    _same_lists(two[:3], (c, i, m), nb)
    o1, o2 = host(two[3]), host(order)
    assert sorted(o2.tolist()) == list(range(Hh * nb))
    cnt = host(c).reshape(-1)
    assert np.array_equal(np.sort(cnt[o1]), np.sort(cnt[o2]))
    rows = Hh * nb
    starts = [(rows // 8) * x + min(x, rows % 8) for x in range(9)]
    for x in range(8):
        seg = cnt[o2[starts[x]:starts[x + 1]]]
        assert (np.diff(seg) <= 0).all(), x
        assert sorted(o2[starts[x]:starts[x + 1]].tolist()) == list(range(starts[x], starts[x + 1]))


def test_wan_shape_fused_equals_two_launches():
    """The Wan2.1-1.3B-shaped layer (12 heads, 32,760 tokens, b 128, k 16), Q in token order: every
    row equal to the two-launch path, for the three rules."""
    say("estimate_mask wan")
    from workloads import get_config, make_inputs
    ops = _ops()
    cfg = get_config(2)
    T, H, W = cfg.T, cfg.H, cfg.W
    N, Hh, d, b, kk = T * H * W, cfg.heads, cfg.d, cfg.b, cfg.k
    qn, kn, _ = make_inputs(cfg)
    permd = dev(perm_gilbert3d(T, H, W).astype(np.int32))
    Npad = -(-N // b) * b
    nb = Npad // b
    scale = 1.0 / np.sqrt(d)
    qd = dev_bf16(qn)
    k_r = ops.reorder(dev_bf16(kn), permd, Npad, b, "rows")
    P = ops.estimate_blocks_tok(qd, permd, k_r, N, b, kk, scale)
    for rule, param in (("cumulative", 0.9), ("topk", 16), ("stat", ops.stat_quantile(16, nb))):
        two = ops.build_mask_rule(P, rule, param, want_mask=True)
        got = ops.estimate_mask(qd, k_r, N, b, kk, scale, rule, param, q_perm=permd, want_mask=True)
        torch.cuda.synchronize()
        _same_lists(two, got[:3], nb)


@pytest.mark.parametrize("case", ["gilbert_bf16", "per_head_k12_ragged", "f32_d64_b128", "packed_qkv_view", "batch2"])
def test_kvtok_equals_reordered_k(case):
    """dbs_estimate_mask_kvtok (K read in token order, its sampled rows gathered into the workspace)
    against dbs_estimate_mask_tok on dbs_reorder's K rows: P_imp, kv_count, the kept lists, the mask
    and the work order equal bit for bit."""
    say("estimate_mask_kvtok", case)
    from oracle.perm import perm_cuboid
    ops = _ops()
    T, H, W, Hh, d, b, kk = 5, 12, 20, 3, 128, 64, 16
    f32 = False
    if case == "per_head_k12_ragged":
        T, H, W, kk = 5, 11, 19, 12
    elif case == "f32_d64_b128":
        d, b, f32 = 64, 128, True
    N = T * H * W
    Bt = 2 if case == "batch2" else 1
    q, k, _ = smooth_qkv(23, Bt, N, Hh, d, grid=(T, H, W))
    if case == "per_head_k12_ragged":
        perm_h = np.stack([perm_gilbert3d(T, H, W), perm_cuboid(T, H, W, 2, 4, 4), perm_cuboid(T, H, W, 1, 2, 8)])
        perm = dev(perm_h.astype(np.int32))
    else:
        perm = dev(perm_gilbert3d(T, H, W).astype(np.int32))
    if f32:   # values off the bf16 grid, so the gather's rounding is exercised
        rng = np.random.default_rng(4)
        qd = dev((q * (1 + rng.uniform(-1e-3, 1e-3, q.shape))).astype(np.float32))
        kd = dev((k * (1 + rng.uniform(-1e-3, 1e-3, k.shape))).astype(np.float32))
    elif case == "packed_qkv_view":   # K a strided view of a packed [B, N, Hh, 3, d] tensor
        qkv = torch.zeros((Bt, N, Hh, 3, d), dtype=torch.bfloat16, device="cuda")
        qkv[:, :, :, 0] = dev_bf16(q)
        qkv[:, :, :, 1] = dev_bf16(k)
        qd, kd = qkv[:, :, :, 0], qkv[:, :, :, 1]
        assert not kd.is_contiguous()
    else:
        qd, kd = dev_bf16(q), dev_bf16(k)
    Npad = -(-N // b) * b
    nb = Npad // b
    scale = 1.0 / np.sqrt(d)
    k_r = ops.reorder(kd, perm, Npad, b, "rows")
    o1 = torch.empty(Bt * Hh * nb, dtype=torch.int32, device="cuda")
    o2 = torch.empty(Bt * Hh * nb, dtype=torch.int32, device="cuda")
    ref = ops.estimate_mask(qd, k_r, N, b, kk, scale, "cumulative", 0.9, q_perm=perm, want_p_imp=True,
                            want_mask=True, order=o1)
    got = ops.estimate_mask_kvtok(qd, kd, perm, b, kk, scale, "cumulative", 0.9, want_p_imp=True, want_mask=True,
                                  order=o2)
    torch.cuda.synchronize()
    assert torch.equal(ref[3], got[3])
    _same_lists(ref[:3], got[:3], nb)
    # the work orders: permutations with the same counts along them (equal counts in any order)
    cnt = host(got[0]).reshape(-1)
    assert sorted(host(o2).tolist()) == list(range(Bt * Hh * nb))
    assert np.array_equal(cnt[host(o1)], cnt[host(o2)])
