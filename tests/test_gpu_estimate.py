"""GPU parity: estimate_blocks against the oracle's float64 estimator (relative
1e-3: the GPU multiplies bf16 inputs with fp32 accumulation)."""
import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, dev, dev_bf16, host, say, smooth_qkv
from oracle.estimator import p_imp as o_p_imp
from oracle.perm import perm_gilbert3d
from oracle.reorder import reorder_fast as o_reorder
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-3, 1e-7


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _run(q, k, N, b, kk, d, Hh, B=1, query_blocks=None):
    ops = _ops()
    Npad = -(-N // b) * b
    perm = np.arange(N, dtype=np.int32)
    q_r = ops.reorder(dev_bf16(q), dev(perm), Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), dev(perm), Npad, b, "rows")
    nb = Npad // b
    gp = Guarded((B, Hh, nb, nb), torch.float32)
    gw = Guarded((max(16, ops.estimate_workspace_bytes(B, Hh, N, d, b, kk)),), torch.uint8, fill=171)
    P = ops.estimate_blocks(q_r, k_r, N, b, kk, 1.0 / np.sqrt(d), p_imp=gp.view, workspace=gw.view)
    torch.cuda.synchronize()
    assert gp.intact() and gw.intact()          # nothing written outside P_imp or the workspace
    P = host(P)
    qr, kr = o_reorder(q, perm, Npad), o_reorder(k, perm, Npad)
    for bi in range(B):
        for h in range(Hh):
            ref = o_p_imp(qr[bi, h], kr[bi, h], N, b, kk, 1.0 / np.sqrt(d), query_blocks=query_blocks)
            rows = range(ref.shape[0]) if query_blocks is None else query_blocks
            for I in rows:
                np.testing.assert_allclose(P[bi, h, I], ref[I], rtol=RTOL, atol=ATOL,
                                           err_msg=f"b{bi} h{h} I{I}")
    return P


@pytest.mark.parametrize("N,b,k,d", [
    (200, 64, 8, 64), (1000, 64, 16, 128), (1000, 128, 16, 64), (777, 128, 16, 128),
    (300, 64, 1, 64), (300, 64, 2, 128), (300, 64, 4, 64), (520, 128, 32, 128),
    (520, 64, 64, 64), (400, 128, 128, 128), (130, 128, 128, 64), (2048, 64, 8, 64),
    # sample counts that are not powers of two (slots padded to the next one)
    (1000, 128, 12, 128), (700, 64, 6, 64), (333, 64, 3, 128), (900, 128, 24, 64), (500, 128, 100, 128),
    (260, 64, 48, 64), (130, 64, 5, 64), (1500, 128, 80, 128),
])
def test_estimate_small(N, b, k, d):
    say("estimate", N, b, k, d)
    q, kk, _ = smooth_qkv(N + k, 2, N, 2, d)
    _run(q, kk, N, b, k, d, Hh=2, B=2)


def test_estimate_k_equals_b_is_exact_blockmax():
    # k = b samples every token: the map must be the max-pooled dense softmax.
    N, b, d = 333, 64, 64
    say("estimate k=b", N, b, d)
    q, k, _ = smooth_qkv(5, 1, N, 1, d)
    P = _run(q, k, N, b, b, d, Hh=1)
    qq, kk = q[0, :, 0].astype(np.float64), k[0, :, 0].astype(np.float64)
    s = qq @ kk.T / np.sqrt(d)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    nb = -(-N // b)
    for I in range(nb):
        for J in range(nb):
            ref = p[I * b:(I + 1) * b, J * b:(J + 1) * b].max()
            assert abs(P[0, 0, I, J] - ref) <= RTOL * ref + ATOL


def test_estimate_wan_heads():
    """Two heads of the Wan2.1-1.3B layer at full length, all query blocks."""
    cfg = get_config(2)
    say("estimate wan", cfg.name)
    q, k, _ = make_inputs(cfg, heads=[0, 7])
    perm = perm_gilbert3d(cfg.T, cfg.H, cfg.W)
    ops = _ops()
    pt = dev(perm.astype(np.int32))
    q_r = ops.reorder(dev_bf16(q), pt, cfg.Npad, cfg.b, "rows")
    k_r = ops.reorder(dev_bf16(k), pt, cfg.Npad, cfg.b, "rows")
    P = host(ops.estimate_blocks(q_r, k_r, cfg.N, cfg.b, cfg.k, cfg.scale))
    qr, kr = o_reorder(q, perm, cfg.Npad), o_reorder(k, perm, cfg.Npad)
    for h in range(2):
        ref = o_p_imp(qr[0, h], kr[0, h], cfg.N, cfg.b, cfg.k, cfg.scale)
        np.testing.assert_allclose(P[0, h], ref, rtol=RTOL, atol=ATOL)


def test_estimate_deterministic():
    N, b, k, d = 1000, 128, 16, 128
    q, kk, _ = smooth_qkv(9, 1, N, 2, d)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), perm, 1024, b, "rows")
    k_r = ops.reorder(dev_bf16(kk), perm, 1024, b, "rows")
    a = host(ops.estimate_blocks(q_r, k_r, N, b, k, 0.088))
    c = host(ops.estimate_blocks(q_r, k_r, N, b, k, 0.088))
    assert np.array_equal(a, c)


@pytest.mark.parametrize("N,b,k,d,per_head,in32", [
    (1000, 128, 16, 128, False, False), (777, 64, 8, 64, True, False), (520, 128, 32, 128, True, True),
    (300, 64, 1, 64, False, True), (1000, 128, 12, 128, True, False), (333, 64, 7, 64, False, True),
])
def test_estimate_token_order_equals_reorder(N, b, k, d, per_head, in32):
    """estimate_blocks_tok (sampled Q rows gathered in token order) is
    bit-identical to estimate_blocks on the reordered Q."""
    say("estimate tok", N, b, k, d, per_head, in32)
    B, Hh = 2, 3
    rng = np.random.default_rng(N + k)
    q, kk, _ = smooth_qkv(N + 3, B, N, Hh, d)
    ops = _ops()
    Npad = -(-N // b) * b
    pm = (np.stack([rng.permutation(N) for _ in range(Hh)]) if per_head else rng.permutation(N)).astype(np.int32)
    perm = dev(pm)
    qd = dev(q) if in32 else dev_bf16(q)
    q_r = ops.reorder(qd, perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(kk), perm, Npad, b, "rows")
    a = host(ops.estimate_blocks(q_r, k_r, N, b, k, 1.0 / np.sqrt(d)))
    c = host(ops.estimate_blocks_tok(qd, perm, k_r, N, b, k, 1.0 / np.sqrt(d)))
    assert np.array_equal(a, c)
