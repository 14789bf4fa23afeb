"""Pins for the oracle's block-masked attention and ASA_G (Video-BLADE, "Step 2.2").

Reference values come from routines the oracle does not use: torch's
scaled_dot_product_attention in float64 on the CPU, and scipy's softmax.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

from oracle.attention import global_bias, masked_attention, meanpool
from oracle.estimator import p_imp
from oracle.mask import build_mask


def _sdpa(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)[0, 0].numpy()


def _rand(N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((N, d)) for _ in range(3)]


@pytest.mark.parametrize("N,b", [(64, 16), (45, 16), (100, 32)])
def test_all_blocks_kept_is_dense(N, b):
    q, k, v = _rand(N, 8, N)
    nb = -(-N // b)
    out, lse = masked_attention(q, k, v, N, b, [list(range(nb))] * nb, 1 / math.sqrt(8))
    np.testing.assert_allclose(out, _sdpa(q, k, v, 1 / math.sqrt(8)), rtol=1e-10, atol=1e-12)
    s = (q @ k.T) / math.sqrt(8)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(1)), rtol=1e-12)


def test_tau_one_mask_gives_dense():
    N, b, d = 96, 16, 8
    q, k, v = _rand(N, d, 3)
    P = p_imp(q, k, N, b, 4, 1 / math.sqrt(d)).astype(np.float32)
    cnt, idx, _, _ = build_mask(P, 1.0)
    kept = [idx[I, :cnt[I]].tolist() for I in range(len(cnt))]
    out, _ = masked_attention(q, k, v, N, b, kept, 1 / math.sqrt(d))
    np.testing.assert_allclose(out, _sdpa(q, k, v, 1 / math.sqrt(d)), rtol=1e-10, atol=1e-12)


def test_single_block_mask_restricts_to_that_block():
    N, b, d = 80, 16, 8
    q, k, v = _rand(N, d, 4)
    nb = N // b
    kept = [[(3 * I + 1) % nb] for I in range(nb)]
    out, _ = masked_attention(q, k, v, N, b, kept, 0.3)
    for I in range(nb):
        J = kept[I][0]
        ref = _sdpa(q[I * b:(I + 1) * b], k[J * b:(J + 1) * b], v[J * b:(J + 1) * b], 0.3)
        np.testing.assert_allclose(out[I * b:(I + 1) * b], ref, rtol=1e-10, atol=1e-12)


def test_padding_keys_ignored():
    N, b, d = 45, 16, 4
    q, k, v = _rand(48, d, 5)
    nb = 3
    kept = [[0, 2], [1, 2], [2]]
    o1, _ = masked_attention(q, k, v, N, b, kept, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[N:] = 1e3
    v2[N:] = 1e3
    o2, _ = masked_attention(q, k2, v2, N, b, kept, 0.5)
    np.testing.assert_array_equal(o1, o2)
    # the kept part of block 2 is tokens 32..44 only
    ref = _sdpa(q[32:45], k[32:45], v[32:45], 0.5)
    np.testing.assert_allclose(o1[32:45], ref, rtol=1e-10, atol=1e-12)


def test_asa_g_n1_all_kept_is_dense():
    # Each global token duplicates one key with bias ln 1 = 0: every weight
    # doubles, the softmax is unchanged.
    N, b, d = 64, 16, 8
    q, k, v = _rand(N, d, 6)
    nb = N // b
    kg, vg = meanpool(k, N, 1), meanpool(v, N, 1)
    out, _ = masked_attention(q, k, v, N, b, [list(range(nb))] * nb, 0.35, kg, vg, global_bias(N, 1))
    np.testing.assert_allclose(out, _sdpa(q, k, v, 0.35), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("N,n", [(13, 4), (64, 8), (50, 8)])
def test_ln_n_bias_makes_global_tokens_stand_for_their_window(N, n):
    # K and V constant over each pooling window: attention over the global
    # region alone (empty mask) with bias ln r_g equals dense attention over
    # all tokens, the equivalence the bias is introduced for.  Without the
    # bias it differs whenever window sizes differ.
    rng = np.random.default_rng(N + n)
    d, b = 6, 16
    Ng = -(-N // n)
    kw, vw = rng.standard_normal((Ng, d)), rng.standard_normal((Ng, d))
    k = np.repeat(kw, n, axis=0)[:N]
    v = np.repeat(vw, n, axis=0)[:N]
    q = rng.standard_normal((N, d))
    kg, vg = meanpool(k, N, n), meanpool(v, N, n)
    np.testing.assert_allclose(kg, kw, rtol=1e-12)
    nb = -(-N // b)
    out, _ = masked_attention(q, k, v, N, b, [[]] * nb, 0.4, kg, vg, global_bias(N, n))
    np.testing.assert_allclose(out, _sdpa(q, k, v, 0.4), rtol=1e-10, atol=1e-12)
    if N % n:
        nob, _ = masked_attention(q, k, v, N, b, [[]] * nb, 0.4, kg, vg, np.zeros(Ng))
        assert np.abs(nob - out).max() > 1e-3


def test_global_bias_values():
    np.testing.assert_allclose(global_bias(17776, 8), np.full(2222, math.log(8)))
    gb = global_bias(13, 4)
    np.testing.assert_allclose(gb, [math.log(4)] * 3 + [0.0])


def test_meanpool_windows():
    x = np.arange(20, dtype=np.float64).reshape(10, 2)
    g = meanpool(x, 10, 4)
    np.testing.assert_allclose(g, [[3, 4], [11, 12], [17, 18]])
    np.testing.assert_allclose(meanpool(x, 7, 4)[-1], x[4:7].mean(0))


def test_asa_g_masked_matches_scipy_softmax():
    N, b, d, n = 40, 8, 4, 8
    q, k, v = _rand(N, d, 9)
    kept = [[0, 3], [1], [2, 4], [0, 1, 2, 3, 4], [4]]
    kg, vg = meanpool(k, N, n), meanpool(v, N, n)
    gb = global_bias(N, n)
    out, _ = masked_attention(q, k, v, N, b, kept, 0.5, kg, vg, gb)
    for I in range(5):
        cols = np.concatenate([np.arange(J * b, (J + 1) * b) for J in kept[I]])
        s = np.concatenate([q[I * b:(I + 1) * b] @ k[cols].T * 0.5,
                            q[I * b:(I + 1) * b] @ kg.T * 0.5 + gb], axis=1)
        w = softmax(s, axis=1)
        ref = w @ np.concatenate([v[cols], vg])
        np.testing.assert_allclose(out[I * b:(I + 1) * b], ref, rtol=1e-10, atol=1e-12)
