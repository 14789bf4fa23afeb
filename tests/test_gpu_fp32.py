"""GPU parity for the float32 operand path (workloads stored in float32:
estimate and attention computed in float32 throughout), against the oracle's
float64 arithmetic on the same float32 values.

Tolerances come from float32 rounding.  A dot product of D terms is off by at
most gamma_D * sum_i |q_i k_i| (gamma_D = D u / (1 - D u), u = 2^-24), so a
score is off by at most eps_s = gamma_D * scale * max sum_i |q_i k_i|.
- P_imp = exp(t - lse): both exponents carry eps_s, and the normaliser sums
  N_s terms: relative error <= 2 eps_s + (N_s + 8) u.
- The output is a softmax-weighted mean of V rows: weights move by a factor
  within exp(+-2 eps_s), so the output moves by at most 2 eps_s max|v| (first
  order; 2.5 eps_s allowed), plus the float32 sum over L keys, (L + 8) u
  max|v|.
Outputs are written into buffers with canary regions on both sides, and the
canaries are checked."""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, dev, host, say
from oracle.attention import masked_attention
from oracle.estimator import p_imp as o_p_imp, sample_rows
from oracle.mask import build_mask as o_build_mask

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _eps(qs, ks, scale):
    D = qs.shape[1]
    g = D * U / (1 - D * U)
    return g * scale * float((np.abs(qs) @ np.abs(ks).T).max())


def _qkv(seed, B, N, Hh, d):
    """Float32 smooth-field Q/K and iid V, not rounded to bf16."""
    from workloads.generator import make_head
    q = np.empty((B, N, Hh, d), np.float32)
    k, v = np.empty_like(q), np.empty_like(q)
    for bi in range(B):
        for h in range(Hh):
            qq, kk, vv = make_head(2000 + seed, bi * 64 + h, (1, 1, N), d, (2.0, 2.0, 2.0))
            q[bi, :, h], k[bi, :, h], v[bi, :, h] = qq, kk, vv
    return q, k, v


EST_CASES = [  # N, d, b, k
    (2048, 64, 64, 8), (1000, 128, 128, 16), (777, 64, 64, 7), (300, 128, 128, 128), (130, 64, 64, 1),
    (2100, 128, 64, 12),
]


@pytest.mark.parametrize("N,d,b,k", EST_CASES)
def test_estimate_f32(N, d, b, k):
    say("estimate f32", N, d, b, k)
    ops = _ops()
    B, Hh = 1, 2
    q, k_, _ = _qkv(N + k, B, N, Hh, d)
    nb = -(-N // b)
    Npad = nb * b
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev(q), perm, Npad, b, "rows", out_dtype=torch.float32)
    k_r = ops.reorder(dev(k_), perm, Npad, b, "rows", out_dtype=torch.float32)
    scale = 1.0 / math.sqrt(d)
    g = Guarded((B, Hh, nb, nb), torch.float32)
    ops.estimate_blocks(q_r, k_r, N, b, k, scale, p_imp=g.view)
    torch.cuda.synchronize()
    assert g.intact(), "P_imp canaries overwritten"
    P = host(g.view)
    sr = np.concatenate(sample_rows(N, b, k))
    for h in range(Hh):
        ref = o_p_imp(q[0, :, h], k_[0, :, h], N, b, k, scale)
        rtol = 2 * _eps(q[0, sr, h], k_[0, sr, h], scale) + (len(sr) + 8) * U
        np.testing.assert_allclose(P[0, h], ref, rtol=rtol, atol=1e-37)


@pytest.mark.parametrize("N,d,b", [(2048, 64, 64), (1000, 128, 128), (777, 128, 64), (337, 64, 128)])
@pytest.mark.parametrize("kind", ["random", "all", "empty"])
def test_attn_f32(N, d, b, kind):
    say("attn f32", N, d, b, kind)
    ops = _ops()
    B, Hh = 1, 2
    rng = np.random.default_rng(N + d + b + len(kind))
    q, k, v = _qkv(N + d, B, N, Hh, d)
    nb = -(-N // b)
    Npad = nb * b
    lists = []
    for _ in range(B * Hh):
        row = []
        for I in range(nb):
            if kind == "all":
                row.append(list(range(nb)))
            elif kind == "empty" and I % 3 == 0:
                row.append([])
            else:
                m = int(rng.integers(1, nb + 1))
                row.append(sorted(rng.choice(nb, size=m, replace=False).tolist()))
        lists.append(row)
    cnt = np.zeros((B, Hh, nb), np.int32)
    idx = np.full((B, Hh, nb, nb), -1, np.int32)
    for r, row in enumerate(lists):
        for I, js in enumerate(row):
            cnt[0, r, I] = len(js)
            idx[0, r, I, :len(js)] = js
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev(q), perm, Npad, b, "rows", out_dtype=torch.float32)
    k_r = ops.reorder(dev(k), perm, Npad, b, "rows", out_dtype=torch.float32)
    v_r = ops.reorder(dev(v), perm, Npad, b, "rows", out_dtype=torch.float32)
    scale = 1.0 / math.sqrt(d)
    go = Guarded((B, Hh, Npad, d), torch.float32)
    gl = Guarded((B, Hh, Npad), torch.float32)
    # a work order (reversed rows) gives the same result
    order = dev(np.arange(B * Hh * nb, dtype=np.int32)[::-1].copy())
    ops.sparse_attn_fwd(q_r, k_r, v_r, N, b, scale, dev(cnt), dev(idx), o_r=go.view, lse=gl.view, order=order)
    torch.cuda.synchronize()
    assert go.intact() and gl.intact(), "canaries overwritten"
    o, l = host(go.view), host(gl.view)
    for h in range(Hh):
        ref, rl = masked_attention(q[0, :, h], k[0, :, h], v[0, :, h], N, b, lists[h], scale)
        for I in range(nb):
            rows = np.arange(I * b, min((I + 1) * b, N))
            if not lists[h][I]:
                assert (o[0, h, rows] == 0).all() and np.isneginf(l[0, h, rows]).all()
                continue
            keys = np.concatenate([np.arange(J * b, min((J + 1) * b, N)) for J in lists[h][I]])
            eps = _eps(q[0, rows, h], k[0, keys, h], scale)
            vmax = float(np.abs(v[0, keys, h]).max())
            tol = 2.5 * eps * vmax + (len(keys) + 8) * U * vmax
            err = np.abs(o[0, h, rows] - ref[rows]).max()
            assert err <= tol, (h, I, err, tol)
            # lse: the log of the normaliser carries eps_s plus the sum's rounding
            assert np.abs(l[0, h, rows] - rl[rows]).max() <= eps + (len(keys) + 8) * U + 1e-6


def test_f32_layer_matches_reordered_calls_and_rejects_global_tokens():
    """The float32 estimate_mask equals estimate + build_mask bit for bit; the float32
    inverse reorder is an exact copy; global tokens are refused on the float32 path."""
    say("f32 layer pieces")
    ops = _ops()
    N, d, b, k = 2048, 64, 64, 8
    q, k_, v = _qkv(7, 1, N, 1, d)
    nb = N // b
    rng = np.random.default_rng(0)
    pm = rng.permutation(N).astype(np.int32)
    perm = dev(pm)
    q_r = ops.reorder(dev(q), perm, N, b, "rows", out_dtype=torch.float32)
    k_r = ops.reorder(dev(k_), perm, N, b, "rows", out_dtype=torch.float32)
    v_r = ops.reorder(dev(v), perm, N, b, "rows", out_dtype=torch.float32)
    assert np.array_equal(host(q_r)[0, 0], q[0, pm, 0])
    scale = 1.0 / math.sqrt(d)
    P = ops.estimate_blocks(q_r, k_r, N, b, k, scale)
    c1, i1, _ = ops.build_mask(P, 0.9)
    c2, i2, _, P2 = ops.estimate_mask(q_r, k_r, N, b, k, scale, "cumulative", 0.9, want_p_imp=True)
    c3, i3, _, _ = ops.estimate_mask(q_r, k_r, N, b, k, scale, "cumulative", 0.9)   # P_imp in the workspace
    torch.cuda.synchronize()
    assert torch.equal(P, P2) and torch.equal(c1, c2) and torch.equal(c1, c3)
    cc = host(c1)
    for I in range(nb):
        m = int(cc[0, 0, I])
        assert np.array_equal(host(i1)[0, 0, I, :m], host(i2)[0, 0, I, :m])
        assert np.array_equal(host(i1)[0, 0, I, :m], host(i3)[0, 0, I, :m])
    # the oracle's mask on the GPU's P_imp
    rc, ri, _, _ = o_build_mask(host(P)[0, 0], 0.9)
    assert np.array_equal(rc, cc[0, 0])
    o_r, _ = ops.sparse_attn_fwd(q_r, k_r, v_r, N, b, scale, c1, i1)
    out = ops.inverse_reorder(o_r, perm, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(out)[0, pm, 0], host(o_r)[0, 0, :N])
    kg = torch.zeros((1, 1, 64, d), dtype=torch.float32, device="cuda")
    with pytest.raises(Exception):
        ops.sparse_attn_fwd(q_r, k_r, v_r, N, b, scale, c1, i1, kg, kg, 256, 8)
