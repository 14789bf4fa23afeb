"""GPU parity: the backward of the block-sparse attention against the oracle's
float64 gradients, and the key-to-query lists against the oracle's (exact).

Tolerance of the gradients, entry by entry, from the arithmetic.  The GPU
takes bf16 inputs exactly and accumulates in fp32; it rounds three things to
bf16 (unit roundoff u = 2^-8): P before dV = P^T dO, dS before dQ = dS K and
dK = dS^T Q, and O (the forward's output) inside D_q = sum_j dO_qj O_qj.  To
first order the errors are then bounded by
    |dV_cj err| <= u * sum_q P_qc |dO_qj|
    |dQ_qj err| <= u * scale * sum_c (|dS_qc| + P_qc A_q) |K_cj|
    |dK_cj err| <= u * scale * sum_q (|dS_qc| + P_qc A_q) |Q_qj|
with A_q = sum_j |dO_qj| (|O_qj| + sum_c P_qc |V_cj|): the forward's O
carries its own rounding of P (u sum_c P_qc |V_cj|) and is then rounded to
bf16 (u |O_qj|), so the error of D_q is at most u A_q.  The
test allows twice these bounds (second-order terms, fp32 accumulation, the
hardware exp2), plus 1e-6 of the largest entry.  The magnitudes are computed
here in float64 from the same definition as the oracle; the reference values
themselves come from the oracle.
"""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import dev, dev_bf16, host, say, smooth_qkv
from oracle.attention_bwd import masked_attention_bwd, transpose_lists
from oracle.reorder import reorder_fast as o_reorder
from workloads.generator import bf16_round

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def _bounds(q, k, v, do, N, b, kept, scale):
    """Per-entry error bounds (see the module docstring) for one (batch, head)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64)[:N] for x in (q, k, v, do))
    nb = -(-N // b)
    key_block = np.arange(N) // b
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for I in range(nb):
        blocks = [J for J in set(kept[I]) if 0 <= J < nb]
        if not blocks:
            continue
        r0, r1 = I * b, min((I + 1) * b, N)
        allowed = np.isin(key_block, np.asarray(blocks, dtype=np.int64))
        s = (q[r0:r1] @ k.T) * scale
        s[:, ~allowed] = -np.inf
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v
        ds = np.abs(p * (do[r0:r1] @ v.T - (do[r0:r1] * o).sum(axis=1, keepdims=True)))
        A = (np.abs(do[r0:r1]) * (np.abs(o) + p @ np.abs(v))).sum(axis=1, keepdims=True)
        w = ds + p * A
        bv += p.T @ np.abs(do[r0:r1])
        bq[r0:r1] = scale * (w @ np.abs(k))
        bk += scale * (w.T @ np.abs(q[r0:r1]))
    return bq, bk, bv


def _check(name, got, ref, bound):
    tol = 2 * U * bound + 1e-6 * max(np.abs(ref).max(), 1e-30)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (name, int(bad.sum()), float(np.abs(got - ref).max()), float(tol[bad].min()))


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _lists(kind, nb, rng):
    out = []
    for I in range(nb):
        if kind == "all":
            out.append(list(range(nb)))
        elif kind == "single":
            out.append([(3 * I + 1) % nb])
        elif kind == "empty":
            out.append([] if I % 3 == 0 else sorted(rng.choice(nb, size=min(nb, 2), replace=False).tolist()))
        else:
            m = int(rng.integers(1, nb + 1))
            out.append(sorted(rng.choice(nb, size=m, replace=False).tolist()))
    return out


def _upload(rows, B, Hh, nb):
    cnt = np.zeros((B, Hh, nb), np.int32)
    idx = np.full((B, Hh, nb, nb), -7, np.int32)
    for r, row in enumerate(rows):
        bi, h = divmod(r, Hh)
        for I, js in enumerate(row):
            cnt[bi, h, I] = len(js)
            idx[bi, h, I, :len(js)] = js
    return cnt, idx


@pytest.mark.parametrize("nb,BH,seed", [(1, 1, 0), (5, 3, 1), (16, 2, 2), (33, 2, 3), (256, 2, 4)])
def test_transpose_lists_bit_exact(nb, BH, seed):
    say("transpose lists", nb, BH)
    rng = np.random.default_rng(seed)
    cnt = rng.integers(-2, nb + 3, size=(1, BH, nb)).astype(np.int32)
    idx = np.full((1, BH, nb, nb), -1, np.int32)
    for h in range(BH):
        for I in range(nb):
            c = min(max(int(cnt[0, h, I]), 0), nb)
            idx[0, h, I, :c] = np.sort(rng.choice(nb, size=c, replace=False))
            if c and rng.random() < 0.2:
                idx[0, h, I, int(rng.integers(0, c))] = nb + 9      # skipped
    tc, ti = _ops().transpose_lists(dev(cnt), dev(idx))
    torch.cuda.synchronize()
    tc, ti = host(tc), host(ti)
    for h in range(BH):
        rc, ri = transpose_lists(cnt[0, h], idx[0, h])
        assert np.array_equal(tc[0, h], rc)
        for J in range(nb):
            assert np.array_equal(ti[0, h, J, :rc[J]], ri[J, :rc[J]]), (h, J)


def _run_case(N, d, b, B, Hh, kind, seed, check_rows=None):
    ops = _ops()
    rng = np.random.default_rng(seed)
    q, k, v = smooth_qkv(seed, B, N, Hh, d)
    do = bf16_round(rng.standard_normal((B, N, Hh, d)).astype(np.float32))
    nb = -(-N // b)
    Npad = nb * b
    rows = [_lists(kind, nb, rng) for _ in range(B * Hh)]
    cnt, idx = _upload(rows, B, Hh, nb)
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_r = ops.reorder(dev_bf16(v), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    do_r = ops.reorder(dev_bf16(do), perm, Npad, b, "rows")
    scale = 1.0 / math.sqrt(d)
    o_r, lse = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, scale, dev(cnt), dev(idx), want_lse=True)
    dq, dk, dv = ops.sparse_attn_bwd(q_r, k_r, v_r, o_r, do_r, lse, N, b, scale, dev(cnt), dev(idx))
    torch.cuda.synchronize()
    dq, dk, dv = host(dq), host(dk), host(dv)
    for bi in range(B):
        for h in range(Hh):
            kept = rows[bi * Hh + h]
            args = (q[bi, :, h], k[bi, :, h], v[bi, :, h], do[bi, :, h], N, b, kept, scale)
            rq, rk, rv = masked_attention_bwd(*args)
            bq, bk, bv = _bounds(*args)
            for name, got, ref, bd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
                g = got[bi, h]
                assert (g[N:] == 0).all(), name
                _check(name, g[:N], ref, bd)


@pytest.mark.parametrize("N,d,b,B,Hh,kind", [
    (300, 64, 64, 1, 2, "random"), (1000, 128, 128, 2, 2, "random"), (777, 128, 64, 1, 3, "empty"),
    (130, 64, 128, 1, 1, "all"), (600, 128, 128, 1, 2, "single"), (1000, 64, 128, 1, 2, "empty"),
])
def test_bwd_small(N, d, b, B, Hh, kind):
    say("attn bwd", N, d, b, B, Hh, kind)
    _run_case(N, d, b, B, Hh, kind, N + d + b)


def test_bwd_deterministic():
    """Two runs give bit-identical gradients (no atomics in the gradient sums)."""
    ops = _ops()
    N, d, b = 1000, 128, 128
    q, k, v = smooth_qkv(5, 1, N, 2, d)
    rng = np.random.default_rng(5)
    do = bf16_round(rng.standard_normal(q.shape).astype(np.float32))
    nb = 8
    cnt, idx = _upload([_lists("random", nb, rng) for _ in range(2)], 1, 2, nb)
    perm = dev(np.arange(N, dtype=np.int32))
    rr = lambda x, lay="rows": ops.reorder(dev_bf16(x), perm, nb * b, b, lay)
    q_r, k_r, v_r, v_t, do_r = rr(q), rr(k), rr(v), rr(v, "tiles_t"), rr(do)
    o_r, lse = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, 0.09, dev(cnt), dev(idx), want_lse=True)
    a = ops.sparse_attn_bwd(q_r, k_r, v_r, o_r, do_r, lse, N, b, 0.09, dev(cnt), dev(idx))
    c = ops.sparse_attn_bwd(q_r, k_r, v_r, o_r, do_r, lse, N, b, 0.09, dev(cnt), dev(idx))
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x, y)


def test_bwd_full_wan_shape_sampled():
    """The Wan2.1-1.3B-shaped layer (12 heads, 32,760 tokens, b 128, k 16) with the mask the layer builds at
    tau 0.9; gradients compared on sampled key blocks (every query block that keeps them is included) and
    the query blocks involved."""
    from workloads import get_config, make_inputs
    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    cfg = get_config(2)
    say("attn bwd full", cfg.name)
    ops = _ops()
    q, k, v = make_inputs(cfg)
    rng = np.random.default_rng(11)
    do = bf16_round(rng.standard_normal(q.shape).astype(np.float32))
    layer = AsaLayer(LayerSpec(T=cfg.T, H=cfg.H, W=cfg.W, heads=cfg.heads, d=cfg.d, b=cfg.b, k=cfg.k, tau=0.9))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    layer.prepare(qd, kd, vd)
    layer.wait_kv()
    layer.mask(0.9)
    q_r = ops.reorder(qd, layer.perm, cfg.Npad, cfg.b, "rows")
    v_r = ops.reorder(vd, layer.perm, cfg.Npad, cfg.b, "rows")
    do_r = ops.reorder(dev_bf16(do), layer.perm, cfg.Npad, cfg.b, "rows")
    o_r, lse = ops.sparse_attn_fwd(q_r, layer.k_r, layer.v_t, cfg.N, cfg.b, cfg.scale, layer.kv_count,
                                   layer.kv_idx, want_lse=True)
    dq, dk, dv = ops.sparse_attn_bwd(q_r, layer.k_r, v_r, o_r, do_r, lse, cfg.N, cfg.b, cfg.scale,
                                     layer.kv_count, layer.kv_idx)
    torch.cuda.synchronize()
    perm = host(layer.perm)
    cnt, idx = host(layer.kv_count), host(layer.kv_idx)
    nb = cfg.nb
    for h, Js in ((0, [0, 131]), (7, [nb - 1])):
        qh, kh, vh, gh = (o_reorder(x[:, :, h:h + 1], perm, cfg.Npad)[0, 0] for x in (q, k, v, do))
        kept_all = [idx[0, h, I, :cnt[0, h, I]].tolist() for I in range(nb)]
        users = sorted({I for I in range(nb) for J in Js if J in kept_all[I]})
        kept = [kept_all[I] if I in users else [] for I in range(nb)]
        rq, rk, rv = masked_attention_bwd(qh, kh, vh, gh, cfg.N, cfg.b, kept, cfg.scale)
        bq, bk, bv = _bounds(qh, kh, vh, gh, cfg.N, cfg.b, kept, cfg.scale)
        rows_k = np.concatenate([np.arange(J * cfg.b, min((J + 1) * cfg.b, cfg.N)) for J in Js])
        rows_q = np.concatenate([np.arange(I * cfg.b, min((I + 1) * cfg.b, cfg.N)) for I in users])
        for name, got, ref, bd, rws in (("dk", host(dk[0, h]), rk, bk, rows_k), ("dv", host(dv[0, h]), rv, bv, rows_k),
                                        ("dq", host(dq[0, h]), rq, bq, rows_q)):
            _check(name, got[rws], ref[rws], bd[rws])
