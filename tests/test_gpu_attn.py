"""GPU parity: sparse_attn_fwd against the oracle's block-masked float64
attention, max-abs 2e-2 (bf16 inputs, fp32 accumulation, P rounded to bf16),
for explicit KV-block lists, partial blocks, empty rows, malformed indices and
the ASA_G global tokens."""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import dev, dev_bf16, host, say, smooth_qkv, tiles_to_rows
from oracle.attention import global_bias, masked_attention
from oracle.reorder import reorder_fast as o_reorder

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _lists(kind, rows, nb, rng):
    out = []
    for r in range(rows):
        row = []
        for I in range(nb):
            if kind == "all":
                row.append(list(range(nb)))
            elif kind == "single":
                row.append([(3 * I + r) % nb])
            elif kind == "empty":
                row.append([] if I % 3 == 0 else sorted(rng.choice(nb, size=min(nb, 2), replace=False).tolist()))
            else:
                m = int(rng.integers(1, nb + 1))
                row.append(sorted(rng.choice(nb, size=m, replace=False).tolist()))
        out.append(row)
    return out


def _upload(lists, B, Hh, nb, bad=False, rng=None):
    cnt = np.zeros((B, Hh, nb), np.int32)
    idx = np.full((B, Hh, nb, nb), -7, np.int32)
    for r, row in enumerate(lists):
        bi, h = divmod(r, Hh)
        for I, js in enumerate(row):
            cnt[bi, h, I] = len(js)
            idx[bi, h, I, :len(js)] = js
    if bad:   # malformed entries must be skipped, not read
        for bi in range(B):
            for h in range(Hh):
                I = int(rng.integers(0, nb))
                if cnt[bi, h, I] < nb:
                    idx[bi, h, I, cnt[bi, h, I]] = 10 ** 6
                    cnt[bi, h, I] += 1
                cnt[bi, h, (I + 1) % nb] = -5 if nb > 1 else cnt[bi, h, 0]
    return cnt, idx


CASES = [  # N, d, b
    (2048, 64, 64), (1000, 128, 128), (777, 128, 64), (700, 64, 128), (128, 128, 128), (337, 64, 64),
]


@pytest.mark.parametrize("N,d,b", CASES)
@pytest.mark.parametrize("kind", ["random", "all", "single", "empty"])
def test_attn_lists(N, d, b, kind):
    say("attn", N, d, b, kind)
    B, Hh = 2, 2
    rng = np.random.default_rng(N + d + b + len(kind))
    q, k, v = smooth_qkv(N + d, B, N, Hh, d)
    nb = -(-N // b)
    Npad = nb * b
    lists = _lists(kind, B * Hh, nb, rng)
    cnt, idx = _upload(lists, B, Hh, nb)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    scale = 1.0 / math.sqrt(d)
    o_r, lse = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, scale, dev(cnt), dev(idx), want_lse=True)
    torch.cuda.synchronize()
    o, l = host(o_r), host(lse)
    for bi in range(B):
        for h in range(Hh):
            ref, rl = masked_attention(q[bi, :, h], k[bi, :, h], v[bi, :, h], N, b, lists[bi * Hh + h], scale)
            got = o[bi, h, :N]
            empty = np.repeat([len(js) == 0 for js in lists[bi * Hh + h]], b)[:N]
            if (~empty).any():
                assert np.abs(got[~empty] - ref[~empty]).max() <= TOL
                assert np.abs(l[bi, h, :N][~empty] - rl[~empty]).max() <= 1e-3
            assert (got[empty] == 0).all()
            assert np.isneginf(l[bi, h, :N][empty]).all()


def test_attn_max_nb():
    """The largest list the kernel takes (nb = 4096 blocks, every entry of the LDS list used):
    short random lists for most query blocks, every block for two of them, a ragged last block;
    sampled query blocks against the oracle."""
    say("attn max nb")
    b, d = 64, 64
    nb = 4096
    N = nb * b - 9
    rng = np.random.default_rng(4096)
    q, k, v = smooth_qkv(11, 1, N, 1, d)
    lists = [[sorted(rng.choice(nb, size=int(rng.integers(1, 9)), replace=False).tolist()) for _ in range(nb)]]
    full = [5, nb - 1]
    for I in full:
        lists[0][I] = list(range(nb))
    lists[0][7] = []
    cnt, idx = _upload(lists, 1, 1, nb)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    Npad = nb * b
    q_r = ops.reorder(dev_bf16(q), perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    scale = 1.0 / math.sqrt(d)
    o_r, lse = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, scale, dev(cnt), dev(idx), want_lse=True)
    torch.cuda.synchronize()
    o, l = host(o_r), host(lse)
    blocks = sorted(set(full + [0, 7, 1000, 2047, 3333]))
    ref, rl = masked_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], N, b, lists[0], scale, query_blocks=blocks)
    for I in blocks:
        rows = np.arange(I * b, min((I + 1) * b, N))
        if not lists[0][I]:
            assert (o[0, 0, rows] == 0).all() and np.isneginf(l[0, 0, rows]).all()
            continue
        assert np.abs(o[0, 0, rows] - ref[rows]).max() <= TOL, I
        assert np.abs(l[0, 0, rows] - rl[rows]).max() <= 1e-3, I


def test_attn_malformed_lists_are_skipped():
    say("attn malformed")
    N, d, b, B, Hh = 600, 128, 128, 1, 3
    rng = np.random.default_rng(2)
    q, k, v = smooth_qkv(3, B, N, Hh, d)
    nb = -(-N // b)
    lists = _lists("random", B * Hh, nb, rng)
    cnt, idx = _upload(lists, B, Hh, nb, bad=True, rng=rng)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    Npad = nb * b
    q_r = ops.reorder(dev_bf16(q), perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    o_r, _ = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, 1 / math.sqrt(d), dev(cnt), dev(idx))
    torch.cuda.synchronize()
    o = host(o_r)
    for h in range(Hh):
        eff = []
        for I in range(nb):
            c = min(max(int(cnt[0, h, I]), 0), nb)
            eff.append([j for j in idx[0, h, I, :c].tolist() if 0 <= j < nb])
        ref, _ = masked_attention(q[0, :, h], k[0, :, h], v[0, :, h], N, b, eff, 1 / math.sqrt(d))
        nz = np.repeat([len(e) > 0 for e in eff], b)[:N]
        assert np.abs(o[0, h, :N][nz] - ref[nz]).max() <= TOL
        assert (o[0, h, :N][~nz] == 0).all()


@pytest.mark.parametrize("N,d,b,n,kind", [
    (1000, 64, 128, 8, "random"), (1000, 128, 64, 7, "empty"), (600, 128, 128, 1, "all"),
    (17776 // 8, 64, 128, 8, "single"), (513, 64, 64, 16, "random"),
])
def test_attn_global_tokens(N, d, b, n, kind):
    say("attn asa_g", N, d, b, n, kind)
    B, Hh = 1, 2
    rng = np.random.default_rng(N * n)
    q, k, v = smooth_qkv(N + n, B, N, Hh, d)
    nb = -(-N // b)
    Npad = nb * b
    lists = _lists(kind, B * Hh, nb, rng)
    cnt, idx = _upload(lists, B, Hh, nb)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    k_g, v_g, Ng = ops.meanpool_kv(k_r, v_t, N, b, n)
    scale = 1.0 / math.sqrt(d)
    o_r, lse = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, scale, dev(cnt), dev(idx), k_g, v_g, Ng, n,
                                   want_lse=True)
    torch.cuda.synchronize()
    o, l = host(o_r), host(lse)
    kg = host(k_g)[:, :, :Ng]
    vg = tiles_to_rows(host(v_g))[:, :, :Ng]
    gb = global_bias(N, n)
    for h in range(Hh):
        # the kernel is compared on the pooled tokens it was given (pooling has its own test)
        ref, rl = masked_attention(q[0, :, h], k[0, :, h], v[0, :, h], N, b, lists[h], scale,
                                   kg[0, h], vg[0, h], gb)
        assert np.abs(o[0, h, :N] - ref).max() <= TOL
        assert np.abs(l[0, h, :N] - rl).max() <= 1e-3


def test_attn_deterministic():
    N, d, b = 1000, 128, 128
    q, k, v = smooth_qkv(11, 1, N, 2, d)
    nb = 8
    rng = np.random.default_rng(0)
    cnt, idx = _upload(_lists("random", 2, nb, rng), 1, 2, nb)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), perm, 1024, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, 1024, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, 1024, b, "tiles_t")
    a = host(ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, 0.088, dev(cnt), dev(idx))[0])
    c = host(ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, 0.088, dev(cnt), dev(idx))[0])
    assert np.array_equal(a, c)


@pytest.mark.parametrize("N,d,b", [(1000, 128, 128), (2048, 64, 64), (700, 64, 128)])
def test_attn_work_order_does_not_change_results(N, d, b):
    """Rows are independent: the schedule from build_mask, a random
    permutation and index order give bit-identical outputs and lse."""
    say("attn order", N, d, b)
    B, Hh = 2, 3
    rng = np.random.default_rng(N + 3 * d + b)
    q, k, v = smooth_qkv(N + 11, B, N, Hh, d)
    nb = -(-N // b)
    Npad = nb * b
    cnt, idx = _upload(_lists("random", B * Hh, nb, rng), B, Hh, nb)
    ops = _ops()
    perm = dev(np.arange(N, dtype=np.int32))
    q_r = ops.reorder(dev_bf16(q), perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    scale = 1.0 / math.sqrt(d)
    P = np.zeros((B, Hh, nb, nb), np.float32)
    for bi in range(B):
        for h in range(Hh):
            for I in range(nb):
                P[bi, h, I, idx[bi, h, I, :cnt[bi, h, I]]] = 1.0
    _, _, _, order = ops.build_mask(dev(P), 1.0, want_order=True)
    outs = []
    for o in (None, order, dev(rng.permutation(B * Hh * nb).astype(np.int32))):
        o_r, lse = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, scale, dev(cnt), dev(idx), want_lse=True, order=o)
        torch.cuda.synchronize()
        outs.append((host(o_r)[:, :, :N].view(np.uint16), host(lse)[:, :, :N]))
    for o_, l_ in outs[1:]:
        assert np.array_equal(o_, outs[0][0]) and np.array_equal(l_, outs[0][1])


@pytest.mark.parametrize("N,d,b,n,per_head,in32,out32", [
    (1000, 128, 128, 0, False, False, False), (700, 64, 128, 8, True, False, True),
    (2048, 64, 64, 0, True, True, False), (1500, 128, 64, 16, False, True, True),
])
def test_attn_token_order_equals_reorder_then_inverse(N, d, b, n, per_head, in32, out32):
    """sparse_attn_fwd_tok (Q read and the output written in token order
    through the permutation) is bit-identical to reorder -> sparse_attn_fwd ->
    inverse_reorder, for bf16 / float32 operands, shared and per-head
    permutations, with and without global tokens, into a strided output."""
    say("attn tok", N, d, b, n, per_head, in32, out32)
    B, Hh = 2, 3
    rng = np.random.default_rng(N + d + n)
    q, k, v = smooth_qkv(N + 5, B, N, Hh, d)
    nb = -(-N // b)
    Npad = nb * b
    cnt, idx = _upload(_lists("random", B * Hh, nb, rng), B, Hh, nb)
    ops = _ops()
    pm = (np.stack([rng.permutation(N) for _ in range(Hh)]) if per_head else rng.permutation(N)).astype(np.int32)
    perm = dev(pm)
    qd = dev(q) if in32 else dev_bf16(q)
    q_r = ops.reorder(qd, perm, Npad, b, "rows")
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), perm, Npad, b, "tiles_t")
    kg = vg = None
    Ng = 0
    if n:
        kg, vg, Ng = ops.meanpool_kv(k_r, v_t, N, b, n)
    scale = 1.0 / math.sqrt(d)
    odt = torch.float32 if out32 else torch.bfloat16
    o_r, lse_a = ops.sparse_attn_fwd(q_r, k_r, v_t, N, b, scale, dev(cnt), dev(idx), kg, vg, Ng, n, want_lse=True)
    ref = ops.inverse_reorder(o_r, perm, N, out_dtype=odt)
    # a strided destination: every other head slot of a wider buffer
    wide = torch.full((B, N, 2 * Hh, d), 7.0, dtype=odt, device=ref.device)
    out, lse_b = ops.sparse_attn_fwd_tok(qd, perm, k_r, v_t, N, b, scale, dev(cnt), dev(idx), kg, vg, Ng, n,
                                         out=wide[:, :, ::2], out_dtype=odt, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(wide[:, :, 1::2], torch.full_like(wide[:, :, 1::2], 7.0))   # untouched
    assert np.array_equal(host(lse_a)[:, :, :N], host(lse_b)[:, :, :N])
