"""GPU parity: BSA query pruning (dbs_query_prune) and the attention over the kept
queries with token filling (dbs_sparse_attn_fwd_pruned_tok), through the C ABI.

- Pruning: q_count, rowsel and keep bit-exact against the oracle's float64
  selection; blocks whose m-th and (m+1)-th candidates lie within 1e-5 in
  dissimilarity (the oracle's tie flag: the GPU ranks float32 values) are
  counted and skipped.
- Attention: kept rows bit-identical to dbs_sparse_attn_fwd_tok on the same
  inputs (the same per-row arithmetic in 64-row workgroups), pruned rows
  bit-identical to their centre's row, and the whole output within max-abs
  2e-2 of the oracle's float64 attention followed by its filling."""
import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, dev, dev_bf16, host, kept_lists, say, smooth_qkv
from oracle.attention import masked_attention
from oracle.perm import perm_cuboid, perm_gilbert3d
from oracle.query_prune import anchors_reordered, fill, query_prune, window_anchors
from oracle.reorder import reorder_fast as o_reorder

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _setup(T, H, W, Hh, d, b, order, win, seed, cub=(4, 4, 4)):
    N = T * H * W
    q, k, v = smooth_qkv(seed, 1, N, Hh, d, grid=(T, H, W))
    perm = perm_gilbert3d(T, H, W) if order == "gilbert" else perm_cuboid(T, H, W, *cub)
    anc = anchors_reordered(perm, window_anchors(T, H, W, win))
    return N, q, k, v, perm.astype(np.int32), anc.astype(np.int32)


def _check_prune(q, perm, anc, N, b, r, Hh, blocks=None, q_in=None):
    """q_in: the device input (default: q as bf16); q is what the oracle reads."""
    ops = _ops()
    Npad = -(-N // b) * b
    nb = Npad // b
    g = [Guarded((1, Hh, nb), torch.int32), Guarded((1, Hh, nb, b), torch.int32),
         Guarded((1, Hh, Npad), torch.uint8, fill=171)]
    qc, rs, kp = ops.query_prune(dev_bf16(q) if q_in is None else q_in, dev(perm), dev(anc), Npad, b, r,
                                 q_count=g[0].view,
                                 rowsel=g[1].view, keep=g[2].view)
    torch.cuda.synchronize()
    assert all(x.intact() for x in g)          # nothing written outside the outputs
    qc, rs, kp = host(qc), host(rs), host(kp)
    qr = o_reorder(q, perm, Npad)
    n_ties = 0
    for h in range(Hh):
        rc, rrs, rkeep, ties = query_prune(qr[0, h], anc, N, b, r)
        tie = set(ties)
        n_ties += len(tie)
        for I in (range(nb) if blocks is None else blocks):
            if I in tie:
                continue
            assert qc[0, h, I] == rc[I], (h, I)
            assert np.array_equal(rs[0, h, I], rrs[I]), (h, I)
            lo, hi = I * b, min((I + 1) * b, N)
            assert np.array_equal(kp[0, h, lo:hi].astype(bool), rkeep[lo:hi]), (h, I)
        assert (kp[0, h, N:] == 0).all()
    return n_ties


@pytest.mark.parametrize("T,H,W,Hh,d,b,order,win,r", [
    (8, 16, 16, 2, 64, 64, "cuboid", (2, 2, 2), 0.5),     # the worked example's geometry, smaller grid
    (8, 16, 16, 1, 128, 64, "cuboid", (2, 2, 2), 0.25),   # r below the centres' share: centres only
    (5, 12, 20, 2, 128, 128, "gilbert", (1, 2, 2), 0.5),  # centres across block borders, ragged N
    (3, 10, 14, 1, 64, 128, "gilbert", (2, 3, 3), 0.8),
    (4, 8, 8, 1, 64, 64, "cuboid", (2, 2, 2), 1.0),       # keep all
])
def test_prune_bit_exact(T, H, W, Hh, d, b, order, win, r):
    say("query_prune", T, H, W, Hh, d, b, order, win, r)
    N, q, _, _, perm, anc = _setup(T, H, W, Hh, d, b, order, win, T * H + W)
    ties = _check_prune(q, perm, anc, N, b, r, Hh)
    assert ties <= max(1, (-(-N // b)) * Hh // 8)


@pytest.mark.parametrize("d", [64, 128])
def test_prune_float32_input(d):
    """A float32 Q is rounded to bf16 (nearest even) before the dissimilarities, as the attention
    reads it: values within a quarter bf16 ulp of the oracle's bf16 Q give its selection."""
    T, H, W, Hh, b = 5, 12, 20, 2, 128
    say("query_prune float32", T, H, W, Hh, d, b)
    N, q, _, _, perm, anc = _setup(T, H, W, Hh, d, b, "gilbert", (1, 2, 2), 17)
    rng = np.random.default_rng(5)
    q32 = (q + q * rng.uniform(-2.0 ** -11, 2.0 ** -11, q.shape)).astype(np.float32)
    assert not np.array_equal(q32, q)
    assert np.array_equal(torch.from_numpy(q32).to(torch.bfloat16).float().numpy(), q)   # rounds back to q
    ties = _check_prune(q, perm, anc, N, b, 0.5, Hh, q_in=dev(q32))
    assert ties <= max(1, (-(-N // b)) * Hh // 8)


def test_worked_example_counts_on_gpu():
    """The notes' example: 16 x 28 x 52 latent tokens, 4 x 4 x 4 blocks, 2 x 2 x 2 windows, r = 0.5:
    23,296 queries -> 11,648."""
    say("query_prune worked example")
    ops = _ops()
    T, H, W = 16, 28, 52
    N, q, _, _, perm, anc = _setup(T, H, W, 1, 64, 64, "cuboid", (2, 2, 2), 5)
    qc, rs, kp = ops.query_prune(dev_bf16(q), dev(perm), dev(anc), N, 64, 0.5)
    torch.cuda.synchronize()
    assert int(host(qc).sum()) == 11648 == int(host(kp).sum())
    assert (host(qc) == 32).all()


@pytest.mark.parametrize("T,H,W,Hh,d,b,order,win,r,fp32_out", [
    (8, 16, 16, 2, 64, 64, "cuboid", (2, 2, 2), 0.5, False),
    (5, 12, 20, 2, 128, 128, "gilbert", (1, 2, 2), 0.5, True),
    (5, 12, 20, 1, 128, 128, "gilbert", (2, 2, 2), 0.7, False),   # two 64-row pieces for some blocks
    (3, 10, 14, 1, 64, 128, "gilbert", (2, 3, 3), 0.3, False),
])
def test_pruned_attention(T, H, W, Hh, d, b, order, win, r, fp32_out):
    say("pruned attention", T, H, W, Hh, d, b, order, win, r)
    ops = _ops()
    N, q, k, v, perm, anc = _setup(T, H, W, Hh, d, b, order, win, 3 * T + H)
    Npad = -(-N // b) * b
    nb = Npad // b
    scale = 1.0 / np.sqrt(d)
    permd = dev(perm)
    qd = dev_bf16(q)
    k_r = ops.reorder(dev_bf16(k), permd, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), permd, Npad, b, "tiles_t")
    P = ops.estimate_blocks(ops.reorder(qd, permd, Npad, b, "rows"), k_r, N, b, min(16, b), scale)
    cnt, idx, _, order_buf = ops.build_mask(P, 0.6, want_order=True)
    qc, rs, kp = ops.query_prune(qd, permd, dev(anc), Npad, b, r)
    odt = torch.float32 if fp32_out else torch.bfloat16
    out, lse = ops.sparse_attn_fwd_pruned_tok(qd, permd, k_r, v_t, N, b, scale, cnt, idx, qc, rs, dev(anc), kp,
                                              out_dtype=odt, want_lse=True, order=order_buf)
    full, lse_f = ops.sparse_attn_fwd_tok(qd, permd, k_r, v_t, N, b, scale, cnt, idx, out_dtype=odt, want_lse=True)
    torch.cuda.synchronize()
    o, f, keep = host(out), host(full), host(kp)[0]
    lo, lf = host(lse), host(lse_f)
    inv = np.empty(N, dtype=np.int64)
    inv[perm] = np.arange(N)
    for h in range(Hh):
        for i in range(N):          # reordered row i is token perm[i]
            t = perm[i]
            if keep[h, i]:
                assert np.array_equal(o[0, t, h], f[0, t, h]), (h, i)
                assert lo[0, h, i] == lf[0, h, i]
            else:
                assert np.array_equal(o[0, t, h], o[0, perm[anc[i]], h]), (h, i)
                assert lo[0, h, i] == lo[0, h, anc[i]]
    # the oracle: attention on every row, then the filling
    qr, kr, vr = (o_reorder(x, perm, Npad) for x in (q, k, v))
    hc, hi = host(cnt), host(idx)
    for h in range(Hh):
        kept = kept_lists(hc[0, h], hi[0, h])[0]
        ref, _ = masked_attention(qr[0, h], kr[0, h], vr[0, h], N, b, kept, scale)
        ref = fill(ref, keep[h, :N].astype(bool), anc)
        got = o[0, perm, h].astype(np.float64)          # reordered rows
        assert np.abs(got - ref).max() <= TOL, np.abs(got - ref).max()


def test_pruned_wan_shape():
    """The Wan2.1-1.3B-shaped layer (12 heads, 32,760 tokens, b 128, Gilbert order) with 2 x 2 x 2
    windows and r = 0.5: sampled blocks against the oracle's pruning and attention; every kept row
    equal to the unpruned attention's, every pruned row to its centre's."""
    say("pruned attention wan")
    from workloads import get_config, make_inputs
    ops = _ops()
    cfg = get_config(2)
    T, H, W = cfg.T, cfg.H, cfg.W
    N, Hh, d, b = T * H * W, cfg.heads, cfg.d, cfg.b
    Npad = -(-N // b) * b
    nb = Npad // b
    q, k, v = make_inputs(cfg)
    perm = perm_gilbert3d(T, H, W).astype(np.int32)
    anc = ops.prune_anchors(T, H, W, (2, 2, 2), perm)
    permd, ancd = dev(perm), dev(anc)
    scale = 1.0 / np.sqrt(d)
    qd = dev_bf16(q)
    k_r = ops.reorder(dev_bf16(k), permd, Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(v), permd, Npad, b, "tiles_t")
    cnt, idx, _, _ = ops.estimate_mask(qd, k_r, N, b, cfg.k, scale, "cumulative", 0.9, q_perm=permd)
    qc, rs, kp = ops.query_prune(qd, permd, ancd, Npad, b, 0.5)
    out, _ = ops.sparse_attn_fwd_pruned_tok(qd, permd, k_r, v_t, N, b, scale, cnt, idx, qc, rs, ancd, kp)
    full, _ = ops.sparse_attn_fwd_tok(qd, permd, k_r, v_t, N, b, scale, cnt, idx)
    torch.cuda.synchronize()
    o, f, keep, qch = host(out), host(full), host(kp)[0], host(qc)[0]
    assert 0.5 * Hh * N <= int(qch.sum()) < 0.6 * Hh * N
    for h in range(Hh):
        kh = keep[h, :N].astype(bool)
        toks = perm[kh]
        assert np.array_equal(o[0, toks, h], f[0, toks, h]), h
        pr = np.nonzero(~kh)[0]
        assert np.array_equal(o[0, perm[pr], h], o[0, perm[anc[pr]], h]), h
    rng = np.random.default_rng(2)
    blocks = sorted({0, nb - 1} | set(rng.choice(nb, 6, replace=False).tolist()))
    qr = o_reorder(q[:, :, :2], perm, Npad)
    kr, vr = (o_reorder(x[:, :, :2], perm, Npad) for x in (k, v))
    hc, hi = host(cnt), host(idx)
    for h in range(2):
        rc, rrs, rkeep, ties = query_prune(qr[0, h], anc, N, b, 0.5)
        for I in blocks:
            if I in ties:
                continue
            assert qch[h, I] == rc[I] and np.array_equal(host(rs)[0, h, I], rrs[I]), (h, I)
        kept = kept_lists(hc[0, h], hi[0, h])[0]
        # rows of the sampled blocks and of their centres
        need = sorted({int(anc[i]) // b for I in blocks for i in range(I * b, min((I + 1) * b, N))} | set(blocks))
        ref, _ = masked_attention(qr[0, h], kr[0, h], vr[0, h], N, b, kept, scale, query_blocks=need)
        for I in blocks:
            for i in range(I * b, min((I + 1) * b, N)):
                src = i if keep[h, i] else int(anc[i])
                got = o[0, perm[i], h].astype(np.float64)
                assert np.abs(got - ref[src]).max() <= TOL, (h, i)


@pytest.mark.parametrize("cid", [2, 5])
def test_layer_forward_pruned(cid):
    """AsaLayer.forward_pruned equals the library calls made one by one, bit for bit; its kept
    rows equal the unpruned layer's rows and its pruned rows their centre's row (per head, for
    the per-head cuboid orders of the 720p-shaped layer)."""
    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    from workloads import get_config, make_inputs
    from workloads.generator import head_cuboid
    say("layer forward_pruned", cid)
    ops = _ops()
    cfg = get_config(cid)
    heads = [0, 1]
    cub = [head_cuboid(cfg, h) for h in heads] if cfg.reorder == "cuboid_per_head" else None
    spec = LayerSpec(T=cfg.T, H=cfg.H, W=cfg.W, heads=len(heads), d=cfg.d, b=cfg.b, k=cfg.k, tau=0.9,
                     order=cfg.reorder, cuboid=cfg.cuboid, cuboids=cub)
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).cuda() for a in make_inputs(cfg, heads=heads, workers=4))
    layer = AsaLayer(spec)
    layer.enable_query_pruning(0.5)
    out = layer.forward_pruned(q, k, v)
    # the same calls one by one
    ref = AsaLayer(spec)
    ref.prepare(q, k, v)
    ref.mask()
    perm_h = ref.perm.cpu().numpy()
    anc = np.stack([ops.prune_anchors(cfg.T, cfg.H, cfg.W, (2, 2, 2), p) for p in perm_h]) if perm_h.ndim == 2 \
        else ops.prune_anchors(cfg.T, cfg.H, cfg.W, (2, 2, 2), perm_h)
    anc_d = torch.from_numpy(anc).cuda()
    assert torch.equal(anc_d, layer.anchor)
    qc, rs, kp = ops.query_prune(q, ref.perm, anc_d, spec.Npad, spec.b, 0.5)
    out2, _ = ops.sparse_attn_fwd_pruned_tok(q, ref.perm, ref.k_r, ref.v_t, spec.N, spec.b, spec.scale,
                                             ref.kv_count, ref.kv_idx, qc, rs, anc_d, kp, order=ref.order)
    full = ref.attend()
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(layer.keep, kp)
    o, f, kpn = host(out).astype(np.float32), host(full).astype(np.float32), host(kp)
    for hi in range(len(heads)):
        p = perm_h[hi] if perm_h.ndim == 2 else perm_h
        a_h = anc[hi] if anc.ndim == 2 else anc
        kept = kpn[0, hi, :spec.N].astype(bool)
        tok = p[:spec.N]
        np.testing.assert_array_equal(o[0, tok[kept], hi], f[0, tok[kept], hi])      # kept rows: unpruned values
        np.testing.assert_array_equal(o[0, tok[~kept], hi], o[0, tok[a_h[:spec.N][~kept]], hi])   # filled rows


def test_layer_pruning_rejects_unsupported_layers():
    """forward_pruned needs enable_query_pruning first (and again after a change of order); the
    float32 and ASA_G layers and keep ratios outside (0, 1] are refused before any launch."""
    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    say("layer pruning errors")
    spec = LayerSpec(T=4, H=8, W=8, heads=1, d=64, b=64, k=8)
    layer = AsaLayer(spec)
    x = torch.zeros((1, spec.N, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="enable_query_pruning"):
        layer.forward_pruned(x, x, x)
    for r in (0.0, 1.5):
        with pytest.raises(ValueError, match="keep ratio"):
            layer.enable_query_pruning(r)
    layer.enable_query_pruning(0.5)
    assert layer.anchor is not None and layer.anchor.shape == (spec.N,)
    layer.choose_cuboids_sics(x, [(1, 8, 8), (2, 4, 8)])
    assert layer.anchor is None   # the order changed: the centres must be rebuilt
    with pytest.raises(RuntimeError, match="enable_query_pruning"):
        layer.forward_pruned(x, x, x)
    with pytest.raises(ValueError, match="bf16 layer without global tokens"):
        AsaLayer(LayerSpec(T=4, H=8, W=8, heads=1, d=64, b=64, k=8, dtype="fp32")).enable_query_pruning(0.5)
    with pytest.raises(ValueError, match="bf16 layer without global tokens"):
        AsaLayer(LayerSpec(T=4, H=8, W=8, heads=1, d=64, b=64, k=8, n_pool=8)).enable_query_pruning(0.5)
