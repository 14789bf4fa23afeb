"""GPU parity: reorder / inverse reorder / mean-pool against the oracle (bit-exact
for data movement; mean-pool within one bf16 rounding of the float64 mean)."""
import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, dev, dev_bf16, host, say, tiles_to_rows
from oracle.attention import meanpool
from oracle.perm import perm_gilbert3d
from oracle.reorder import inverse_reorder as o_inverse
from oracle.reorder import reorder_fast as o_reorder
from workloads import get_config, make_inputs
from workloads.generator import bf16_round

pytestmark = pytest.mark.gpu


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _tiles_to_rows(yt: np.ndarray) -> np.ndarray:
    return tiles_to_rows(yt)


CASES = [  # B, N, Hh, d, b, per_head, in_dtype
    (1, 300, 3, 64, 64, False, "bf16"),
    (2, 300, 3, 128, 128, True, "bf16"),
    (2, 257, 2, 128, 64, False, "fp32"),
    (1, 1000, 4, 64, 128, True, "fp32"),
    (1, 128, 1, 128, 128, False, "bf16"),
    (1, 1, 1, 64, 64, False, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_reorder_rows_and_tiles(case):
    B, N, Hh, d, b, per_head, in_dt = case
    say("reorder", case)
    ops = _ops()
    rng = np.random.default_rng(N + d)
    x = rng.standard_normal((B, N, Hh, d)).astype(np.float32)
    if in_dt == "bf16":
        x = bf16_round(x)
    perm = np.stack([rng.permutation(N) for _ in range(Hh)]).astype(np.int32) if per_head else \
        rng.permutation(N).astype(np.int32)
    Npad = -(-N // b) * b
    xt = dev_bf16(x) if in_dt == "bf16" else dev(x)
    pt = dev(perm)
    gy = Guarded((B, Hh, Npad, d), torch.bfloat16)
    gt = Guarded((B, Hh, Npad // b, d, b), torch.bfloat16)
    y = ops.reorder(xt, pt, Npad, b, "rows", y=gy.view)
    yt = ops.reorder(xt, pt, Npad, b, "tiles_t", y=gt.view)
    torch.cuda.synchronize()
    assert gy.intact() and gt.intact()          # nothing written outside the outputs
    ref = bf16_round(o_reorder(x, perm, Npad))
    assert np.array_equal(host(y), ref)
    assert np.array_equal(_tiles_to_rows(host(yt)), ref)
    # K and V in one launch: the same rows and tiles as the two separate calls
    v = rng.standard_normal((B, N, Hh, d)).astype(np.float32)
    if in_dt == "bf16":
        v = bf16_round(v)
    vt_in = dev_bf16(v) if in_dt == "bf16" else dev(v)
    k_r, v_t = ops.reorder_kv(xt, vt_in, pt, Npad, b)
    torch.cuda.synchronize()
    assert np.array_equal(host(k_r), ref)
    assert np.array_equal(_tiles_to_rows(host(v_t)), bf16_round(o_reorder(v, perm, Npad)))
    if in_dt == "fp32":
        y32 = ops.reorder(xt, pt, Npad, b, "rows", out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(host(y32), o_reorder(x, perm, Npad))
    # inverse: bf16 rows back to token order, bf16 and fp32 outputs
    gb = Guarded((B, N, Hh, d), torch.bfloat16)
    back = ops.inverse_reorder(y, pt, N, out=gb.view)
    back32 = ops.inverse_reorder(y, pt, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert gb.intact()
    assert np.array_equal(host(back), bf16_round(x))
    assert np.array_equal(host(back32), o_inverse(ref, perm, N))


def test_reorder_strided_views():
    say("reorder strided")
    ops = _ops()
    B, N, Hh, d, b = 2, 200, 3, 128, 64
    rng = np.random.default_rng(7)
    base = bf16_round(rng.standard_normal((B, Hh, N, d)).astype(np.float32))
    xt = dev_bf16(base).permute(0, 2, 1, 3)          # [B, N, Hh, d] view, head-major storage
    x = base.transpose(0, 2, 1, 3)
    perm = rng.permutation(N).astype(np.int32)
    Npad = 256
    y = ops.reorder(xt, dev(perm), Npad, b, "rows")
    vbase = bf16_round(rng.standard_normal((B, Hh, N, d)).astype(np.float32))
    k_r, v_t = ops.reorder_kv(xt, dev_bf16(vbase).permute(0, 2, 1, 3), dev(perm), Npad, b)
    out = torch.zeros((B, Hh, N, d), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    ops.inverse_reorder(y, dev(perm), N, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), o_reorder(x, perm, Npad))
    assert np.array_equal(host(out), x)
    assert np.array_equal(host(k_r), o_reorder(x, perm, Npad))
    assert np.array_equal(_tiles_to_rows(host(v_t)), o_reorder(vbase.transpose(0, 2, 1, 3), perm, Npad))


@pytest.mark.parametrize("N,n,d,b", [(300, 8, 64, 64), (1000, 7, 128, 128), (17776, 8, 64, 128),
                                     (129, 1, 128, 64), (50, 50, 64, 64)])
def test_meanpool(N, n, d, b):
    say("meanpool", N, n, d, b)
    ops = _ops()
    rng = np.random.default_rng(N * n)
    B, Hh = 1, 2
    x = bf16_round(rng.standard_normal((B, N, Hh, 2 * d)).astype(np.float32))
    kx, vx = x[..., :d].copy(), x[..., d:].copy()
    perm = np.arange(N, dtype=np.int32)
    Npad = -(-N // b) * b
    k_r = ops.reorder(dev_bf16(kx), dev(perm), Npad, b, "rows")
    v_t = ops.reorder(dev_bf16(vx), dev(perm), Npad, b, "tiles_t")
    k_g, v_g, Ng = ops.meanpool_kv(k_r, v_t, N, b, n)
    torch.cuda.synchronize()
    kg = host(k_g)
    vg = _tiles_to_rows(host(v_g))
    assert Ng == -(-N // n)
    assert (kg[:, :, Ng:] == 0).all() and (vg[:, :, Ng:] == 0).all()
    for h in range(Hh):
        rk = meanpool(kx[0, :, h], N, n)
        rv = meanpool(vx[0, :, h], N, n)
        # within one bf16 rounding (8 mantissa bits) of the exact mean, plus the
        # float32 summation error for means near zero
        for got, ref in ((kg[0, h, :Ng], rk), (vg[0, h, :Ng], rv)):
            err = np.abs(got - ref)
            assert (err <= np.abs(ref) * 2.0 ** -8 + 1e-5).all(), err.max()


def test_reorder_full_wan_shape():
    """Whole 12-head Wan2.1-1.3B layer input, the launch configuration of the bench."""
    cfg = get_config(2)
    say("reorder full", cfg.name)
    ops = _ops()
    q, k, v = make_inputs(cfg)
    perm = ops.perm_gilbert3d(cfg.T, cfg.H, cfg.W)
    assert np.array_equal(perm, perm_gilbert3d(cfg.T, cfg.H, cfg.W))
    pt = dev(perm)
    y = ops.reorder(dev_bf16(q), pt, cfg.Npad, cfg.b, "rows")
    yt = ops.reorder(dev_bf16(v), pt, cfg.Npad, cfg.b, "tiles_t")
    k_r, v_t = ops.reorder_kv(dev_bf16(k), dev_bf16(v), pt, cfg.Npad, cfg.b)   # the layer's launch
    torch.cuda.synchronize()
    assert np.array_equal(host(y), o_reorder(q, perm, cfg.Npad))
    v_rows = o_reorder(v, perm, cfg.Npad)
    assert np.array_equal(_tiles_to_rows(host(yt)), v_rows)
    assert np.array_equal(_tiles_to_rows(host(v_t)), v_rows)
    assert np.array_equal(host(k_r), o_reorder(k, perm, cfg.Npad))


@pytest.mark.parametrize("N,n,d,b,order,f32", [
    (300, 8, 64, 64, "gilbert", False), (17776, 8, 64, 128, "gilbert", False),   # config 3's window and block
    (1000, 16, 128, 128, "identity", True), (129, 1, 128, 64, "gilbert", False),
    (1000, 7, 128, 128, "gilbert", False),    # 7 does not divide 128: the two passes
    (640, 64, 64, 64, "identity", False), (50, 50, 64, 64, "identity", False)])
def test_reorder_kv_pool_equals_two_calls(N, n, d, b, order, f32):
    """dbs_reorder_kv_pool: k_r, v_t, k_g and v_g bit-identical to dbs_reorder_kv followed by
    dbs_meanpool_kv (whose means the test above checks against the oracle)."""
    say("reorder_kv_pool", N, n, d, b, order)
    ops = _ops()
    rng = np.random.default_rng(N + n)
    B, Hh = 1, 2
    x = rng.standard_normal((B, N, Hh, 2 * d)).astype(np.float32)
    if not f32:
        x = bf16_round(x)
    kx, vx = x[..., :d].copy(), x[..., d:].copy()
    if order == "gilbert":
        perm = np.random.default_rng(1).permutation(N).astype(np.int32)
    else:
        perm = np.arange(N, dtype=np.int32)
    Npad = -(-N // b) * b
    kd, vd = (dev(kx), dev(vx)) if f32 else (dev_bf16(kx), dev_bf16(vx))
    pd = dev(perm)
    k1, v1 = ops.reorder_kv(kd, vd, pd, Npad, b)
    kg1, vg1, _ = ops.meanpool_kv(k1, v1, N, b, n)
    k2, v2, kg2, vg2 = ops.reorder_kv(kd, vd, pd, Npad, b, n_pool=n)
    torch.cuda.synchronize()
    for a, c in ((k1, k2), (v1, v2), (kg1, kg2), (vg1, vg2)):
        assert torch.equal(a, c)
