"""The estimate-and-mask call that allocates nothing (dbs_estimate_mask_tok_noalloc), against the
same call with a caller's workspace (dbs_estimate_mask_tok): every output identical, bit for bit,
on two calls in a row, the second smaller, so that it runs over what the first left in the
library's static scratch."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, dev_bf16, say
from workloads.configs import get_config
from workloads.generator import make_inputs

pytestmark = pytest.mark.gpu


def _ops():
    from dynamic_block_sparse_gilbert_amd import ops
    return ops


def _outputs(B, Hh, nb, dv, fill):
    return dict(kv_count=torch.full((B, Hh, nb), fill, dtype=torch.int32, device=dv),
                kv_idx=torch.full((B, Hh, nb, nb), fill, dtype=torch.int32, device=dv),
                order=torch.full((B * Hh * nb,), fill, dtype=torch.int32, device=dv),
                p_imp=torch.full((B, Hh, nb, nb), float(fill), dtype=torch.float32, device=dv),
                mask=torch.full((B, Hh, nb, nb), 3, dtype=torch.uint8, device=dv))


def _case(cid, heads, rule, param, per_head, seed):
    """q in token order, k_r in curve order (reordered by the library), perm, sizes."""
    ops = _ops()
    cfg = get_config(cid)
    q, k, _ = make_inputs(cfg, heads=heads, workers=8)
    N, b, d, Hh = cfg.N, cfg.b, cfg.d, len(heads)
    Npad = -(-N // b) * b
    rng = np.random.default_rng(seed)
    if per_head:
        pm = np.stack([rng.permutation(N) for _ in range(Hh)]).astype(np.int32)
    else:
        pm = ops.perm_gilbert3d(cfg.T, cfg.H, cfg.W, cfg.text_prefix)
    perm = dev(pm)
    qd = dev_bf16(q)
    k_r = ops.reorder(dev_bf16(k), perm, Npad, b, "rows")
    return qd, perm, k_r, N, b, cfg.k, cfg.scale, rule, param


def _same_order(got: torch.Tensor, ref: torch.Tensor, kv_count: torch.Tensor) -> None:
    """The work order lists rows by kept count, descending, inside fixed ranges; rows of equal count
    may come in any order.  So: a permutation, the same count at every position, and the same rows
    in every run of equal counts."""
    g, r = got.cpu().numpy().astype(np.int64), ref.cpu().numpy().astype(np.int64)
    c = kv_count.cpu().numpy().reshape(-1)
    R = c.size
    assert np.array_equal(np.sort(g), np.arange(R))
    assert np.array_equal(c[g], c[r])
    seg = np.concatenate([[0], np.cumsum(c[r][1:] != c[r][:-1])]).astype(np.int64)
    assert np.array_equal(np.sort(seg * R + g), np.sort(seg * R + r))


def _check(qd, perm, k_r, N, b, k, scale, rule, param):
    ops = _ops()
    B, Hh, Npad, _ = k_r.shape
    nb = Npad // b
    ref = _outputs(B, Hh, nb, k_r.device, -7)
    got = _outputs(B, Hh, nb, k_r.device, -7)
    ops.estimate_mask(qd, k_r, N, b, k, scale, rule, param, q_perm=perm, kv_count=ref["kv_count"],
                      kv_idx=ref["kv_idx"], order=ref["order"], p_imp=ref["p_imp"], want_mask=False)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    ops.estimate_mask_noalloc(qd, perm, k_r, N, b, k, scale, rule, param, got["kv_count"], got["kv_idx"],
                              order=got["order"], p_imp=got["p_imp"], mask=got["mask"])
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before       # the binding allocated nothing either
    for name in ("kv_count", "kv_idx"):
        assert torch.equal(got[name], ref[name]), name
    _same_order(got["order"], ref["order"], ref["kv_count"])
    assert torch.equal(got["p_imp"].view(torch.int32), ref["p_imp"].view(torch.int32))
    # the mask agrees with the lists
    cnt = got["kv_count"].cpu().numpy().reshape(-1, nb)
    idx = got["kv_idx"].cpu().numpy().reshape(-1, nb, nb)
    msk = got["mask"].cpu().numpy().reshape(-1, nb, nb)
    assert set(np.unique(msk).tolist()) <= {0, 1}
    for r in range(0, cnt.shape[0], max(1, cnt.shape[0] // 4)):
        for I in range(0, nb, max(1, nb // 16)):
            row = np.zeros(nb, np.uint8)
            row[idx[r, I, :cnt[r, I]]] = 1
            assert np.array_equal(msk[r, I], row)
    return float(cnt.sum()) / (cnt.shape[0] * nb * nb)


def test_noalloc_two_calls_second_smaller():
    """Wan2.1-1.3B-shaped layer (12 heads, 32,760 tokens, d 128, k 16, tau 0.9, Gilbert order),
    then 5 heads of the CogVideoX-shaped layer (17,776 tokens, d 64, per-head orders, top-8)."""
    ops = _ops()
    say("noalloc call 1: 12 heads x 32760, d 128, cumulative 0.9")
    a = _case(2, list(range(12)), "cumulative", 0.9, False, 1)
    need = ops.estimate_workspace_bytes(1, 12, a[3], 128, a[4], a[5])
    assert 0 < need <= ops.NOALLOC_SCRATCH_BYTES
    dens = _check(*a)
    assert 0.0 < dens < 0.5
    say("noalloc call 2: 5 heads x 17776, d 64, per-head perms, top-8")
    c = _case(3, [0, 7, 19, 30, 47], "topk", 8.0, True, 2)
    dens = _check(*c)
    assert abs(dens - 8.0 / 139) < 1e-9
    say("noalloc call 3: the first shape again")
    _check(*a)


def test_noalloc_rejects_oversized_shape():
    """The 153,600-token layer's workspace exceeds the static scratch: the call says so and
    writes nothing."""
    ops = _ops()
    from dynamic_block_sparse_gilbert_amd._lib import DbsError
    N, b, Hh, d = 153600, 128, 2, 128
    nb = N // b
    need = ops.estimate_workspace_bytes(1, Hh, N, d, b, 16)
    if need <= ops.NOALLOC_SCRATCH_BYTES:
        Hh = 24
    say("noalloc oversized", Hh, N)
    q = torch.zeros((1, N, Hh, d), dtype=torch.bfloat16, device="cuda")
    perm = torch.arange(N, dtype=torch.int32, device="cuda")
    k_r = torch.zeros((1, Hh, N, d), dtype=torch.bfloat16, device="cuda")
    cnt = torch.full((1, Hh, nb), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((1, Hh, nb, nb), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(DbsError, match="scratch"):
        ops.estimate_mask_noalloc(q, perm, k_r, N, b, 16, 1.0 / np.sqrt(d), "cumulative", 0.9, cnt, idx)
    torch.cuda.synchronize()
    assert (cnt == -7).all().item()
