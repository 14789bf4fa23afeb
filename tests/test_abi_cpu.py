"""CPU tier for the C-ABI library: it loads, exports every declared symbol, its
host permutation helpers match the oracle bit for bit, and every device entry
point rejects bad arguments on the host (no launch happens, so no GPU is
needed)."""
import ctypes as C
import itertools
import os
import re

import numpy as np
import pytest

from oracle.perm import perm_cuboid as o_cuboid
from oracle.perm import perm_gilbert3d as o_gilbert
from workloads.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dbs():
    from dynamic_block_sparse_gilbert_amd import _lib, ops
    _lib.lib()
    return ops, _lib


def _declared():
    src = open(os.path.join(ROOT, "include", "dbs.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+)+\*?(dbs_\w+)\s*\(", src, re.M)))


def test_all_declared_symbols_exported(dbs):
    _, L = dbs
    names = _declared()
    assert len(names) >= 12, names
    h = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)
    assert L.lib().dbs_abi_version() == 13


@pytest.mark.parametrize("T,H,W", list(itertools.product(range(1, 7), repeat=3)))
def test_gilbert_cpp_matches_oracle_small(dbs, T, H, W):
    ops, _ = dbs
    assert np.array_equal(ops.perm_gilbert3d(T, H, W), o_gilbert(T, H, W))


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_gilbert_cpp_matches_oracle_workloads(dbs, cfg):
    ops, _ = dbs
    assert np.array_equal(ops.perm_gilbert3d(cfg.T, cfg.H, cfg.W, cfg.text_prefix),
                          o_gilbert(cfg.T, cfg.H, cfg.W, cfg.text_prefix))


@pytest.mark.parametrize("grid", [(40, 48, 80), (31, 45, 80), (5, 9, 7)])
@pytest.mark.parametrize("cub", [(4, 4, 8), (1, 8, 16), (2, 8, 8), (8, 4, 4), (3, 2, 5)])
def test_cuboid_cpp_matches_oracle(dbs, grid, cub):
    ops, _ = dbs
    assert np.array_equal(ops.perm_cuboid(*grid, *cub, prefix=3), o_cuboid(*grid, *cub, prefix=3))


def test_perm_invert(dbs):
    ops, L = dbs
    p = ops.perm_gilbert3d(3, 4, 5, prefix=2)
    inv = ops.perm_invert(p)
    assert np.array_equal(inv[p], np.arange(p.size))
    with pytest.raises(L.DbsError, match="INVALID_ARG"):
        ops.perm_invert(np.array([0, 2, 2], dtype=np.int32))


def test_perm_errors(dbs):
    ops, L = dbs
    with pytest.raises(L.DbsError, match="INVALID_ARG"):
        ops.perm_gilbert3d(0, 3, 3)
    with pytest.raises(L.DbsError, match="INVALID_ARG"):
        ops.perm_cuboid(2, 2, 2, 0, 1, 1)
    out = np.empty(8, dtype=np.int32)
    assert L.lib().dbs_perm_gilbert3d(2, 2, 2, -1, out.ctypes.data) == -1
    assert b"prefix" in L.lib().dbs_last_error()
    assert L.lib().dbs_perm_gilbert3d(1 << 16, 1 << 16, 2, 0, out.ctypes.data) == -1


# ---- device entry points: argument validation only (nothing is launched) ----
# These pass fake device addresses that validation must reject before any
# launch; they run only where no GPU is present, so a regression in the checks
# shows up as a failed launch on the CPU, never as an access on a real device.


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs without a GPU only")

A = 1 << 20          # a fake, 16-byte aligned "device" address; never dereferenced
MIS = A + 4          # misaligned


def _reorder(L, **kw):
    a = dict(x=A, x_dt=0, sb=0, sn=1024, sh=128, y=A, y_dt=0, lay=0, perm=A, ph=0,
             B=1, Hh=8, N=100, Npad=128, d=128, b=128)
    a.update(kw)
    return L.lib().dbs_reorder(a["x"], a["x_dt"], a["sb"], a["sn"], a["sh"], a["y"], a["y_dt"], a["lay"],
                               a["perm"], a["ph"], a["B"], a["Hh"], a["N"], a["Npad"], a["d"], a["b"], None)


@cpu_only
def test_reorder_validation(dbs):
    _, L = dbs
    assert _reorder(L, x=0) == -1
    assert _reorder(L, y=MIS) == -3
    assert _reorder(L, d=96) == -2
    assert _reorder(L, b=32) == -2
    assert _reorder(L, Npad=120) == -1
    assert _reorder(L, Npad=256) == -1          # a whole empty block
    assert _reorder(L, sn=1025) == -3
    assert _reorder(L, x_dt=0, y_dt=1) == -2
    assert _reorder(L, lay=1, y_dt=1, x_dt=1) == -2
    assert _reorder(L, ph=2) == -1
    assert _reorder(L, N=0) == -1


@cpu_only
def test_estimate_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_estimate_blocks
    ws = L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 8)
    # 1 split of (m, l) per sampled query + the block maxima of each sampled query (nb = 2 cells
    # of k = 8 keys)
    assert ws == 1 * 2 * 1 * 16 * 8 + 1 * 2 * 16 * 2 * 4
    ok = (A, A, 0, 1, 2, 100, 128, 128, 64, 8, 0.125, A, A, ws, None)
    def call(**kw):
        a = list(ok)
        names = ["q", "k", "dt", "B", "Hh", "N", "Npad", "d", "b", "k_", "scale", "p", "w", "wb", "s"]
        for n, v in kw.items():
            a[names.index(n)] = v
        return f(*a)
    assert call(q=0) == -1
    assert call(dt=2) == -1               # no such dtype (float32 is a supported path: not launched here)
    assert call(dt=1, p=MIS) == -3
    assert call(dt=1, k_=0) == -1
    assert call(dt=1, wb=ws - 4) == -1
    # any k in [1, b] is a valid size: k = 6 reaches the workspace check (slots padded to 8)
    assert L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 6) == ws
    assert call(k_=6, wb=ws - 4) == -1
    assert "workspace" in L.lib().dbs_last_error().decode()
    assert call(k_=0) == -1
    assert call(k_=128) == -1
    assert call(wb=ws - 4) == -1
    assert call(scale=float("nan")) == -1
    assert call(p=MIS) == -3
    assert L.lib().dbs_estimate_workspace_bytes(0, 1, 1, 64, 1, 1) == 0
    assert L.lib().dbs_estimate_workspace_bytes(1, 1, 1, 96, 1, 1) == 0


@cpu_only
def test_estimate_tok_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_estimate_blocks_tok
    ws = L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 8)
    # q, q_dt, sb, sn, sh, perm, per_head, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, ws, ws_bytes, stream
    ok = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, A, 1, 2, 100, 128, 128, 64, 8, 0.125, A, A, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(0, 0) == -1               # q NULL
    assert call(5, 0) == -1               # perm NULL
    assert call(0, A + 2) == -3           # misaligned q
    assert call(5, A + 2) == -3           # misaligned perm
    assert call(1, 7) == -1               # bad dtype
    assert call(6, 2) == -1               # perm_per_head
    assert call(3, 2 * 128 + 4) == -3     # row stride breaks 16-byte rows
    assert call(3, -1) == -1
    assert call(7, 0) == -1               # k_r NULL
    a = list(ok)
    a[14], a[18] = 6, ws - 4              # k = 6 is accepted; the small workspace is not
    assert f(*a) == -1 and "workspace" in L.lib().dbs_last_error().decode()
    assert call(18, ws - 4) == -1         # small workspace


@cpu_only
def test_estimate_mask_noalloc_validation(dbs):
    """The no-alloc call checks its arguments as dbs_estimate_mask_tok does and refuses a shape whose
    workspace exceeds the static scratch, all before any device work (nothing is launched here)."""
    _, L = dbs
    g = L.lib().dbs_estimate_mask_tok_noalloc
    # q, q_dt, sb, sn, sh, perm, per_head, k_r, B, Hh, N, Npad, d, b, k, scale, rule, param, p_imp, kv_count,
    # kv_idx, mask, order, stream
    ok = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, A, 1, 2, 100, 128, 128, 64, 8, 0.125, 0, 0.9, None, A, A, None,
          None, None]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)
    assert call(a0=0) == -1               # q NULL
    assert call(a5=0) == -1               # perm NULL
    assert call(a19=0) == -1              # kv_count NULL
    assert call(a22=A + 2) == -3          # misaligned order
    assert call(a16=9) == -1              # unknown rule
    assert call(a17=0.0) == -1            # tau 0
    assert call(a12=96) == -2             # head dimension
    assert call(a11=192) == -1            # Npad not the padded length
    # 24 heads of 153,600 tokens: gigabytes of workspace, above the static maximum
    N, b, k, Hh = 153600, 128, 16, 24
    need = L.lib().dbs_estimate_workspace_bytes(1, Hh, N, 128, b, k)
    assert need > 128 << 20
    st = call(a2=N * Hh * 128, a3=Hh * 128, a4=128, a9=Hh, a10=N, a11=N, a13=b, a14=k)
    assert st == -2
    msg = L.lib().dbs_last_error().decode()
    assert "scratch" in msg and str(need) in msg and str(128 << 20) in msg


@cpu_only
def test_attn_tok_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_sparse_attn_fwd_tok
    # q, q_dt, qsb, qsn, qsh, perm, per_head, k_r, v_r, B, Hh, N, Npad, d, b, scale, kv_count, kv_idx, order,
    # k_g, v_g, Ng, n_pool, out, out_dt, osb, osn, osh, lse, stream
    ok = [A, 0, 1000 * 4 * 128, 4 * 128, 128, A, 1, A, A, 1, 4, 1000, 1024, 128, 128, 0.088, A, A, None,
          None, None, 0, 0, A, 1, 1000 * 4 * 128, 4 * 128, 128, None, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(0, 0) == -1               # q NULL
    assert call(23, 0) == -1              # out NULL
    assert call(5, 0) == -1               # perm NULL
    assert call(23, A + 4) == -3          # misaligned out
    assert call(24, 9) == -1              # bad out dtype
    assert call(26, 4 * 128 + 2) == -3    # out row stride
    assert call(16, 0) == -1              # kv_count NULL
    assert call(13, 80) == -2             # head dim
    assert call(19, A) == -1              # k_g without v_g
    a = list(ok); a[11] = 4097 * 64 - 10; a[12] = 4097 * 64; a[14] = 64
    assert f(*a) == -2                    # nb > 4096


@cpu_only
def test_reorder_kv_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_reorder_kv
    # k, v, x_dt, sb, sn, sh, k_r, v_t, perm, per_head, B, Hh, N, Npad, d, b, stream
    ok = [A, A, 1, 1000 * 4 * 128, 4 * 128, 128, A, A, A, 0, 1, 4, 1000, 1024, 128, 128, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(0, 0) == -1               # k NULL
    assert call(1, 0) == -1               # v NULL
    assert call(7, 0) == -1               # v_t NULL
    assert call(6, A + 8) == -3           # misaligned k_r
    assert call(2, 7) == -1               # bad dtype
    assert call(4, 4 * 128 + 2) == -3     # token stride breaks 16-byte chunks
    assert call(14, 96) == -2             # head dim
    assert call(13, 1000) == -1           # Npad not a multiple of b
    assert call(9, 2) == -1               # perm_per_head


@cpu_only
def test_backward_validation(dbs):
    _, L = dbs
    t = L.lib().dbs_transpose_lists
    assert t(0, A, 1, 2, 16, A, A, None) == -1           # NULL
    assert t(A, A, 1, 2, 4097, A, A, None) == -2         # nb > 4096
    assert t(A + 2, A, 1, 2, 16, A, A, None) == -3       # misaligned
    assert L.lib().dbs_attn_bwd_workspace_bytes(1, 2, 256, 128) == 2 * 256 * 4      # D, one float per row
    assert L.lib().dbs_attn_bwd_workspace_bytes(1, 2, 256, 96) == 0
    f = L.lib().dbs_sparse_attn_bwd
    ws = L.lib().dbs_attn_bwd_workspace_bytes(1, 2, 1024, 128)
    # q, k, v, o, do, lse, B, Hh, N, Npad, d, b, scale, cnt, idx, cntT, idxT, dq, dk, dv, ws, ws_bytes, stream
    ok = [A, A, A, A, A, A, 1, 2, 1000, 1024, 128, 128, 0.088, A, A, A, A, A, A, A, A, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(4, 0) == -1                # do NULL
    assert call(5, 0) == -1                # lse NULL
    assert call(15, 0) == -1               # kvT_count NULL
    assert call(17, A + 8) == -3           # misaligned dq
    assert call(10, 96) == -2              # head dim
    assert call(9, 1000) == -1             # Npad not a multiple of b
    assert call(21, ws - 1) == -1          # small workspace
    assert call(12, float("inf")) == -1    # scale


@cpu_only
def test_mask_rule_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_build_mask_rule
    assert f(A, 1, 1, 16, 7, 0.5, A, A, None, None, None) == -1           # unknown rule
    assert f(A, 1, 1, 16, 0, 1.5, A, A, None, None, None) == -1           # tau > 1
    assert f(A, 1, 1, 16, 1, 0.0, A, A, None, None, None) == -1           # k < 1
    assert f(A, 1, 1, 16, 1, 2.5, A, A, None, None, None) == -1           # k not an integer
    assert f(A, 1, 1, 16, 2, float("nan"), A, A, None, None, None) == -1  # u not finite
    assert f(A, 1, 1, 4097, 2, 1.0, A, A, None, None, None) == -2         # nb > 4096
    assert f(0, 1, 1, 16, 2, 1.0, A, A, None, None, None) == -1           # NULL
    assert f(A, 1, 1, 16, 3, 0.0, A, A, None, None, None) == -1           # expected count must be > 0
    assert f(A, 1, 1, 16, 3, 16.0, A, A, None, None, None) == -1          # ... and < nb


@cpu_only
def test_estimate_mask_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_estimate_mask
    ws = L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 8)
    # q_r, k_r, dt, B, Hh, N, Npad, d, b, k, scale, rule, param, p_imp, kv_count, kv_idx, mask, order, ws, wsb, s
    ok = [A, A, 0, 1, 2, 100, 128, 128, 64, 8, 0.125, 0, 0.9, None, A, A, None, None, A, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(0, 0) == -1               # q NULL
    assert call(14, 0) == -1              # kv_count NULL
    assert call(15, 0) == -1              # kv_idx NULL
    assert call(13, A + 4) == -3          # misaligned p_imp (16 bytes, as dbs_estimate_blocks)
    assert call(17, A + 2) == -3          # misaligned order
    assert call(11, 9) == -1              # unknown rule
    assert call(12, 1.5) == -1            # tau > 1
    ws3 = L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 3)
    assert ws3 == L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 4)   # slots padded to 4
    a = list(ok)
    a[9], a[19] = 3, ws3 - 1              # k = 3 is accepted; the small workspace is not
    assert f(*a) == -1 and "workspace" in L.lib().dbs_last_error().decode()
    assert call(19, ws - 1) == -1         # small workspace
    assert call(10, float("nan")) == -1   # scale
    g = L.lib().dbs_estimate_mask_tok
    okt = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, A, 1, 2, 100, 128, 128, 64, 8, 0.125, 1, 4.0, None, A, A, None,
           None, A, ws, None]
    def callt(i, v):
        a = list(okt)
        a[i] = v
        return g(*a)
    assert callt(5, 0) == -1              # perm NULL
    assert callt(17, 0.5) == -1           # top-k count not an integer >= 1
    assert callt(20, 0) == -1             # kv_idx NULL
    assert callt(24, ws - 1) == -1        # small workspace


@cpu_only
def test_estimate_mask_kvtok_validation(dbs):
    """The estimate with K in token order checks K as it checks Q and asks for the larger workspace
    (the estimator's own plus the gathered sampled K rows), all before any launch."""
    _, L = dbs
    ws = L.lib().dbs_estimate_workspace_bytes(1, 2, 100, 128, 64, 8)
    wk = L.lib().dbs_estimate_kvtok_workspace_bytes(1, 2, 100, 128, 64, 8)
    # nb = 2 blocks of 8 slots: 16 slots padded to 64 rows of 128 bf16 per head, after 256-byte rounding
    assert wk == -(-ws // 256) * 256 + 2 * 64 * 128 * 2
    assert L.lib().dbs_estimate_kvtok_workspace_bytes(1, 2, 100, 96, 64, 8) == 0
    assert L.lib().dbs_estimate_kvtok_workspace_bytes(1, 2, 100, 128, 64, 3) == \
        L.lib().dbs_estimate_kvtok_workspace_bytes(1, 2, 100, 128, 64, 4)       # slots padded to 4
    g = L.lib().dbs_estimate_mask_kvtok
    # q, q_dt, qsb, qsn, qsh, key, key_dt, ksb, ksn, ksh, perm, per_head, B, Hh, N, Npad, d, b, k, scale, rule,
    # param, p_imp, kv_count, kv_idx, mask, order, ws, wsb, stream
    st = 100 * 2 * 128
    ok = [A, 0, st, 2 * 128, 128, A, 0, st, 2 * 128, 128, A, 0, 1, 2, 100, 128, 128, 64, 8, 0.125, 0, 0.9, None, A,
          A, None, None, A, wk, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return g(*a)
    assert call(0, 0) == -1               # q NULL
    assert call(5, 0) == -1               # key NULL
    assert call(10, 0) == -1              # perm NULL
    assert call(5, A + 2) == -3           # misaligned key
    assert call(6, 7) == -1               # bad key dtype
    assert call(8, 2 * 128 + 4) == -3     # key row stride breaks 16-byte rows
    assert call(9, -8) == -1              # negative key stride
    assert call(23, 0) == -1              # kv_count NULL
    assert call(20, 9) == -1              # unknown rule
    assert call(16, 96) == -2             # head dimension
    assert call(28, wk - 1) == -1         # the workspace of the reordered-K call is not enough
    assert "workspace" in L.lib().dbs_last_error().decode()
    assert call(28, ws) == -1


@pytest.mark.parametrize("T,H,W,win,prefix,order", [
    (4, 8, 8, (2, 2, 2), 0, "cuboid"), (5, 7, 9, (2, 3, 2), 0, "gilbert"), (3, 6, 10, (1, 4, 3), 5, "gilbert"),
    (16, 28, 52, (2, 2, 2), 0, "cuboid"), (2, 3, 3, (5, 5, 5), 2, "cuboid")])
def test_prune_anchors_match_oracle(dbs, T, H, W, win, prefix, order):
    from oracle.query_prune import anchors_reordered, window_anchors
    ops, _ = dbs
    perm = o_gilbert(T, H, W, prefix) if order == "gilbert" else o_cuboid(T, H, W, 4, 4, 4, prefix)
    got = ops.prune_anchors(T, H, W, win, perm, prefix)
    want = anchors_reordered(perm, window_anchors(T, H, W, win, prefix))
    assert np.array_equal(got, want)


@cpu_only
def test_prune_validation(dbs):
    ops, L = dbs
    f = L.lib().dbs_prune_anchors
    perm = np.arange(8, dtype=np.int32)
    out = np.empty(8, dtype=np.int32)
    assert f(2, 2, 2, 0, 0, 1, 1, perm.ctypes.data, out.ctypes.data) == -1        # window side 0
    bad = perm.copy(); bad[3] = 2
    assert f(2, 2, 2, 0, 1, 1, 1, bad.ctypes.data, out.ctypes.data) == -1         # not a permutation
    g = L.lib().dbs_query_prune
    # q, q_dt, sb, sn, sh, perm, pph, anchor, B, Hh, N, Npad, d, b, r, q_count, rowsel, keep, stream
    ok = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, A, 1, 2, 100, 128, 128, 64, 0.5, A, A, A, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return g(*a)
    assert call(14, 0.0) == -1            # r = 0
    assert call(14, 1.5) == -1            # r > 1
    assert call(7, 0) == -1               # anchor NULL
    assert call(17, 0) == -1              # keep NULL
    assert call(15, A + 2) == -3          # misaligned q_count
    assert call(13, 32) == -2             # block size
    h = L.lib().dbs_sparse_attn_fwd_pruned_tok
    okh = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, A, A, 1, 2, 100, 128, 128, 64, 0.125, A, A, None, A, A, A, A,
           A, 0, 100 * 2 * 128, 2 * 128, 128, None, None]
    def callh(i, v):
        a = list(okh)
        a[i] = v
        return h(*a)
    assert callh(19, 0) == -1             # q_count NULL
    assert callh(22, 0) == -1             # keep NULL
    assert callh(21, A + 1) == -3         # misaligned anchor
    assert callh(13, 96) == -2            # head dim


@cpu_only
def test_pooled_and_sics_validation(dbs):
    _, L = dbs
    ws = L.lib().dbs_pooled_workspace_bytes(1, 2, 100, 128, 64)
    assert ws == 2 * 1 * 2 * 2 * 3 * 128 * 4
    assert L.lib().dbs_pooled_workspace_bytes(1, 2, 100, 96, 64) == 0
    f = L.lib().dbs_estimate_pooled_tok
    # q, q_dt, sb, sn, sh, perm, pph, k_r, B, Hh, N, Npad, d, b, kind, p_imp, ws, wsb, stream
    ok = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, A, 1, 2, 100, 128, 128, 64, 1, A, A, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(14, 2) == -1              # unknown kind
    assert call(17, ws - 1) == -1         # small workspace
    assert call(15, 0) == -1              # p_imp NULL
    assert call(7, A + 8) == -3           # misaligned k_r
    assert call(12, 32) == -2             # head dim
    g = L.lib().dbs_sics_tok
    okg = [A, 0, 100 * 2 * 128, 2 * 128, 128, A, 0, 1, 2, 100, 128, 128, 64, A, A, None]
    def callg(i, v):
        a = list(okg)
        a[i] = v
        return g(*a)
    assert callg(13, 0) == -1             # sics NULL
    assert callg(14, A + 2) == -3         # misaligned as
    assert callg(12, 96) == -2            # block size


@cpu_only
def test_mask_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_build_mask
    assert f(A, 1, 1, 16, 0.0, A, A, None, None, None) == -1
    assert f(A, 1, 1, 16, 1.5, A, A, None, None, None) == -1
    assert f(A, 1, 1, 16, float("nan"), A, A, None, None, None) == -1
    assert f(A, 1, 1, 5000, 0.9, A, A, None, None, None) == -2
    assert f(0, 1, 1, 16, 0.9, A, A, None, None, None) == -1
    assert f(A + 2, 1, 1, 16, 0.9, A, A, None, None, None) == -3
    assert f(A, 1, 1, 16, 0.9, A, A, None, A + 2, None) == -3      # misaligned order


@cpu_only
def test_attn_and_pool_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_sparse_attn_fwd
    base = [A, A, A, 0, 1, 4, 1000, 1024, 128, 128, 0.088, A, A, None, None, None, 0, 0, A, None, None]
    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, 0) == -1
    assert call(3, 2) == -1               # no such dtype
    a = list(base); a[3] = 1; a[14] = A; a[15] = A; a[16] = 125; a[17] = 8
    assert f(*a) == -2                    # float32 attention takes no global tokens
    assert call(8, 80) == -2
    assert call(14, A) == -1              # k_g without v_g
    a = list(base); a[14] = A; a[15] = A; a[16] = 126; a[17] = 8
    assert f(*a) == -1                    # Ng must be ceil(N / n) = 125
    assert call(10, float("inf")) == -1
    assert call(19, A + 2) == -3
    assert call(13, A + 2) == -3          # misaligned order
    a = list(base); a[6] = 4097 * 64 - 10; a[7] = 4097 * 64; a[9] = 64
    assert f(*a) == -2                    # nb = 4097 > 4096: the list no longer fits LDS
    g = L.lib().dbs_meanpool_kv
    assert g(A, A, 0, 1, 4, 1000, 1024, 128, 128, 0, A, A, None) == -1
    assert g(A, A, 1, 1, 4, 1000, 1024, 128, 128, 8, A, A, None) == -2
    assert g(A, MIS, 0, 1, 4, 1000, 1024, 128, 128, 8, A, A, None) == -3


@cpu_only
def test_inverse_validation(dbs):
    _, L = dbs
    f = L.lib().dbs_inverse_reorder
    assert f(A, 1, A, 0, 0, 1024, 128, A, 0, 1, 8, 100, 128, 128, None) == -2
    assert f(A, 0, A, 0, 0, 1024, 128, 0, 0, 1, 8, 100, 128, 128, None) == -1
    assert f(A, 0, A, 0, 0, 1024, 128, A, 0, 1, 8, 100, 128, 96, None) == -2


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    from dynamic_block_sparse_gilbert_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_normal_quantile_matches_scipy(dbs):
    """The library's AS 241 quantile against scipy's independent implementation (ndtri), from the
    far tails to the centre, and its limits."""
    from scipy.special import ndtri
    ops, _ = dbs
    ps = np.concatenate([np.logspace(-300, -1, 120), np.linspace(0.01, 0.99, 99), 1 - np.logspace(-15, -1, 40),
                         [0.5, 0.075, 0.925, 1 - 16 / 1200, 1 - 16 / 256]])
    got = np.array([ops.normal_quantile(p) for p in ps])
    ref = ndtri(ps)
    assert np.all(np.abs(got - ref) <= 1e-14 * np.maximum(np.abs(ref), 1.0))
    assert ops.normal_quantile(0.5) == 0.0
    assert ops.normal_quantile(0.0) == -np.inf and ops.normal_quantile(1.0) == np.inf
    assert np.isnan(ops.normal_quantile(1.5)) and np.isnan(ops.normal_quantile(-0.1))
    # the symmetry U(1 - p) = -U(p), at dyadic p (1 - p exact)
    for p in (2.0 ** -20, 2.0 ** -7, 0.25, 0.375):
        assert abs(ops.normal_quantile(1 - p) + ops.normal_quantile(p)) < 1e-12
    assert abs(ops.stat_quantile(16, 256) - ndtri(1 - 16 / 256)) < 1e-14


def test_wrappers_reject_bad_index_tensors(dbs, monkeypatch):
    """The binding refuses index operands that the kernels would misread (an int64 permutation is
    read as pairs of int32 words): wrong dtype, non-contiguous, wrong length.  The device check is
    bypassed so that the argument checks run on CPU tensors; nothing reaches the library."""
    import torch
    ops, _ = dbs
    monkeypatch.setattr(ops, "_dev", lambda *a: None)
    called = []
    monkeypatch.setattr(ops, "lib", lambda: called.append(1))
    x = torch.zeros((1, 100, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="int32"):
        ops.reorder(x, torch.arange(100), 128, 64)                      # int64 permutation
    with pytest.raises(ValueError, match="contiguous"):
        ops.reorder(x, torch.arange(200, dtype=torch.int32)[::2], 128, 64)
    with pytest.raises(ValueError, match="trailing dimension"):
        ops.reorder(x, torch.arange(99, dtype=torch.int32), 128, 64)
    with pytest.raises(ValueError, match="rows"):
        ops.reorder(x, torch.zeros((3, 100), dtype=torch.int32), 128, 64)   # per-head rows != heads
    P = torch.zeros((1, 2, 4, 4), dtype=torch.float32)
    with pytest.raises(TypeError, match="int32"):
        ops.build_mask(P, 0.9, kv_count=torch.zeros((1, 2, 4), dtype=torch.int64))
    with pytest.raises(ValueError, match="shape"):
        ops.build_mask(P, 0.9, kv_idx=torch.zeros((1, 2, 4, 3), dtype=torch.int32))
    q = torch.zeros((1, 100, 2, 64), dtype=torch.bfloat16)
    kr = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16)
    vt = torch.zeros((1, 2, 2, 64, 64), dtype=torch.bfloat16)
    cnt = torch.zeros((1, 2, 2), dtype=torch.int32)
    idx = torch.zeros((1, 2, 2, 2), dtype=torch.int32)
    with pytest.raises(TypeError, match="int32"):
        ops.sparse_attn_fwd_tok(q, torch.arange(100), kr, vt, 100, 64, 0.125, cnt, idx)
    with pytest.raises(TypeError, match="int32"):
        ops.sparse_attn_fwd_tok(q, torch.arange(100, dtype=torch.int32), kr, vt, 100, 64, 0.125, cnt.long(), idx)
    with pytest.raises(TypeError, match="int32"):
        ops.sics_choose(q, None, torch.zeros((2, 100), dtype=torch.int64), 128, 64)
    assert not called
