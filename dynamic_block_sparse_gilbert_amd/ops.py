"""Python binding of the C ABI: one wrapper per entry point, same names.

The wrappers only marshal arguments: they read data_ptr(), strides and the
current HIP stream from torch tensors, allocate outputs with torch when the
caller does not pass them, and call the library.  Every step of the
computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from ._lib import DBS_BF16, DBS_FP32, DBS_ROWS, DBS_TILES_T, check, lib

_DT = {torch.bfloat16: DBS_BF16, torch.float32: DBS_FP32}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("device tensors required")


def _i32(t: Optional[torch.Tensor], name: str, last: Optional[int] = None, lead: Optional[tuple] = None) -> None:
    """An index operand must be a contiguous int32 tensor (an int64 tensor would be read as pairs of
    int32 words), with the given trailing dimension and leading dimensions when stated."""
    if t is None:
        return
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be torch.int32 (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if last is not None and (t.dim() == 0 or t.shape[-1] != last):
        raise ValueError(f"{name} must have trailing dimension {last} (got shape {tuple(t.shape)})")
    if lead is not None and tuple(t.shape[:-1]) != tuple(lead):
        raise ValueError(f"{name} must have shape {tuple(lead) + (last,)} (got {tuple(t.shape)})")


def _perm(perm: torch.Tensor, N: int, Hh: int, name: str = "perm") -> int:
    """Checks a device permutation [N] or [Hh, N]; returns perm_per_head."""
    _i32(perm, name, N)
    if perm.dim() == 2:
        if perm.shape[0] != Hh:
            raise ValueError(f"{name} has {perm.shape[0]} rows for {Hh} heads")
        return 1
    if perm.dim() != 1:
        raise ValueError(f"{name} must be [N] or [Hh, N]")
    return 0


def _lists(kv_count: Optional[torch.Tensor], kv_idx: Optional[torch.Tensor], B: int, Hh: int, nb: int) -> None:
    _i32(kv_count, "kv_count", nb, (B, Hh))
    _i32(kv_idx, "kv_idx", nb, (B, Hh, nb))


def _stream() -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t: Optional[torch.Tensor]) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


# ---------------------------------------------------------------------------- host


def perm_gilbert3d(T: int, H: int, W: int, prefix: int = 0) -> np.ndarray:
    out = np.empty(prefix + T * H * W, dtype=np.int32)
    check("dbs_perm_gilbert3d", lib().dbs_perm_gilbert3d(T, H, W, prefix, out.ctypes.data))
    return out


def perm_cuboid(T: int, H: int, W: int, ct: int, ch: int, cw: int, prefix: int = 0) -> np.ndarray:
    out = np.empty(prefix + T * H * W, dtype=np.int32)
    check("dbs_perm_cuboid", lib().dbs_perm_cuboid(T, H, W, ct, ch, cw, prefix, out.ctypes.data))
    return out


def perm_invert(perm: np.ndarray) -> np.ndarray:
    p = np.ascontiguousarray(perm, dtype=np.int32)
    out = np.empty_like(p)
    check("dbs_perm_invert", lib().dbs_perm_invert(p.ctypes.data, p.size, out.ctypes.data))
    return out


def prune_anchors(T: int, H: int, W: int, win, perm: np.ndarray, prefix: int = 0) -> np.ndarray:
    """Reordered index of the window centre of every reordered token (query pruning)."""
    p = np.ascontiguousarray(perm, dtype=np.int32)
    out = np.empty_like(p)
    check("dbs_prune_anchors", lib().dbs_prune_anchors(T, H, W, prefix, int(win[0]), int(win[1]), int(win[2]),
                                                       p.ctypes.data, out.ctypes.data))
    return out


# --------------------------------------------------------------------------- device


def reorder(x: torch.Tensor, perm: torch.Tensor, Npad: int, b: int, layout: str = "rows",
            out_dtype: torch.dtype = torch.bfloat16, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B, N, Hh, d] (any strides, d contiguous) -> y rows [B, Hh, Npad, d] or tiles [B, Hh, Npad/b, d, b]."""
    _dev(x, perm)
    B, N, Hh, d = x.shape
    if x.stride(3) != 1:
        raise ValueError("the d axis of x must be contiguous")
    lay = {"rows": DBS_ROWS, "tiles_t": DBS_TILES_T}[layout]
    if y is None:
        shape = (B, Hh, Npad, d) if lay == DBS_ROWS else (B, Hh, Npad // b, d, b)
        y = torch.empty(shape, dtype=out_dtype, device=x.device)
    per_head = _perm(perm, N, Hh)
    check("dbs_reorder", lib().dbs_reorder(
        _p(x), _dt(x), x.stride(0), x.stride(1), x.stride(2), _p(y), _dt(y), lay, _p(perm), per_head,
        B, Hh, N, Npad, d, b, _stream()))
    return y


def reorder_kv(k: torch.Tensor, v: torch.Tensor, perm: torch.Tensor, Npad: int, b: int,
               k_r: Optional[torch.Tensor] = None, v_t: Optional[torch.Tensor] = None, n_pool: int = 0,
               k_g: Optional[torch.Tensor] = None, v_g: Optional[torch.Tensor] = None):
    """k, v [B, N, Hh, d] (same strides, d contiguous) -> k_r rows [B, Hh, Npad, d] and v_t tiles
    [B, Hh, Npad/b, d, b], both bf16, in one launch.  With n_pool > 0 also the ASA_G global tokens
    (dbs_reorder_kv_pool): returns (k_r, v_t, k_g, v_g), k_g / v_g as meanpool_kv's."""
    _dev(k, v, perm, k_r, v_t, k_g, v_g)
    B, N, Hh, d = k.shape
    if v.shape != k.shape or v.stride() != k.stride() or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape, strides and dtype")
    if k.stride(3) != 1:
        raise ValueError("the d axis of k and v must be contiguous")
    if k_r is None:
        k_r = torch.empty((B, Hh, Npad, d), dtype=torch.bfloat16, device=k.device)
    if v_t is None:
        v_t = torch.empty((B, Hh, Npad // b, d, b), dtype=torch.bfloat16, device=k.device)
    if k_r.shape != (B, Hh, Npad, d) or v_t.shape != (B, Hh, Npad // b, d, b):
        raise ValueError("k_r / v_t have the wrong shape")
    if k_r.dtype != torch.bfloat16 or v_t.dtype != torch.bfloat16 or not (k_r.is_contiguous() and v_t.is_contiguous()):
        raise ValueError("k_r and v_t must be contiguous bf16")
    per_head = _perm(perm, N, Hh)
    if n_pool:
        Ng = -(-N // n_pool)
        Ngpad = -(-Ng // b) * b
        if k_g is None:
            k_g = torch.empty((B, Hh, Ngpad, d), dtype=torch.bfloat16, device=k.device)
        if v_g is None:
            v_g = torch.empty((B, Hh, Ngpad // b, d, b), dtype=torch.bfloat16, device=k.device)
        check("dbs_reorder_kv_pool", lib().dbs_reorder_kv_pool(
            _p(k), _p(v), _dt(k), k.stride(0), k.stride(1), k.stride(2), _p(k_r), _p(v_t), _p(perm), per_head,
            B, Hh, N, Npad, d, b, int(n_pool), _p(k_g), _p(v_g), _stream()))
        return k_r, v_t, k_g, v_g
    check("dbs_reorder_kv", lib().dbs_reorder_kv(
        _p(k), _p(v), _dt(k), k.stride(0), k.stride(1), k.stride(2), _p(k_r), _p(v_t), _p(perm), per_head,
        B, Hh, N, Npad, d, b, _stream()))
    return k_r, v_t


def inverse_reorder(y: torch.Tensor, perm: torch.Tensor, N: int,
                    out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """y rows [B, Hh, Npad, d] bf16 -> out [B, N, Hh, d] (out may be a strided view)."""
    _dev(y, perm, out)
    B, Hh, Npad, d = y.shape
    if out is None:
        out = torch.empty((B, N, Hh, d), dtype=out_dtype, device=y.device)
    if out.stride(3) != 1:
        raise ValueError("the d axis of out must be contiguous")
    per_head = _perm(perm, N, Hh)
    check("dbs_inverse_reorder", lib().dbs_inverse_reorder(
        _p(y), _dt(y), _p(out), _dt(out), out.stride(0), out.stride(1), out.stride(2), _p(perm), per_head,
        B, Hh, N, Npad, d, _stream()))
    return out


def estimate_workspace_bytes(B: int, Hh: int, N: int, d: int, b: int, k: int) -> int:
    return int(lib().dbs_estimate_workspace_bytes(B, Hh, N, d, b, k))


def estimate_blocks(q_r: torch.Tensor, k_r: torch.Tensor, N: int, b: int, k: int, scale: float,
                    p_imp: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_r, k_r rows [B, Hh, Npad, d] -> p_imp float32 [B, Hh, nb, nb]."""
    _dev(q_r, k_r, p_imp, workspace)
    B, Hh, Npad, d = q_r.shape
    nb = Npad // b
    if q_r.dtype != k_r.dtype:
        raise TypeError("q_r and k_r must have one dtype (it selects the compute path)")
    if p_imp is None:
        p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=q_r.device)
    need = estimate_workspace_bytes(B, Hh, N, d, b, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_r.device)
    check("dbs_estimate_blocks", lib().dbs_estimate_blocks(
        _p(q_r), _p(k_r), _dt(q_r), B, Hh, N, Npad, d, b, k, float(scale), _p(p_imp), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return p_imp


def estimate_blocks_tok(q: torch.Tensor, perm: torch.Tensor, k_r: torch.Tensor, N: int, b: int, k: int,
                        scale: float, p_imp: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q [B, N, Hh, d] in token order (any strides, d contiguous), k_r rows [B, Hh, Npad, d] ->
    p_imp float32 [B, Hh, nb, nb]; equal to estimate_blocks on the reordered Q."""
    _dev(q, perm, k_r, p_imp, workspace)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, Hh, Npad, d = k_r.shape
    nb = Npad // b
    if p_imp is None:
        p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=k_r.device)
    need = estimate_workspace_bytes(B, Hh, N, d, b, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k_r.device)
    per_head = _perm(perm, N, Hh)
    check("dbs_estimate_blocks_tok", lib().dbs_estimate_blocks_tok(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perm), per_head, _p(k_r),
        B, Hh, N, Npad, d, b, k, float(scale), _p(p_imp), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return p_imp


def build_mask(p_imp: torch.Tensor, tau: float, kv_count: Optional[torch.Tensor] = None,
               kv_idx: Optional[torch.Tensor] = None, want_mask: bool = False,
               mask: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
               want_order: bool = False):
    """p_imp [B, Hh, nb, nb] float32 -> (kv_count [B, Hh, nb], kv_idx [B, Hh, nb, nb], mask or None);
    with want_order (or an `order` buffer) also the attention work order int32 [B * Hh * nb] as a
    fourth element."""
    _dev(p_imp, kv_count, kv_idx, mask, order)
    B, Hh, nb, _ = p_imp.shape
    _lists(kv_count, kv_idx, B, Hh, nb)
    _i32(order, "order", B * Hh * nb, ())
    if kv_count is None:
        kv_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=p_imp.device)
    if kv_idx is None:
        kv_idx = torch.empty((B, Hh, nb, nb), dtype=torch.int32, device=p_imp.device)
    if want_mask and mask is None:
        mask = torch.empty((B, Hh, nb, nb), dtype=torch.uint8, device=p_imp.device)
    if want_order and order is None:
        order = torch.empty((B * Hh * nb,), dtype=torch.int32, device=p_imp.device)
    check("dbs_build_mask", lib().dbs_build_mask(
        _p(p_imp), B, Hh, nb, float(tau), _p(kv_count), _p(kv_idx), _p(mask), _p(order), _stream()))
    if order is not None:
        return kv_count, kv_idx, mask, order
    return kv_count, kv_idx, mask


MASK_RULES = {"cumulative": 0, "topk": 1, "stat": 2, "stat_k": 3}


def normal_quantile(p: float) -> float:
    """The library's standard normal quantile U(p) (dbs_normal_quantile)."""
    return float(lib().dbs_normal_quantile(float(p)))


def stat_quantile(k: float, n: int) -> float:
    """u = U(1 - k/n), the quantile the statistical rule uses to keep about k of n blocks on normally
    spread scores, from the library (rule 'stat_k' lets the library compute it itself)."""
    if not 0 < k < n:
        raise ValueError("need 0 < k < n")
    return normal_quantile(1.0 - k / n)


def build_mask_rule(p_imp: torch.Tensor, rule: str, param: float, kv_count: Optional[torch.Tensor] = None,
                    kv_idx: Optional[torch.Tensor] = None, want_mask: bool = False,
                    order: Optional[torch.Tensor] = None):
    """Kept-block lists under `rule`: 'cumulative' (param = tau), 'topk' (param = k) or 'stat'
    (param = u, see stat_quantile).  Returns (kv_count, kv_idx, mask or None)."""
    _dev(p_imp, kv_count, kv_idx, order)
    B, Hh, nb, _ = p_imp.shape
    _lists(kv_count, kv_idx, B, Hh, nb)
    _i32(order, "order", B * Hh * nb, ())
    if kv_count is None:
        kv_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=p_imp.device)
    if kv_idx is None:
        kv_idx = torch.empty((B, Hh, nb, nb), dtype=torch.int32, device=p_imp.device)
    mask = torch.empty((B, Hh, nb, nb), dtype=torch.uint8, device=p_imp.device) if want_mask else None
    check("dbs_build_mask_rule", lib().dbs_build_mask_rule(
        _p(p_imp), B, Hh, nb, MASK_RULES[rule], float(param), _p(kv_count), _p(kv_idx), _p(mask), _p(order),
        _stream()))
    return kv_count, kv_idx, mask


def estimate_mask(q_r: torch.Tensor, k_r: torch.Tensor, N: int, b: int, k: int, scale: float, rule: str,
                  param: float, q_perm: Optional[torch.Tensor] = None, want_p_imp: bool = False,
                  want_mask: bool = False, kv_count: Optional[torch.Tensor] = None,
                  kv_idx: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, p_imp: Optional[torch.Tensor] = None):
    """The estimate and the block selection in one call (dbs_estimate_mask, or with q_perm
    dbs_estimate_mask_tok: q is then [B, N, Hh, d] in token order).  k_r rows [B, Hh, Npad, d].
    Returns (kv_count, kv_idx, mask or None, p_imp or None); P_imp is written when want_p_imp or a
    p_imp buffer is given."""
    _dev(q_r, q_perm, k_r, kv_count, kv_idx, order, workspace, p_imp)
    B, Hh, Npad, d = k_r.shape
    nb = Npad // b
    dv = k_r.device
    _lists(kv_count, kv_idx, B, Hh, nb)
    _i32(order, "order", B * Hh * nb, ())
    if kv_count is None:
        kv_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=dv)
    if kv_idx is None:
        kv_idx = torch.empty((B, Hh, nb, nb), dtype=torch.int32, device=dv)
    mask = torch.empty((B, Hh, nb, nb), dtype=torch.uint8, device=dv) if want_mask else None
    if p_imp is None and want_p_imp:
        p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=dv)
    need = estimate_workspace_bytes(B, Hh, N, d, b, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dv)
    wsb = workspace.numel() * workspace.element_size()
    tail = (b, k, float(scale), MASK_RULES[rule], float(param), _p(p_imp), _p(kv_count), _p(kv_idx), _p(mask),
            _p(order), _p(workspace), wsb, _stream())
    if q_perm is None:
        if q_r.dtype != k_r.dtype:
            raise TypeError("q_r and k_r must have one dtype (it selects the compute path)")
        check("dbs_estimate_mask", lib().dbs_estimate_mask(_p(q_r), _p(k_r), _dt(q_r), B, Hh, N, Npad, d, *tail))
    else:
        if q_r.stride(3) != 1:
            raise ValueError("the d axis of q must be contiguous")
        per_head = _perm(q_perm, N, Hh, "q_perm")
        check("dbs_estimate_mask_tok", lib().dbs_estimate_mask_tok(
            _p(q_r), _dt(q_r), q_r.stride(0), q_r.stride(1), q_r.stride(2), _p(q_perm), per_head, _p(k_r),
            B, Hh, N, Npad, d, *tail))
    return kv_count, kv_idx, mask, p_imp


def estimate_kvtok_workspace_bytes(B: int, Hh: int, N: int, d: int, b: int, k: int) -> int:
    return int(lib().dbs_estimate_kvtok_workspace_bytes(B, Hh, N, d, b, k))


def estimate_mask_kvtok(q: torch.Tensor, key: torch.Tensor, perm: torch.Tensor, b: int, k: int, scale: float,
                        rule: str, param: float, want_p_imp: bool = False, want_mask: bool = False,
                        kv_count: Optional[torch.Tensor] = None, kv_idx: Optional[torch.Tensor] = None,
                        order: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        p_imp: Optional[torch.Tensor] = None):
    """dbs_estimate_mask_kvtok: the estimate and the block selection with Q and K both in token
    order ([B, N, Hh, d], d contiguous), so no reordered K is needed.  Returns (kv_count, kv_idx,
    mask or None, p_imp or None), as estimate_mask."""
    _dev(q, key, perm, kv_count, kv_idx, order, workspace, p_imp)
    B, N, Hh, d = q.shape
    if key.shape != q.shape:
        raise ValueError("q and key must have one shape")
    if q.stride(3) != 1 or key.stride(3) != 1:
        raise ValueError("the d axis of q and key must be contiguous")
    Npad = -(-N // b) * b
    nb = Npad // b
    dv = q.device
    _lists(kv_count, kv_idx, B, Hh, nb)
    _i32(order, "order", B * Hh * nb, ())
    per_head = _perm(perm, N, Hh)
    if kv_count is None:
        kv_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=dv)
    if kv_idx is None:
        kv_idx = torch.empty((B, Hh, nb, nb), dtype=torch.int32, device=dv)
    mask = torch.empty((B, Hh, nb, nb), dtype=torch.uint8, device=dv) if want_mask else None
    if p_imp is None and want_p_imp:
        p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=dv)
    need = estimate_kvtok_workspace_bytes(B, Hh, N, d, b, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dv)
    wsb = workspace.numel() * workspace.element_size()
    check("dbs_estimate_mask_kvtok", lib().dbs_estimate_mask_kvtok(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(key), _dt(key), key.stride(0), key.stride(1),
        key.stride(2), _p(perm), per_head, B, Hh, N, Npad, d, b, k, float(scale), MASK_RULES[rule], float(param),
        _p(p_imp), _p(kv_count), _p(kv_idx), _p(mask), _p(order), _p(workspace), wsb, _stream()))
    return kv_count, kv_idx, mask, p_imp


NOALLOC_SCRATCH_BYTES = 128 << 20     # DBS_NOALLOC_SCRATCH_BYTES


def estimate_mask_noalloc(q: torch.Tensor, q_perm: torch.Tensor, k_r: torch.Tensor, N: int, b: int, k: int,
                          scale: float, rule: str, param: float, kv_count: torch.Tensor, kv_idx: torch.Tensor,
                          order: Optional[torch.Tensor] = None, p_imp: Optional[torch.Tensor] = None,
                          mask: Optional[torch.Tensor] = None):
    """estimate_mask with q in token order [B, N, Hh, d] and no workspace (dbs_estimate_mask_tok_noalloc):
    the library's static scratch holds the intermediate results and nothing is allocated, here or
    in the library; the caller brings every output.  Returns (kv_count, kv_idx, mask, p_imp)."""
    _dev(q, q_perm, k_r, kv_count, kv_idx, order, p_imp, mask)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, Hh, Npad, d = k_r.shape
    nb = Npad // b
    _lists(kv_count, kv_idx, B, Hh, nb)
    _i32(order, "order", B * Hh * nb, ())
    for t, name in ((p_imp, "p_imp"), (mask, "mask")):
        if t is not None and (tuple(t.shape) != (B, Hh, nb, nb) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [{B}, {Hh}, {nb}, {nb}] tensor")
    if p_imp is not None and p_imp.dtype != torch.float32:
        raise TypeError("p_imp must be float32")
    if mask is not None and mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8")
    per_head = _perm(q_perm, N, Hh, "q_perm")
    check("dbs_estimate_mask_tok_noalloc", lib().dbs_estimate_mask_tok_noalloc(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(q_perm), per_head, _p(k_r),
        B, Hh, N, Npad, d, b, k, float(scale), MASK_RULES[rule], float(param), _p(p_imp), _p(kv_count),
        _p(kv_idx), _p(mask), _p(order), _stream()))
    return kv_count, kv_idx, mask, p_imp


def query_prune(q: torch.Tensor, perm: torch.Tensor, anchor: torch.Tensor, Npad: int, b: int, r: float,
                q_count: Optional[torch.Tensor] = None, rowsel: Optional[torch.Tensor] = None,
                keep: Optional[torch.Tensor] = None):
    """q [B, N, Hh, d] in token order -> (q_count [B, Hh, nb], rowsel [B, Hh, nb, b], keep [B, Hh, Npad])."""
    _dev(q, perm, anchor, q_count, rowsel, keep)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, N, Hh, d = q.shape
    nb = Npad // b
    dv = q.device
    if q_count is None:
        q_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=dv)
    if rowsel is None:
        rowsel = torch.empty((B, Hh, nb, b), dtype=torch.int32, device=dv)
    if keep is None:
        keep = torch.empty((B, Hh, Npad), dtype=torch.uint8, device=dv)
    per_head = _perm(perm, N, Hh)
    _perm(anchor, N, Hh, "anchor")
    check("dbs_query_prune", lib().dbs_query_prune(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perm), per_head, _p(anchor), B, Hh, N, Npad, d, b,
        float(r), _p(q_count), _p(rowsel), _p(keep), _stream()))
    return q_count, rowsel, keep


def sparse_attn_fwd_pruned_tok(q: torch.Tensor, perm: torch.Tensor, k_r: torch.Tensor, v_t: torch.Tensor, N: int,
                               b: int, scale: float, kv_count: torch.Tensor, kv_idx: torch.Tensor,
                               q_count: torch.Tensor, rowsel: torch.Tensor, anchor: torch.Tensor,
                               keep: torch.Tensor, out: Optional[torch.Tensor] = None,
                               out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
                               want_lse: bool = False, order: Optional[torch.Tensor] = None):
    """Attention for the kept query rows, then token filling; returns (out [B, N, Hh, d], lse or None)."""
    _dev(q, perm, k_r, v_t, kv_count, kv_idx, q_count, rowsel, anchor, keep, out, lse, order)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, Hh, Npad, d = k_r.shape
    if out is None:
        out = torch.empty((B, N, Hh, d), dtype=out_dtype, device=k_r.device)
    if out.stride(3) != 1:
        raise ValueError("the d axis of out must be contiguous")
    if want_lse and lse is None:
        lse = torch.empty((B, Hh, Npad), dtype=torch.float32, device=k_r.device)
    per_head = _perm(perm, N, Hh)
    _perm(anchor, N, Hh, "anchor")
    _lists(kv_count, kv_idx, B, Hh, Npad // b)
    _i32(order, "order", B * Hh * (Npad // b), ())
    _i32(q_count, "q_count", Npad // b, (B, Hh))
    _i32(rowsel, "rowsel", b, (B, Hh, Npad // b))
    check("dbs_sparse_attn_fwd_pruned_tok", lib().dbs_sparse_attn_fwd_pruned_tok(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perm), per_head, _p(k_r), _p(v_t),
        B, Hh, N, Npad, d, b, float(scale), _p(kv_count), _p(kv_idx), _p(order), _p(q_count), _p(rowsel),
        _p(anchor), _p(keep), _p(out), _dt(out), out.stride(0), out.stride(1), out.stride(2), _p(lse), _stream()))
    return out, lse


POOL_KINDS = {"mean": 0, "trip": 1}


def estimate_pooled(q: torch.Tensor, perm: torch.Tensor, k_r: torch.Tensor, N: int, b: int, kind: str,
                    p_imp: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pooled block estimate (kind 'mean' or 'trip'): q [B, N, Hh, d] token order, k_r rows ->
    p_imp float32 [B, Hh, nb, nb]."""
    _dev(q, perm, k_r, p_imp, workspace)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, Hh, Npad, d = k_r.shape
    nb = Npad // b
    if p_imp is None:
        p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=k_r.device)
    need = lib().dbs_pooled_workspace_bytes(B, Hh, N, d, b)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k_r.device)
    per_head = _perm(perm, N, Hh)
    check("dbs_estimate_pooled_tok", lib().dbs_estimate_pooled_tok(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perm), per_head, _p(k_r), B, Hh, N, Npad, d, b,
        POOL_KINDS[kind], _p(p_imp), _p(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return p_imp


def sics(q: torch.Tensor, perm: torch.Tensor, Npad: int, b: int):
    """SICS of every block of the reordering perm and each head's aggregation score:
    q [B, N, Hh, d] token order -> (sics [B, Hh, nb], as [B, Hh]) float32."""
    _dev(q, perm)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, N, Hh, d = q.shape
    nb = Npad // b
    out = torch.empty((B, Hh, nb), dtype=torch.float32, device=q.device)
    agg = torch.empty((B, Hh), dtype=torch.float32, device=q.device)
    per_head = _perm(perm, N, Hh)
    check("dbs_sics_tok", lib().dbs_sics_tok(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perm), per_head, B, Hh, N, Npad, d, b, _p(out),
        _p(agg), _stream()))
    return out, agg


def sics_choose(q: torch.Tensor, k: Optional[torch.Tensor], perms: torch.Tensor, Npad: int, b: int,
                block_scores: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                choice: Optional[torch.Tensor] = None):
    """SPADE scheme choice in one call (dbs_sics_choose): q, k [B, N, Hh, d] token order (k may be
    None: Q alone), perms int32 [n_cand, N] candidate orders.  Returns (choice int32 [B, Hh],
    scores float32 [n_cand, B, Hh], block_scores float32 [n_cand, T, B, Hh, nb])."""
    _dev(q, k, perms, block_scores, scores, choice)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, N, Hh, d = q.shape
    if k is not None and (k.shape != q.shape or k.stride() != q.stride() or k.dtype != q.dtype):
        raise ValueError("k must have q's shape, strides and dtype")
    if perms.dim() != 2:
        raise ValueError("perms must be [n_cand, N]")
    _i32(perms, "perms", N)
    nc = perms.shape[0]
    nb = Npad // b
    T = 1 if k is None else 2
    dv = q.device
    if block_scores is None:
        block_scores = torch.empty((nc, T, B, Hh, nb), dtype=torch.float32, device=dv)
    if scores is None:
        scores = torch.empty((nc, B, Hh), dtype=torch.float32, device=dv)
    if choice is None:
        choice = torch.empty((B, Hh), dtype=torch.int32, device=dv)
    if block_scores.numel() < nc * T * B * Hh * nb or scores.numel() < nc * B * Hh or choice.numel() < B * Hh:
        raise ValueError("output buffers too small")
    _i32(choice, "choice")
    check("dbs_sics_choose", lib().dbs_sics_choose(
        _p(q), _p(k), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perms), nc, B, Hh, N, Npad, d, b,
        _p(block_scores), _p(scores), _p(choice), _stream()))
    return choice, scores, block_scores


def meanpool_kv(k_r: torch.Tensor, v_t: torch.Tensor, N: int, b: int, n: int,
                k_g: Optional[torch.Tensor] = None, v_g: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, int]:
    """k_r rows, v_t tiles -> (k_g rows [B,Hh,Ngpad,d], v_g tiles [B,Hh,Ngpad/b,d,b], Ng)."""
    _dev(k_r, v_t, k_g, v_g)
    B, Hh, Npad, d = k_r.shape
    Ng = -(-N // n)
    Ngpad = -(-Ng // b) * b
    if k_g is None:
        k_g = torch.empty((B, Hh, Ngpad, d), dtype=torch.bfloat16, device=k_r.device)
    if v_g is None:
        v_g = torch.empty((B, Hh, Ngpad // b, d, b), dtype=torch.bfloat16, device=k_r.device)
    check("dbs_meanpool_kv", lib().dbs_meanpool_kv(
        _p(k_r), _p(v_t), _dt(k_r), B, Hh, N, Npad, d, b, n, _p(k_g), _p(v_g), _stream()))
    return k_g, v_g, Ng


def sparse_attn_fwd(q_r: torch.Tensor, k_r: torch.Tensor, v_t: torch.Tensor, N: int, b: int, scale: float,
                    kv_count: torch.Tensor, kv_idx: torch.Tensor,
                    k_g: Optional[torch.Tensor] = None, v_g: Optional[torch.Tensor] = None,
                    Ng: int = 0, n_pool: int = 0, o_r: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                    order: Optional[torch.Tensor] = None):
    """Returns (o_r rows [B, Hh, Npad, d] bf16, lse float32 [B, Hh, Npad] or None).  `order` is the
    work order from build_mask (None: index order)."""
    _dev(q_r, k_r, v_t, kv_count, kv_idx, k_g, v_g, o_r, lse, order)
    B, Hh, Npad, d = q_r.shape
    _lists(kv_count, kv_idx, B, Hh, Npad // b)
    _i32(order, "order", B * Hh * (Npad // b), ())
    if q_r.dtype == torch.float32 and (k_r.dtype != torch.float32 or v_t.dtype != torch.float32
                                       or v_t.shape != q_r.shape):
        raise TypeError("float32 attention takes float32 rows for q_r, k_r and v (v as rows [B, Hh, Npad, d])")
    if o_r is None:
        o_r = torch.empty_like(q_r)
    if want_lse and lse is None:
        lse = torch.empty((B, Hh, Npad), dtype=torch.float32, device=q_r.device)
    check("dbs_sparse_attn_fwd", lib().dbs_sparse_attn_fwd(
        _p(q_r), _p(k_r), _p(v_t), _dt(q_r), B, Hh, N, Npad, d, b, float(scale), _p(kv_count), _p(kv_idx),
        _p(order), _p(k_g), _p(v_g), int(Ng), int(n_pool), _p(o_r), _p(lse), _stream()))
    return o_r, lse


def sparse_attn_fwd_tok(q: torch.Tensor, perm: torch.Tensor, k_r: torch.Tensor, v_t: torch.Tensor, N: int,
                        b: int, scale: float, kv_count: torch.Tensor, kv_idx: torch.Tensor,
                        k_g: Optional[torch.Tensor] = None, v_g: Optional[torch.Tensor] = None,
                        Ng: int = 0, n_pool: int = 0, out: Optional[torch.Tensor] = None,
                        out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
                        want_lse: bool = False, order: Optional[torch.Tensor] = None):
    """Q [B, N, Hh, d] in token order -> (out [B, N, Hh, d] in token order, lse [B, Hh, Npad] or None);
    equal to inverse_reorder(sparse_attn_fwd(reordered Q)) bit for bit.  out may be a strided view."""
    _dev(q, perm, k_r, v_t, kv_count, kv_idx, k_g, v_g, out, lse, order)
    if q.stride(3) != 1:
        raise ValueError("the d axis of q must be contiguous")
    B, Hh, Npad, d = k_r.shape
    if out is None:
        out = torch.empty((B, N, Hh, d), dtype=out_dtype, device=k_r.device)
    if out.stride(3) != 1:
        raise ValueError("the d axis of out must be contiguous")
    if want_lse and lse is None:
        lse = torch.empty((B, Hh, Npad), dtype=torch.float32, device=k_r.device)
    per_head = _perm(perm, N, Hh)
    _lists(kv_count, kv_idx, B, Hh, Npad // b)
    _i32(order, "order", B * Hh * (Npad // b), ())
    check("dbs_sparse_attn_fwd_tok", lib().dbs_sparse_attn_fwd_tok(
        _p(q), _dt(q), q.stride(0), q.stride(1), q.stride(2), _p(perm), per_head, _p(k_r), _p(v_t),
        B, Hh, N, Npad, d, b, float(scale), _p(kv_count), _p(kv_idx), _p(order), _p(k_g), _p(v_g),
        int(Ng), int(n_pool), _p(out), _dt(out), out.stride(0), out.stride(1), out.stride(2), _p(lse),
        _stream()))
    return out, lse


# --------------------------------------------------------------------------- backward


def transpose_lists(kv_count: torch.Tensor, kv_idx: torch.Tensor):
    """Key-to-query lists: (kvT_count [B, Hh, nb], kvT_idx [B, Hh, nb, nb]) int32; row J lists, ascending,
    the query blocks whose kept list holds J (entries past kvT_count unspecified)."""
    _dev(kv_count, kv_idx)
    B, Hh, nb = kv_count.shape
    _lists(kv_count, kv_idx, B, Hh, nb)
    kvT_count = torch.empty_like(kv_count)
    kvT_idx = torch.empty_like(kv_idx)
    check("dbs_transpose_lists", lib().dbs_transpose_lists(
        _p(kv_count), _p(kv_idx), B, Hh, nb, _p(kvT_count), _p(kvT_idx), _stream()))
    return kvT_count, kvT_idx


def attn_bwd_workspace_bytes(B: int, Hh: int, Npad: int, d: int) -> int:
    return int(lib().dbs_attn_bwd_workspace_bytes(B, Hh, Npad, d))


def sparse_attn_bwd(q_r: torch.Tensor, k_r: torch.Tensor, v_r: torch.Tensor, o_r: torch.Tensor,
                    do_r: torch.Tensor, lse: torch.Tensor, N: int, b: int, scale: float,
                    kv_count: torch.Tensor, kv_idx: torch.Tensor,
                    kvT_count: Optional[torch.Tensor] = None, kvT_idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Gradients of sparse_attn_fwd (no global tokens).  q_r, k_r, v_r (V in rows layout), o_r, do_r:
    rows [B, Hh, Npad, d] bf16; lse from the forward.  Returns (dq, dk, dv) float32 rows."""
    _dev(q_r, k_r, v_r, o_r, do_r, lse, kv_count, kv_idx, kvT_count, kvT_idx, workspace)
    B, Hh, Npad, d = q_r.shape
    _lists(kv_count, kv_idx, B, Hh, Npad // b)
    _lists(kvT_count, kvT_idx, B, Hh, Npad // b)
    for t in (k_r, v_r, o_r, do_r):
        if t.shape != q_r.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("q_r, k_r, v_r, o_r, do_r must be contiguous bf16 rows of one shape")
    if kvT_count is None or kvT_idx is None:
        kvT_count, kvT_idx = transpose_lists(kv_count, kv_idx)
    need = attn_bwd_workspace_bytes(B, Hh, Npad, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_r.device)
    dq = torch.empty((B, Hh, Npad, d), dtype=torch.float32, device=q_r.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    check("dbs_sparse_attn_bwd", lib().dbs_sparse_attn_bwd(
        _p(q_r), _p(k_r), _p(v_r), _p(o_r), _p(do_r), _p(lse), B, Hh, N, Npad, d, b, float(scale),
        _p(kv_count), _p(kv_idx), _p(kvT_count), _p(kvT_idx), _p(dq), _p(dk), _p(dv), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return dq, dk, dv
