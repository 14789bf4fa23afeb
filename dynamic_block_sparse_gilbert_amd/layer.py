"""One ASA / ASA_G attention layer on the GPU, composed from the C-ABI calls.

Video-BLADE: "Preprocessing" (reorder), "Step 1" (estimate), "Step 2.1"
(mask), "Step 2.2" (block-sparse attention, optional global tokens), then the
output goes back to token order.  K and V are reordered into the curve-order
layouts the attention streams; Q is read in token order through the
permutation by the estimator and the attention, which also writes the output
straight to token order (dbs_estimate_blocks_tok, dbs_sparse_attn_fwd_tok),
so neither Q nor the output makes an extra pass through HBM.  Buffers are
allocated once per shape and reused; permutations are built on the host by
the library and uploaded once.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import ops


@dataclass
class LayerSpec:
    T: int
    H: int
    W: int
    heads: int
    d: int
    b: int = 128
    k: int = 16
    tau: float = 0.9
    prefix: int = 0                     # text tokens before the video tokens (identity order)
    order: str = "gilbert"              # "gilbert", "cuboid", "cuboid_per_head", "identity"
    cuboid: Optional[Tuple[int, int, int]] = None
    cuboids: Optional[Sequence[Tuple[int, int, int]]] = None   # per head (cuboid_per_head)
    n_pool: int = 0                     # ASA_G window; 0 = plain ASA
    batch: int = 1

    @property
    def N(self) -> int:
        return self.prefix + self.T * self.H * self.W

    @property
    def nb(self) -> int:
        return -(-self.N // self.b)

    @property
    def Npad(self) -> int:
        return self.nb * self.b

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def build_perm(spec: LayerSpec) -> np.ndarray:
    """Host permutation: int32 [N] or [heads, N]."""
    if spec.order == "gilbert":
        return ops.perm_gilbert3d(spec.T, spec.H, spec.W, spec.prefix)
    if spec.order == "cuboid":
        return ops.perm_cuboid(spec.T, spec.H, spec.W, *spec.cuboid, prefix=spec.prefix)
    if spec.order == "cuboid_per_head":
        return np.stack([ops.perm_cuboid(spec.T, spec.H, spec.W, *c, prefix=spec.prefix) for c in spec.cuboids])
    if spec.order == "identity":
        return np.arange(spec.N, dtype=np.int32)
    raise ValueError(spec.order)


class AsaLayer:
    """Holds the device permutation and the intermediate buffers of one layer shape."""

    def __init__(self, spec: LayerSpec, device="cuda", fused: bool = True, overlap: bool = False):
        """fused: the estimate and the mask in one call (dbs_estimate_mask_tok; P_imp is then not
        written unless mask(keep_p_imp=True)), else dbs_estimate_blocks_tok + dbs_build_mask.
        overlap: reorder V on a second stream (default priority) while the estimate runs, the
        attention waiting for it; otherwise K and V are reordered in one launch (the default: on
        the Wan-shaped layer the overlap measured 0.616-0.625 against 0.600-0.607 ms per step,
        the two reorders being slower than the one launch and the V copy slowing the estimate)."""
        self.spec = spec
        self.fused = fused
        self.overlap = overlap and not spec.n_pool
        self._side = torch.cuda.Stream(device=device) if self.overlap else None
        self.device = torch.device(device)
        self.perm = torch.from_numpy(build_perm(spec)).to(self.device)
        s = spec
        B, Hh, Npad, d, nb = s.batch, s.heads, s.Npad, s.d, s.nb
        bf = dict(dtype=torch.bfloat16, device=self.device)
        self.k_r = torch.empty((B, Hh, Npad, d), **bf)
        self.v_t = torch.empty((B, Hh, nb, d, s.b), **bf)
        self.q: Optional[torch.Tensor] = None   # the caller's Q, token order
        self.p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=self.device)
        self.ws = torch.empty(max(16, ops.estimate_workspace_bytes(B, Hh, s.N, d, s.b, s.k)),
                              dtype=torch.uint8, device=self.device)
        self.kv_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=self.device)
        self.kv_idx = torch.empty((B, Hh, nb, nb), dtype=torch.int32, device=self.device)
        self.order = torch.empty((B * Hh * nb,), dtype=torch.int32, device=self.device)
        self.k_g = self.v_g = None
        self.Ng = 0
        if s.n_pool:
            self.Ng = -(-s.N // s.n_pool)
            Ngpad = -(-self.Ng // s.b) * s.b
            self.k_g = torch.empty((B, Hh, Ngpad, d), **bf)
            self.v_g = torch.empty((B, Hh, Ngpad // s.b, d, s.b), **bf)

    def choose_cuboids_sics(self, q: torch.Tensor, candidates: Sequence[Tuple[int, int, int]]):
        """Per head, the candidate cuboid with the largest SICS aggregation score on q (SPADE's
        scheme choice, dbs_sics_tok once per candidate); the layer switches to cuboid_per_head order
        with those shapes and uploads the new permutation.  q [B, N, Hh, d] token order (the first
        batch entry decides).  Returns the chosen cuboid of each head."""
        s = self.spec
        choice, _ = ops.choose_cuboids_sics(q, s.T, s.H, s.W, candidates, s.b, prefix=s.prefix)
        chosen = [tuple(candidates[int(c)]) for c in choice[0].tolist()]
        s.order, s.cuboids = "cuboid_per_head", chosen
        self.perm = torch.from_numpy(build_perm(s)).to(self.device)
        return chosen

    def prepare(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """Reorder (and pool) K and V and keep Q; q, k, v are [B, N, Hh, d]."""
        s = self.spec
        self.q = q
        if s.n_pool:   # the global tokens in the same launch (two passes when n does not divide b)
            ops.reorder_kv(k, v, self.perm, s.Npad, s.b, k_r=self.k_r, v_t=self.v_t, n_pool=s.n_pool, k_g=self.k_g,
                           v_g=self.v_g)
        elif self.overlap:
            # V is needed only by the attention: its reorder (HBM-bound) runs beside the
            # estimate (MFMA / exp-bound); the side stream first waits for everything queued
            # before (the inputs, and the previous step's attention reading v_t)
            main = torch.cuda.current_stream()
            ops.reorder(k, self.perm, s.Npad, s.b, "rows", y=self.k_r)
            self._side.wait_stream(main)
            with torch.cuda.stream(self._side):
                ops.reorder(v, self.perm, s.Npad, s.b, "tiles_t", y=self.v_t)
        else:
            ops.reorder_kv(k, v, self.perm, s.Npad, s.b, k_r=self.k_r, v_t=self.v_t)

    def mask(self, tau: Optional[float] = None, keep_p_imp: bool = False) -> None:
        s = self.spec
        tau = s.tau if tau is None else tau
        if self.fused:
            ops.estimate_mask(self.q, self.k_r, s.N, s.b, s.k, s.scale, "cumulative", tau, q_perm=self.perm,
                              kv_count=self.kv_count, kv_idx=self.kv_idx, order=self.order, workspace=self.ws,
                              p_imp=self.p_imp if keep_p_imp else None)
            return
        ops.estimate_blocks_tok(self.q, self.perm, self.k_r, s.N, s.b, s.k, s.scale, p_imp=self.p_imp,
                                workspace=self.ws)
        ops.build_mask(self.p_imp, tau, kv_count=self.kv_count, kv_idx=self.kv_idx,
                       order=self.order)

    def wait_v(self) -> None:
        """Make the current stream wait for prepare()'s V reorder (side stream); needed before any
        direct use of self.v_t after prepare() (attend() does it)."""
        if self.overlap:
            torch.cuda.current_stream().wait_stream(self._side)

    def attend(self, out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16) -> torch.Tensor:
        s = self.spec
        self.wait_v()
        out, _ = ops.sparse_attn_fwd_tok(self.q, self.perm, self.k_r, self.v_t, s.N, s.b, s.scale, self.kv_count,
                                         self.kv_idx, self.k_g, self.v_g, self.Ng, s.n_pool, out=out,
                                         out_dtype=out_dtype, order=self.order)
        return out

    def forward(self, q, k, v, out: Optional[torch.Tensor] = None, tau: Optional[float] = None,
                out_dtype=torch.bfloat16, keep_p_imp: bool = False) -> torch.Tensor:
        """keep_p_imp: also write P_imp to self.p_imp (always written on the unfused path)."""
        self.prepare(q, k, v)
        self.mask(tau, keep_p_imp)
        return self.attend(out, out_dtype)
