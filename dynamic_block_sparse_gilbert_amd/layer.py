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
    dtype: str = "bf16"                 # "bf16", or "fp32": float32 operands and arithmetic throughout

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


# The largest launch (query blocks over all batches and heads) that runs longest rows first.
ORDER_MAX_BLOCKS = 4096


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


class SicsChooser:
    """SPADE's runtime scheme choice over candidate cuboid shapes of one latent grid: the
    candidates' token orders are built by the library and uploaded once, and each choose() is one
    dbs_sics_choose call (SICS aggregation score of Q and, when given, K for every candidate, then
    the per-head argmax, all on the GPU)."""

    def __init__(self, T: int, H: int, W: int, candidates: Sequence[Tuple[int, int, int]], b: int,
                 prefix: int = 0, device="cuda"):
        self.candidates = [tuple(int(x) for x in c) for c in candidates]
        self.b = b
        self.N = prefix + T * H * W
        self.Npad = -(-self.N // b) * b
        self.host_perms = np.stack([ops.perm_cuboid(T, H, W, *c, prefix=prefix) for c in self.candidates])
        self.perms = torch.from_numpy(self.host_perms).to(device)
        self.choice = self.scores = self.block_scores = None

    def choose(self, q: torch.Tensor, k: Optional[torch.Tensor] = None) -> torch.Tensor:
        """int32 [B, Hh] index of the chosen candidate of every head (left on the device)."""
        B, _, Hh, _ = q.shape
        if self.choice is None or self.choice.shape != (B, Hh) or \
                self.block_scores.shape[1] != (1 if k is None else 2):
            self.choice = self.scores = self.block_scores = None
        self.choice, self.scores, self.block_scores = ops.sics_choose(
            q, k, self.perms, self.Npad, self.b, block_scores=self.block_scores, scores=self.scores,
            choice=self.choice)
        return self.choice

    def chosen(self, batch: int = 0):
        return [self.candidates[int(c)] for c in self.choice[batch].tolist()]

    def per_head_perm(self, batch: int = 0) -> torch.Tensor:
        """int32 [Hh, N] (host): each head's order under its chosen candidate."""
        idx = self.choice[batch].cpu().numpy()
        return torch.from_numpy(np.ascontiguousarray(self.host_perms[idx]))


class AsaLayer:
    """Holds the device permutation and the intermediate buffers of one layer shape."""

    def __init__(self, spec: LayerSpec, device="cuda", fused: bool = True, overlap: bool = False):
        """fused: the estimate and the mask in one call (P_imp is then not written unless
        mask(keep_p_imp=True)), else dbs_estimate_blocks_tok + dbs_build_mask.
        overlap (bf16, fused): the reorder of K and V (and the ASA_G pooling) runs on a second
        stream (default priority) while the estimate, which reads its sampled K rows in token
        order (dbs_estimate_mask_kvtok), runs on the caller's; the attention waits for both.
        Otherwise (the default) the reorder comes first and the estimate reads the reordered K
        (dbs_estimate_mask_tok).  The two give the same masks and outputs bit for bit; the overlap
        measured no faster (21.12-21.20 against 21.07-21.11 ms per step on the 153,600-token
        layer): a reorder workgroup (52 VGPRs x 8 wavefronts) does not fit beside the estimate's two
        workgroups per CU, so the two kernels only take turns on the CUs."""
        if spec.dtype not in ("bf16", "fp32"):
            raise ValueError(f"dtype {spec.dtype!r}: bf16 or fp32")
        if spec.dtype == "fp32" and spec.n_pool:
            raise ValueError("the float32 path takes no ASA_G global tokens")
        self.spec = spec
        self.fused = fused
        self.f32 = spec.dtype == "fp32"
        self.overlap = overlap and fused and not self.f32
        self._side = torch.cuda.Stream(device=device) if self.overlap else None
        self.device = torch.device(device)
        self.perm = torch.from_numpy(build_perm(spec)).to(self.device)
        s = spec
        B, Hh, Npad, d, nb = s.batch, s.heads, s.Npad, s.d, s.nb
        bf = dict(dtype=torch.bfloat16, device=self.device)
        if self.f32:
            # float32 rows for Q, K, V and the output (the float32 kernels read V as rows)
            f4 = dict(dtype=torch.float32, device=self.device)
            self.q_r = torch.empty((B, Hh, Npad, d), **f4)
            self.k_r = torch.empty((B, Hh, Npad, d), **f4)
            self.v_t = torch.empty((B, Hh, Npad, d), **f4)
            self.o_r = torch.empty((B, Hh, Npad, d), **f4)
        else:
            self.k_r = torch.empty((B, Hh, Npad, d), **bf)
            self.v_t = torch.empty((B, Hh, nb, d, s.b), **bf)
        self.q: Optional[torch.Tensor] = None   # the caller's Q, token order
        self.p_imp = torch.empty((B, Hh, nb, nb), dtype=torch.float32, device=self.device)
        wsb = ops.estimate_workspace_bytes(B, Hh, s.N, d, s.b, s.k)
        if self.overlap:
            wsb = max(wsb, ops.estimate_kvtok_workspace_bytes(B, Hh, s.N, d, s.b, s.k))
        self.ws = torch.empty(max(16, wsb), dtype=torch.uint8, device=self.device)
        self.k: Optional[torch.Tensor] = None   # the caller's K, token order (overlap)
        self._pending = None                      # overlap: (k, v) whose reorder is not yet queued
        self._inputs_ready = None
        self.kv_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=self.device)
        self.kv_idx = torch.empty((B, Hh, nb, nb), dtype=torch.int32, device=self.device)
        # Work order of the attention launch.  Longest rows first evens out the tail when the
        # launch is a few rounds of workgroups; on larger launches the plain index order is faster
        # (neighbouring query blocks of a head run together and share most kept key blocks in L2:
        # 16.9 against 17.6 ms on the 153,600-token layer, 0.50 against 0.51 ms the other way on
        # the 32,760-token one), and the mask then writes no order at all.
        self.order = torch.empty((B * Hh * nb,), dtype=torch.int32, device=self.device) \
            if B * Hh * nb <= ORDER_MAX_BLOCKS else None
        self.k_g = self.v_g = None
        self.Ng = 0
        self.anchor: Optional[torch.Tensor] = None   # query pruning (enable_query_pruning)
        if s.n_pool:
            self.Ng = -(-s.N // s.n_pool)
            Ngpad = -(-self.Ng // s.b) * s.b
            self.k_g = torch.empty((B, Hh, Ngpad, d), **bf)
            self.v_g = torch.empty((B, Hh, Ngpad // s.b, d, s.b), **bf)

    def choose_cuboids_sics(self, q: torch.Tensor, candidates: Sequence[Tuple[int, int, int]],
                            k: Optional[torch.Tensor] = None):
        """Per head, the candidate cuboid with the largest SICS aggregation score of q (and k when
        given) (SPADE's scheme choice, one dbs_sics_choose call); the layer switches to
        cuboid_per_head order with those shapes and uploads the new permutation.  q, k
        [B, N, Hh, d] token order (the first batch entry decides).  Returns the chosen cuboid of
        each head."""
        s = self.spec
        ch = SicsChooser(s.T, s.H, s.W, candidates, s.b, prefix=s.prefix, device=self.device)
        ch.choose(q, k)
        chosen = ch.chosen(0)
        s.order, s.cuboids = "cuboid_per_head", chosen
        self.perm = ch.per_head_perm(0).to(self.device)
        self.anchor = None   # window centres follow the order: enable_query_pruning() again
        return chosen

    def prepare(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """Reorder (and pool) K and V and keep Q; q, k, v are [B, N, Hh, d]."""
        s = self.spec
        self.q = q
        if self.f32:
            for x, y in ((q, self.q_r), (k, self.k_r), (v, self.v_t)):
                if x.dtype != torch.float32:
                    raise TypeError("the float32 layer takes float32 q, k, v")
                ops.reorder(x, self.perm, s.Npad, s.b, "rows", y=y)
            return
        if self.overlap:
            # K and V are needed only by the attention: their reorder (HBM-bound) is queued on the
            # side stream right after the estimate (VALU-bound), which gathers its own sampled K
            # rows, so the estimate's workgroups are dispatched first and the reorder fills the
            # CUs its last round leaves idle.  The side stream waits for everything queued before
            # this point (the inputs, and the previous step's attention reading k_r / v_t).
            self.k = k
            self._inputs_ready = torch.cuda.Event()
            self._inputs_ready.record(torch.cuda.current_stream())
            self._pending = (k, v)
        else:
            self._reorder_kv(k, v)

    def _reorder_kv(self, k, v) -> None:
        s = self.spec
        # the global tokens in the same launch (two passes when n does not divide b)
        pool = dict(n_pool=s.n_pool, k_g=self.k_g, v_g=self.v_g) if s.n_pool else {}
        ops.reorder_kv(k, v, self.perm, s.Npad, s.b, k_r=self.k_r, v_t=self.v_t, **pool)

    def _launch_side_reorder(self) -> None:
        """Queue the deferred K / V reorder on the side stream (overlap), once per prepare()."""
        if self._pending is None:
            return
        k, v = self._pending
        self._pending = None
        self._side.wait_event(self._inputs_ready)
        with torch.cuda.stream(self._side):
            self._reorder_kv(k, v)
        k.record_stream(self._side)
        v.record_stream(self._side)

    def mask(self, tau: Optional[float] = None, keep_p_imp: bool = False) -> None:
        s = self.spec
        tau = s.tau if tau is None else tau
        if self.f32:
            ops.estimate_mask(self.q_r, self.k_r, s.N, s.b, s.k, s.scale, "cumulative", tau, kv_count=self.kv_count,
                              kv_idx=self.kv_idx, order=self.order, workspace=self.ws,
                              p_imp=self.p_imp if (keep_p_imp or not self.fused) else None)
            return
        if self.overlap:
            ops.estimate_mask_kvtok(self.q, self.k, self.perm, s.b, s.k, s.scale, "cumulative", tau,
                                    kv_count=self.kv_count, kv_idx=self.kv_idx, order=self.order,
                                    workspace=self.ws, p_imp=self.p_imp if keep_p_imp else None)
            self._launch_side_reorder()
            return
        if self.fused:
            ops.estimate_mask(self.q, self.k_r, s.N, s.b, s.k, s.scale, "cumulative", tau, q_perm=self.perm,
                              kv_count=self.kv_count, kv_idx=self.kv_idx, order=self.order, workspace=self.ws,
                              p_imp=self.p_imp if keep_p_imp else None)
            return
        self.estimate_only()
        ops.build_mask(self.p_imp, tau, kv_count=self.kv_count, kv_idx=self.kv_idx,
                       order=self.order)

    def estimate_only(self) -> torch.Tensor:
        """The importance estimate alone (P_imp written to self.p_imp), as the unfused path runs it."""
        s = self.spec
        if self.f32:
            return ops.estimate_blocks(self.q_r, self.k_r, s.N, s.b, s.k, s.scale, p_imp=self.p_imp, workspace=self.ws)
        self.wait_kv()
        return ops.estimate_blocks_tok(self.q, self.perm, self.k_r, s.N, s.b, s.k, s.scale, p_imp=self.p_imp,
                                       workspace=self.ws)

    def block_sparsity(self) -> float:
        """1 - (kept blocks) / (B * Hh * nb^2) of the current kv_count (one device-to-host copy)."""
        s = self.spec
        kept = int(self.kv_count.sum(dtype=torch.int64).item())
        return 1.0 - kept / float(s.batch * s.heads * s.nb * s.nb)

    def tune_tau(self, target: float, iters: int = 40) -> Tuple[float, float]:
        """The largest float32 tau in (0, 1] whose cumulative mask on the current P_imp has block
        sparsity >= target, found by bisection with dbs_build_mask (the kept count never falls as
        tau grows, so the sparsity is monotone in tau).  P_imp must be current: call
        mask(keep_p_imp=True) (or forward(..., keep_p_imp=True)) first.  Leaves the mask of the
        returned tau in kv_count / kv_idx / order.  Returns (tau, its block sparsity)."""
        if not 0.0 < target < 1.0:
            raise ValueError("target sparsity must lie in (0, 1)")
        f32 = np.float32
        lo, hi = f32(2.0 ** -24), f32(1.0)

        def sparsity_at(t):
            ops.build_mask(self.p_imp, float(t), kv_count=self.kv_count, kv_idx=self.kv_idx, order=self.order)
            return self.block_sparsity()

        if sparsity_at(lo) < target:
            raise ValueError(f"no tau reaches sparsity {target}: the argmax-only mask has {sparsity_at(lo):.4f}")
        for _ in range(iters):
            mid = f32((float(lo) + float(hi)) / 2.0)
            if mid == lo or mid == hi:
                break
            if sparsity_at(mid) >= target:
                lo = mid
            else:
                hi = mid
        return float(lo), sparsity_at(lo)

    def wait_kv(self) -> None:
        """Make the current stream wait for prepare()'s K and V reorder (side stream); needed before
        any direct use of self.k_r, self.v_t, self.k_g or self.v_g after prepare() (attend() and
        estimate_only() do it)."""
        if self.overlap:
            self._launch_side_reorder()
            torch.cuda.current_stream().wait_stream(self._side)

    def attend(self, out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16) -> torch.Tensor:
        s = self.spec
        if self.f32:
            ops.sparse_attn_fwd(self.q_r, self.k_r, self.v_t, s.N, s.b, s.scale, self.kv_count, self.kv_idx,
                                o_r=self.o_r, order=self.order)
            if out is None:
                out = torch.empty((s.batch, s.N, s.heads, s.d), dtype=torch.float32, device=self.device)
            return ops.inverse_reorder(self.o_r, self.perm, s.N, out=out)
        self.wait_kv()
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

    def enable_query_pruning(self, r: float, window: Tuple[int, int, int] = (2, 2, 2)) -> None:
        """BSA query pruning for forward_pruned() (the BSA notes, key design 1): every query block
        keeps the centres of its (t, h, w) windows plus its most distinct other rows, up to ceil(r * n)
        of its n rows; the pruned rows take their centre's output.  Computes the window centres of
        this layer's order once (host) and allocates the pruning lists.  bf16 layers without ASA_G
        global tokens only, as the library's pruned attention."""
        s = self.spec
        if self.f32 or s.n_pool:
            raise ValueError("query pruning takes a bf16 layer without global tokens")
        if not 0.0 < r <= 1.0:
            raise ValueError("the keep ratio r must lie in (0, 1]")
        perm = self.perm.cpu().numpy()
        if perm.ndim == 1:
            anc = ops.prune_anchors(s.T, s.H, s.W, window, perm, prefix=s.prefix)
        else:
            anc = np.stack([ops.prune_anchors(s.T, s.H, s.W, window, p, prefix=s.prefix) for p in perm])
        self.anchor = torch.from_numpy(anc).to(self.device)
        B, Hh, nb = s.batch, s.heads, s.nb
        self.q_count = torch.empty((B, Hh, nb), dtype=torch.int32, device=self.device)
        self.rowsel = torch.empty((B, Hh, nb, s.b), dtype=torch.int32, device=self.device)
        self.keep = torch.empty((B, Hh, s.Npad), dtype=torch.uint8, device=self.device)
        self.prune_r = float(r)

    def forward_pruned(self, q, k, v, out: Optional[torch.Tensor] = None, tau: Optional[float] = None,
                       out_dtype=torch.bfloat16) -> torch.Tensor:
        """The layer with BSA query pruning: K/V reorder, estimate and mask as forward(), then the
        kept query rows (dbs_query_prune), attention for those rows only and token filling
        (dbs_sparse_attn_fwd_pruned_tok).  Call enable_query_pruning() first."""
        if self.anchor is None:
            raise RuntimeError("call enable_query_pruning() first (again after a change of order)")
        s = self.spec
        self.prepare(q, k, v)
        self.mask(tau)
        ops.query_prune(q, self.perm, self.anchor, s.Npad, s.b, self.prune_r, q_count=self.q_count,
                        rowsel=self.rowsel, keep=self.keep)
        self.wait_kv()
        out, _ = ops.sparse_attn_fwd_pruned_tok(q, self.perm, self.k_r, self.v_t, s.N, s.b, s.scale, self.kv_count,
                                                self.kv_idx, self.q_count, self.rowsel, self.anchor, self.keep,
                                                out=out, out_dtype=out_dtype, order=self.order)
        return out

    def capture(self, q, k, v, out: torch.Tensor, tau: Optional[float] = None, warmup: int = 1):
        """One forward pass on these buffers recorded as a HIP graph (torch.cuda.CUDAGraph).

        replay() then runs the same launches (K/V reorder, estimate and mask, attention) with no
        host work per launch, which is what bounds the small layers' steps. q, k, v and out stay
        bound to the graph: refill them in place between replays. The graph also reuses this
        layer's buffers (reordered K/V, kept-block lists, estimator workspace), so a replay
        overwrites them like forward() does. Replays and eager calls on the same layer must not
        overlap on different streams. Every launch of the step is a kernel; the library issues no
        memset and no host synchronisation, so the graph holds kernel nodes only. The two-stream
        layer (overlap=True) is not captured."""
        if self.overlap:
            raise ValueError("capture() takes a one-stream layer (overlap=False)")
        if out is None:
            raise ValueError("capture() needs the output buffer the graph writes")
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                self.forward(q, k, v, out=out, tau=tau, out_dtype=out.dtype)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(q, k, v, out=out, tau=tau, out_dtype=out.dtype)
        return g
