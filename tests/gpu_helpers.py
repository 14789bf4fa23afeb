"""Helpers shared by the GPU parity tests (device tensors from the seeded
workloads; nothing here computes any part of the method)."""
import sys

import numpy as np
import torch

from workloads.generator import bf16_round


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 values that are exactly bf16 -> bf16 device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.array(x, copy=True, order="C")).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def smooth_qkv(seed: int, B: int, N: int, Hh: int, d: int, grid=None, noise=0.3):
    """Smooth-field Q/K (shared field) and iid V, bf16-representable, [B, N, Hh, d]."""
    from workloads.generator import make_head
    if grid is None:
        grid = (1, 1, N)
    q = np.empty((B, N, Hh, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    for bi in range(B):
        for h in range(Hh):
            qq, kk, vv = make_head(1000 + seed, bi * 64 + h, grid, d, (2.0, 2.0, 2.0), prefix=N - int(np.prod(grid)))
            q[bi, :, h], k[bi, :, h], v[bi, :, h] = bf16_round(qq), bf16_round(kk), bf16_round(vv)
    return q, k, v


def kept_lists(kv_count: np.ndarray, kv_idx: np.ndarray):
    """[.., nb] counts + [.., nb, nb] index rows -> nested python lists per row."""
    nb = kv_idx.shape[-1]
    c = kv_count.reshape(-1, nb)
    i = kv_idx.reshape(-1, nb, nb)
    return [[i[r, I, :c[r, I]].tolist() for I in range(nb)] for r in range(c.shape[0])]


def tile_col(t):
    """Column of token offset t in a tiles-transposed tile (bits 2 and 3 swapped)."""
    t = np.asarray(t)
    return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1)


def tiles_to_rows(yt: np.ndarray) -> np.ndarray:
    """[B, Hh, nt, d, b] tiles-transposed -> [B, Hh, nt * b, d] rows."""
    B, Hh, nt, d, b = yt.shape
    cols = tile_col(np.arange(b))
    return yt[..., cols].transpose(0, 1, 2, 4, 3).reshape(B, Hh, nt * b, d)


class Guarded:
    """A device buffer with canary regions before and after it: `view` is the tensor the call
    writes, `intact()` says whether every canary element still holds its fill value."""

    def __init__(self, shape, dtype, fill=-12345.0, pad=4096, device="cuda"):
        n = int(np.prod(shape))
        self.pad = pad
        self.fill = fill
        # the view starts 4096 elements in, so 16-byte alignment is kept for every element size
        self.base = torch.full((pad + n + pad,), fill, dtype=dtype, device=device)
        self.view = self.base[pad:pad + n].view(*shape)

    def intact(self) -> bool:
        f = torch.tensor(self.fill, dtype=self.base.dtype, device=self.base.device)
        return bool((self.base[:self.pad] == f).all().item()) and bool((self.base[-self.pad:] == f).all().item())
