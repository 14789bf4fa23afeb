"""The five workload shapes.

The pages measure on real activations of Wan2.1-1.3B, CogVideoX-5B, Waver and
720p Hunyuan/Wan-14B runs.  No weights or prompts are available, so these
synthetic inputs stand in for them: they take those workloads' latent grids,
head counts, head dimensions and text length, and replace the activations with
smooth random fields (see generator.py).

Latent grids follow the Wan VAE + 1x2x2 patchify arithmetic that the BSA notes'
worked example uses (61 x 448 x 832 video -> 23,296 tokens): frames
(F - 1) / 4 + 1, spatial sides / 16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    T: int
    H: int
    W: int
    heads: int
    d: int
    dtype: str                      # "fp32" or "bf16": storage type of Q, K, V
    b: int                          # block size (tokens)
    k: int                          # sampled tokens per block
    taus: Tuple[float, ...]         # cumulative-mass thresholds
    reorder: str                    # "gilbert", "cuboid", "cuboid_per_head"
    sigma: Tuple[float, float, float] = (3.0, 3.0, 3.0)   # field std in tokens (t, h, w)
    text_prefix: int = 0            # iid text tokens placed before the video tokens
    cuboid: Optional[Tuple[int, int, int]] = None
    cuboid_choices: Tuple[Tuple[int, int, int], ...] = ()
    per_head_sigma: bool = False    # config 5: sigma per head, log-uniform in [1, 8]
    global_pool: int = 0            # ASA_G window n (0: plain ASA)
    target_sparsity: Tuple[float, ...] = ()
    batch: int = 1

    @property
    def n_video(self) -> int:
        return self.T * self.H * self.W

    @property
    def N(self) -> int:
        return self.text_prefix + self.n_video

    @property
    def nb(self) -> int:
        return -(-self.N // self.b)

    @property
    def Npad(self) -> int:
        return self.nb * self.b

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def Ng(self) -> int:
        return -(-self.N // self.global_pool) if self.global_pool else 0

    def dense_flop(self) -> float:
        """Dense-equivalent forward FLOP: 4 * B * H * N^2 * d with the true N."""
        return 4.0 * self.batch * self.heads * float(self.N) ** 2 * self.d


CONFIGS: List[Config] = [
    Config(1, "tiny-2x32x32-d64-fp32", 2, 32, 32, heads=1, d=64, dtype="fp32", b=64, k=8,
           taus=(0.90,), reorder="gilbert", sigma=(3.0, 3.0, 3.0)),
    Config(2, "wan2.1-1.3b-21x30x52", 21, 30, 52, heads=12, d=128, dtype="bf16", b=128, k=16,
           taus=(0.90, 0.95), reorder="gilbert", sigma=(4.0, 4.0, 4.0)),
    Config(3, "cogvideox-5b-13x30x45+226", 13, 30, 45, heads=48, d=64, dtype="bf16", b=128,
           k=16, taus=(0.95,), reorder="gilbert", sigma=(4.0, 4.0, 4.0), text_prefix=226,
           global_pool=8),
    Config(4, "long-40x48x80-cuboid", 40, 48, 80, heads=24, d=128, dtype="bf16", b=128, k=16,
           taus=(), reorder="cuboid", sigma=(2.0, 6.0, 6.0), cuboid=(4, 4, 8),
           target_sparsity=(0.95,)),
    Config(5, "720p-31x45x80-per-head", 31, 45, 80, heads=40, d=128, dtype="bf16", b=128, k=16,
           taus=(), reorder="cuboid_per_head", per_head_sigma=True,
           cuboid_choices=((1, 8, 16), (2, 8, 8), (4, 4, 8), (8, 4, 4)),
           target_sparsity=(0.90, 0.95)),
]


def get_config(cid: int) -> Config:
    for c in CONFIGS:
        if c.cid == cid:
            return c
    raise KeyError(cid)


def latent_grid(frames: int, height: int, width: int) -> Tuple[int, int, int]:
    """Latent token grid of a video after a 4x temporal / 8x spatial VAE and a 2x2 patchify."""
    return ((frames - 1) // 4 + 1, height // 16, width // 16)
