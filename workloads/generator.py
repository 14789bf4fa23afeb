"""Seeded synthetic Q/K/V shaped like video-DiT attention inputs.

Recipe, per (config, head):
1. W ~ iid N(0, 1) on the (T, H, W) latent grid x d channels.
2. F = separable Gaussian low-pass of W along (t, h, w) with per-axis std
   sigma (in tokens); the kernel is truncated at 4 sigma and the borders are
   reflected (scipy.ndimage's defaults).
3. F is standardised per channel to zero mean and unit variance.
4. Q = F + 0.3 eps_Q, K = F + 0.3 eps_K with independent iid N(0, 1) noise;
   V ~ iid N(0, 1).  Q and K share the field, so attention concentrates on
   nearby tokens, as it does in video latents.
5. Text tokens (a prefix, CogVideoX-style) get iid N(0, 1) Q and K.
6. Everything is laid out as [B, N, H, d] in raster order (t, h, w), prefix
   first, and rounded to bf16 (round to nearest even) unless the config keeps
   fp32.  Both the oracle and the GPU path read these same values.

Seeds: numpy.random.default_rng(SeedSequence([config id, head, tensor id]))
with tensor ids 0 field, 1 eps_Q, 2 eps_K, 3 V, 4 text Q, 5 text K,
7 per-head sigma draw, 8 per-head cuboid draw.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np
from scipy import ndimage

from .configs import Config

T_FIELD, T_EPSQ, T_EPSK, T_V, T_TEXTQ, T_TEXTK, T_SIGMA, T_CUBOID = 0, 1, 2, 3, 4, 5, 7, 8


def _rng(key: Sequence[int]) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (returned as float32)."""
    return bf16_to_f32(bf16_bits(x))


def smooth_field(rng: np.random.Generator, grid: Tuple[int, int, int], d: int,
                 sigma: Tuple[float, float, float]) -> np.ndarray:
    T, H, W = grid
    w = rng.standard_normal((T, H, W, d), dtype=np.float32)
    f = ndimage.gaussian_filter(w, sigma=(sigma[0], sigma[1], sigma[2], 0.0), mode="reflect",
                                truncate=4.0)
    f = f.reshape(T * H * W, d).astype(np.float64)
    f -= f.mean(axis=0, keepdims=True)
    sd = f.std(axis=0, keepdims=True)
    f /= np.where(sd > 0, sd, 1.0)
    return f.astype(np.float32)


def head_sigma(cfg: Config, head: int) -> Tuple[float, float, float]:
    if not cfg.per_head_sigma:
        return cfg.sigma
    r = _rng([cfg.cid, head, T_SIGMA])
    return tuple(float(math.exp(r.uniform(0.0, math.log(8.0)))) for _ in range(3))


def head_cuboid(cfg: Config, head: int) -> Optional[Tuple[int, int, int]]:
    if cfg.reorder == "cuboid":
        return cfg.cuboid
    if cfg.reorder == "cuboid_per_head":
        r = _rng([cfg.cid, head, T_CUBOID])
        return cfg.cuboid_choices[int(r.integers(0, len(cfg.cuboid_choices)))]
    return None


def make_head(cid: int, head: int, grid: Tuple[int, int, int], d: int,
              sigma: Tuple[float, float, float], prefix: int = 0, noise: float = 0.3):
    """One head's (q, k, v), each float32 [prefix + T*H*W, d], before any rounding."""
    f = smooth_field(_rng([cid, head, T_FIELD]), grid, d, sigma)
    n = f.shape[0]
    q = f + noise * _rng([cid, head, T_EPSQ]).standard_normal((n, d), dtype=np.float32)
    k = f + noise * _rng([cid, head, T_EPSK]).standard_normal((n, d), dtype=np.float32)
    if prefix:
        tq = _rng([cid, head, T_TEXTQ]).standard_normal((prefix, d), dtype=np.float32)
        tk = _rng([cid, head, T_TEXTK]).standard_normal((prefix, d), dtype=np.float32)
        q = np.concatenate([tq, q], axis=0)
        k = np.concatenate([tk, k], axis=0)
    v = _rng([cid, head, T_V]).standard_normal((prefix + n, d), dtype=np.float32)
    return q.astype(np.float32), k.astype(np.float32), v


def _head_job(args):
    cfg, h, round_bf16 = args
    qkv = make_head(cfg.cid, h, (cfg.T, cfg.H, cfg.W), cfg.d, head_sigma(cfg, h), cfg.text_prefix)
    return tuple(bf16_round(x) if round_bf16 else x for x in qkv)


def make_inputs(cfg: Config, heads: Optional[Sequence[int]] = None, round_bf16: Optional[bool] = None,
                workers: int = 1):
    """Q, K, V as float32 [1, N, len(heads), d] (bf16-representable unless the config is fp32).
    workers > 1 draws the heads in that many threads (the filter and the draws run outside the
    interpreter lock); every head has its own seeds, so the values do not depend on the worker
    count."""
    if heads is None:
        heads = range(cfg.heads)
    heads = list(heads)
    if round_bf16 is None:
        round_bf16 = cfg.dtype == "bf16"
    N, d = cfg.N, cfg.d
    out = [np.empty((1, N, len(heads), d), dtype=np.float32) for _ in range(3)]
    jobs = [(cfg, h, round_bf16) for h in heads]
    if workers > 1 and len(heads) > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=min(workers, len(heads))) as ex:
            results = ex.map(_head_job, jobs)
            for j, qkv in enumerate(results):
                for t in range(3):
                    out[t][0, :, j, :] = qkv[t]
    else:
        for j, job in enumerate(jobs):
            qkv = _head_job(job)
            for t in range(3):
                out[t][0, :, j, :] = qkv[t]
    return out[0], out[1], out[2]
