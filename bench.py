#!/usr/bin/env python3
"""Benchmark: ASA attention layers on one MI355X.

Headline workload: the long-sequence layer -- batch 1, 24 heads, head dim 128,
bf16, latent 40 x 48 x 80 = 153,600 tokens in 4 x 4 x 8 cuboid blocks of 128,
smooth-field Q/K (temporal sigma 2, spatial sigma 6) + 0.3 noise, iid V;
b = 128, k = 16, and the cumulative threshold tau bisected (outside the timed
region) to the largest value whose block sparsity is at least 0.95.  The other
workload shapes are measured in the same run and reported under
extra.configs: the 2 x 32 x 32 single-head layer (d 64, tau 0.9), the
Wan2.1-1.3B-shaped layer (tau 0.90 and 0.95), the CogVideoX-5B-shaped layer
with ASA_G global tokens (tau 0.95) and the 720p layer with per-head cuboid
shapes (tau bisected to block sparsity 0.90 and 0.95).  Synthetic inputs
stand in for the models' activations.

A step is one pass of the whole hot path over one batch, on one stream:
reorder K, V (with the ASA_G pooling where enabled) -> estimate_mask (sampled
estimate with the selection fused into its final launch) -> sparse_attn_fwd
(Q read and the output written in token order).  Inputs are resident in HBM
before timing; buffers and the permutation are set up outside the timed
region.

value = dense-equivalent TFLOP/s = 4 * B * H * N^2 * d / (seconds per step).
graph_ms_per_step / graph_value: the same step recorded once as a HIP graph
(AsaLayer.capture) and replayed back to back, which removes the host launch
work per kernel (it bounds the smallest layers); value stays the eager step.
The timed region holds HIP events at its two ends only; per-stage times come
from a separate untimed pass with HIP events between the stages on the launch
stream.  roofline = the attention kernel (the dominant one): executed FLOP
(4 d sum over kept block pairs of |I| |J|, plus 4 d N Ng per head for the
global tokens) / its mean launch time in that pass, against the bf16 dense
MFMA peak.  stage_rooflines add the reorder and the mask (HBM), and the
estimate (MFMA and exponential bound).  cpu_baseline = the CPU oracle on a
bounded sample of the same layer (some heads, some query blocks), scaled to
the whole layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E peak
# v_exp_f32 issues at half the 32-bit VALU rate (8 cycles per 64-lane wavefront):
# 256 CUs x 4 SIMDs x 8 results per clock x 2.4 GHz
EXP_PEAK_PER_S = 256 * 4 * 8 * 2.4e9
# 32-bit VALU issue: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz (a 64-lane instruction takes
# 4 clocks; packed FP32 is not used).  Every sampled score of the estimate needs an fma (scale and
# running maximum), an add (the softmax sum), half a v_max3 (the block maximum) and an exponential
# at half rate (two issue slots): 4.5 slots per score.
VALU_PEAK_PER_S = 256 * 4 * 16 * 2.4e9
EST_VALU_SLOTS_PER_SCORE = 4.5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
ATTN_SRC = os.path.join(ROOT, "dynamic_block_sparse_gilbert_amd", "csrc", "kernels", "attn.hip")
METRIC = "ms/layer + dense-equiv TFLOP/s, block-sparse attn at 90-95% sparsity, 1 GPU"

HEADLINE = (4, "target", 0.95)
# config id -> the thresholds it is measured at: ("tau", value) fixed by the config,
# ("target", s) bisected for block sparsity >= s
EXTRA_RUNS = {1: [("tau", 0.90)], 2: [("tau", 0.90), ("tau", 0.95)], 3: [("tau", 0.95)],
              5: [("target", 0.90), ("target", 0.95)]}
# CPU baseline sample per config: (heads, query blocks per head or None for all)
CPU_SAMPLE = {1: (1, None), 2: (2, 16), 3: (2, 16), 4: (2, 32), 5: (2, 8)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE[0], help="headline config id")
    ap.add_argument("--target", type=float, default=None,
                    help="headline block-sparsity target (tau bisected); default 0.95 for config 4")
    ap.add_argument("--tau", type=float, default=None, help="headline fixed tau instead of a target")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="estimate and mask as two calls")
    ap.add_argument("--no-extra", action="store_true", help="headline only: no other configs, no extra legs")
    ap.add_argument("--no-legs", action="store_true", help="skip the backward / pruning / pooled / rules legs")
    ap.add_argument("--configs", type=str, default="1,2,3,5", help="other configs measured under extra")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="after the headline, run each stage (and the whole step) back to back for this "
                         "many seconds, with wall-clock stamps, for power and clock sampling beside it")
    return ap.parse_args()


def log(*a):
    """Progress on stderr (the result line alone goes to stdout)."""
    print("[bench]", *a, file=sys.stderr, flush=True)


def src_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kept_pair_tokens(cnt, idx, N, b, q_rows=None):
    """sum over kept (I, J) of |I| * |J| with valid-token block sizes; q_rows (same shape as cnt):
    the query rows computed per block instead of |I| (pruned queries)."""
    import numpy as np
    nb = cnt.shape[-1]
    L = np.array([min(b, N - J * b) for J in range(nb)], dtype=np.float64)
    c = cnt.reshape(-1, nb).astype(np.int64)
    ix = idx.reshape(-1, nb, nb)
    qr = None if q_rows is None else q_rows.reshape(-1, nb).astype(np.float64)
    # per row: sum of L over its first c entries (entries past the count are ignored)
    valid = np.arange(nb)[None, None, :] < c[:, :, None]
    kl = np.where(valid, L[np.clip(ix, 0, nb - 1)], 0.0).sum(axis=2)
    rows = L[None, :] if qr is None else qr
    return float((rows * kl).sum())


def sampled_tokens(cfg):
    return sum(min(cfg.k, min(cfg.b, cfg.N - J * cfg.b)) for J in range(cfg.nb))


def _timed(fn, reps, torch, warm=1):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_steps(layer, q, k, v, out, tau, steps, warmup, torch):
    """The timed region: `steps` whole layer steps, back to back on one stream, with HIP events
    only at its two ends.  Returns (host ms per step between synchronisations, event ms per step)."""
    for _ in range(warmup):
        layer.forward(q, k, v, out=out, tau=tau)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        layer.forward(q, k, v, out=out, tau=tau)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, e0.elapsed_time(e1) / steps


def run_graph_steps(layer, q, k, v, out, tau, steps, warmup, torch):
    """The same step recorded once as a HIP graph (AsaLayer.capture) and replayed: `steps`
    replays back to back with HIP events at the two ends.  Returns ms per step, or None for a
    two-stream layer.  The replays run the same kernels on the same buffers as the eager steps
    (bit-identical results, tested); only the host launch work per kernel is gone."""
    if layer.overlap:
        return None
    g = layer.capture(q, k, v, out, tau=tau)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return ms


def stage_times(layer, q, k, v, out, tau, steps, torch):
    """Per-stage breakdown in a separate, untimed pass over the same steps: HIP events on the
    launch stream between the stages of each step (each stage time carries one event's cost).
    The attention entry is the mean attention launch duration used for the roofline.  The stages
    run one after another here (the launch stream waits for the K/V reorder before the estimate),
    while the timed steps overlap the reorder with the estimate."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    names = ["reorder_kv", "estimate_mask", "attn"] if layer.fused else ["reorder_kv", "estimate", "mask", "attn"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for s in range(steps):
        e = ev[s]
        e[0].record()
        layer.prepare(q, k, v)
        layer.wait_kv()
        e[1].record()
        if layer.fused:
            layer.mask(tau)
        else:
            layer.estimate_only()
            e[2].record()
            ops.build_mask(layer.p_imp, tau, kv_count=layer.kv_count, kv_idx=layer.kv_idx, order=layer.order)
        e[len(names) - 1].record()
        layer.attend(out)
        e[len(names)].record()
    torch.cuda.synchronize()
    return {n: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
            for i, n in enumerate(names)}


def traffic_lookup(cid, tau):
    """HBM bytes per attention launch from the committed counter record, if it was taken on the
    current attention source at this config and tau; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        recs = json.load(open(TRAFFIC_FILE))["records"]
    except Exception:
        return None
    h = src_hash(ATTN_SRC)
    for r in recs:
        if r.get("config") == cid and r.get("attn_src_sha256_16") == h and abs(r.get("tau", -1) - tau) < 1e-6:
            return r.get("bytes_per_launch")
    return None


def make_layer(cfg, dev, fused=True):
    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    from workloads.generator import head_cuboid
    cub = [head_cuboid(cfg, h) for h in range(cfg.heads)] if cfg.reorder == "cuboid_per_head" else None
    spec = LayerSpec(T=cfg.T, H=cfg.H, W=cfg.W, heads=cfg.heads, d=cfg.d, b=cfg.b, k=cfg.k, tau=0.9,
                     prefix=cfg.text_prefix, order=cfg.reorder, cuboid=cfg.cuboid, cuboids=cub,
                     n_pool=cfg.global_pool, dtype=cfg.dtype)
    return AsaLayer(spec, device=dev, fused=fused)


def workload_name(cfg):
    grid = f"{cfg.T}x{cfg.H}x{cfg.W}"
    if cfg.text_prefix:
        grid = f"{cfg.text_prefix} text + {grid}"
    order = {"gilbert": "Gilbert-curve order", "cuboid": "cuboid order %s" % (cfg.cuboid,),
             "cuboid_per_head": "per-head cuboid order"}[cfg.reorder]
    g = f", ASA_G n={cfg.global_pool}" if cfg.global_pool else ""
    return (f"{cfg.name}: B=1, {cfg.heads} heads, d={cfg.d}, {cfg.dtype}, {grid} = {cfg.N:,} tokens, "
            f"b={cfg.b}, k={cfg.k}, {order}{g}")


def mask_stage_bytes(rows_bh, nb, kept, with_order):
    """Bytes dbs_build_mask must move: P_imp read once (rows_bh = B * H heads of nb x nb float32),
    kv_count written (one int32 per row), the kept entries of kv_idx written (kept = the total
    over all rows and heads), and the work order (one int32 per row) when it is written."""
    rows = rows_bh * nb
    return 4.0 * rows * nb + 4.0 * rows + 4.0 * kept + (4.0 * rows if with_order else 0.0)


def measure(layer, cfg, qd, kd, vd, out, tau, steps, warmup, torch):
    """One layer at one tau: the timed steps, the stage breakdown, the attention roofline and the
    byte / estimate stages, each against its own bound."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    ms, ms_ev = run_steps(layer, qd, kd, vd, out, tau, steps, warmup, torch)
    ms_graph = run_graph_steps(layer, qd, kd, vd, out, tau, steps, warmup, torch)
    stage = stage_times(layer, qd, kd, vd, out, tau, max(steps, 5), torch)
    cnt, idx = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy()
    nb, H, N, d = cfg.nb, cfg.heads, cfg.N, cfg.d
    sparsity = 1.0 - cnt.sum() / (cnt.size * nb)
    pairs = kept_pair_tokens(cnt, idx, N, cfg.b)
    exec_flop = 4.0 * d * pairs + (4.0 * d * H * N * cfg.Ng if cfg.global_pool else 0.0)
    attn_ms = stage["attn"]
    attn_tflops = exec_flop / (attn_ms * 1e-3) / 1e12
    dense = cfg.dense_flop()
    reps = max(5, steps)
    # the estimate and the mask as separate launches, each `reps` times back to back
    t_est = _timed(layer.estimate_only, reps, torch)
    t_mask = _timed(lambda: ops.build_mask(layer.p_imp, tau, kv_count=layer.kv_count, kv_idx=layer.kv_idx,
                                           order=layer.order), reps, torch)
    ns = sampled_tokens(cfg)
    est_flop = 2.0 * H * ns * ns * d
    est_exp = float(H) * ns * ns
    est_valu_ms = est_exp * EST_VALU_SLOTS_PER_SCORE / VALU_PEAK_PER_S * 1e3
    if cfg.dtype == "fp32":
        # the float32 estimate forms its scores on the VALU too: one fma per two FLOP
        est_valu_ms += est_flop / 2.0 / VALU_PEAK_PER_S * 1e3
    est_bound_ms = max(est_flop / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3 if cfg.dtype != "fp32" else 0.0,
                       est_exp / EXP_PEAK_PER_S * 1e3, est_valu_ms)
    kept = float(cnt.sum())          # kept blocks over every row of every head
    mask_bytes = mask_stage_bytes(cnt.shape[0] * H, nb, kept, with_order=layer.order is not None)
    e = 4 if cfg.dtype == "fp32" else 2
    # bf16: K and V read and written; float32: Q, K and V (the float32 path reorders Q too)
    nt = 3 if cfg.dtype == "fp32" else 2
    reorder_bytes = nt * H * N * d * e + nt * H * cfg.Npad * d * e
    if cfg.global_pool:
        reorder_bytes += 2.0 * H * (-(-cfg.Ng // cfg.b) * cfg.b) * d * e
    res = {
        "workload": workload_name(cfg),
        "tau": tau,
        "block_sparsity": round(float(sparsity), 4),
        "ms_per_step": round(ms, 4),
        "value": round(dense / (ms * 1e-3) / 1e12, 2),
        "unit": "dense-equiv TFLOP/s",
        "step_ms_events": round(ms_ev, 4),
        "graph_ms_per_step": None if ms_graph is None else round(ms_graph, 4),
        "graph_value": None if ms_graph is None else round(dense / (ms_graph * 1e-3) / 1e12, 2),
        "stages_ms": {kk: round(vv, 4) for kk, vv in stage.items()},
        "step_streams": ("reorder_kv on a second stream beside estimate_mask (dbs_estimate_mask_kvtok); "
                         "stages_ms times the stages one after another" if layer.overlap else "one stream"),
        "token_pairs_kept": pairs,
        "executed_attn_flop": exec_flop,
        "dense_equiv_flop": dense,
        "roofline": {
            # the float32 path runs on the vector ALUs (no float32 MFMA): its peak is the fp32 vector rate
            "bound": "mfma" if cfg.dtype != "fp32" else "alu",
            "kernel": "attn_fwd_kernel<%d,%d>" % (d, cfg.b) if cfg.dtype != "fp32" else "attn_f32_kernel",
            "achieved": round(attn_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS if cfg.dtype != "fp32" else 157.3,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / (MFMA_BF16_PEAK_TFLOPS if cfg.dtype != "fp32" else 157.3), 4),
            "traffic": traffic_lookup(cfg.cid, tau),
            "launch_ms": round(attn_ms, 4),
        },
        "stage_rooflines": {
            "reorder_kv": {"bound": "hbm", "bytes": reorder_bytes, "ms": round(stage["reorder_kv"], 4),
                           "achieved_GBs": round(reorder_bytes / (stage["reorder_kv"] * 1e-3) / 1e9, 1),
                           "peak_GBs": HBM_PEAK_GBS,
                           "frac": round(reorder_bytes / (stage["reorder_kv"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "estimate": {"bound": "mfma+valu", "flop": est_flop, "exp": est_exp, "ms": round(t_est, 4),
                         "bound_ms": round(est_bound_ms, 4), "frac": round(est_bound_ms / t_est, 4),
                         "valu_floor_ms": round(est_valu_ms, 4),
                         "what": "dbs_estimate_blocks_tok alone (pass + final, P_imp written); bound = "
                                 "max(FLOP / bf16 MFMA peak, exponentials / %.3g per s, the VALU issue floor of %.1f slots "
                                 "per sampled score at %.3g lane-slots per s)" % (EXP_PEAK_PER_S, EST_VALU_SLOTS_PER_SCORE,
                                                                                VALU_PEAK_PER_S)},
            "mask": {"bound": "hbm", "bytes": mask_bytes, "ms": round(t_mask, 4),
                     "achieved_GBs": round(mask_bytes / (t_mask * 1e-3) / 1e9, 1), "peak_GBs": HBM_PEAK_GBS,
                     "frac": round(mask_bytes / (t_mask * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "what": "dbs_build_mask alone on a stored P_imp (read once; kv_count, the kept kv_idx "
                             "entries and the work order written), as the tau search and the unfused path run "
                             "it; the timed step selects inside the fused estimate_mask call instead"},
            "estimate_mask_fused_ms": round(stage.get("estimate_mask", float("nan")), 4),
        },
    }
    # restore this tau's lists (the legs above left them in place, but keep the contract explicit)
    layer.mask(tau)
    return res


def cpu_baseline(cfg, q, k, v, perm, tau, heads, blocks, seed=0):
    """The oracle, as it stands, on a bounded sample of the same layer: `heads` heads, and on each
    either every query block or `blocks` of them (first, last and seeded random ones) for the
    estimator rows, the mask rows and the attention rows; the time is scaled to all heads and
    blocks (each stage's work is proportional to the query rows it covers)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.attention import global_bias, masked_attention, meanpool
    from oracle.estimator import p_imp
    from oracle.mask import build_mask
    from oracle.reorder import reorder_fast

    nb = cfg.nb
    rng = np.random.default_rng(seed)
    t_est = t_mask = t_attn = 0.0
    for h in range(heads):
        ph = perm[h] if perm.ndim == 2 else perm
        x = [reorder_fast(t[:, :, h:h + 1], ph, cfg.Npad)[0, 0] for t in (q, k, v)]
        if blocks is None or blocks >= nb:
            qb = list(range(nb))
        else:
            qb = sorted(set([0, nb - 1] + rng.choice(np.arange(1, nb - 1), size=blocks - 2, replace=False).tolist()))
        t0 = time.perf_counter()
        P = p_imp(x[0], x[1], cfg.N, cfg.b, cfg.k, cfg.scale, query_blocks=qb).astype(np.float32)
        t_est += time.perf_counter() - t0
        t0 = time.perf_counter()
        cnt, idx, _, _ = build_mask(P[qb], tau)
        t_mask += time.perf_counter() - t0
        kept = [[] for _ in range(nb)]
        for j, I in enumerate(qb):
            kept[I] = idx[j, :cnt[j]].tolist()
        kg = vg = gb = None
        t0 = time.perf_counter()
        if cfg.global_pool:
            kg, vg = meanpool(x[1], cfg.N, cfg.global_pool), meanpool(x[2], cfg.N, cfg.global_pool)
            gb = global_bias(cfg.N, cfg.global_pool)
        masked_attention(x[0], x[1], x[2], cfg.N, cfg.b, kept, cfg.scale, kg, vg, gb, query_blocks=qb)
        t_attn += time.perf_counter() - t0
    frac = heads / cfg.heads * len(qb) / nb
    sample = t_est + t_mask + t_attn
    total = sample / frac
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blk = "every query block" if len(qb) == nb else f"{len(qb)} of {nb} query blocks"
    return {
        "value": cfg.dense_flop() / total / 1e12,
        "unit": "dense-equiv TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"heads 0-{heads - 1} of {cfg.heads}, {blk} each (estimator rows, mask rows, attention rows): "
                   f"estimator {t_est:.2f} s, mask {t_mask:.2f} s, attention {t_attn:.2f} s "
                   f"({sample:.1f} s of CPU work); scaled x{1 / frac:.4g} -> {total:.1f} s per layer"),
        "mask_builder_single_thread_s": round(t_mask, 3),
        "mask_rows_timed": heads * len(qb),
        "cpu_model": model,
        "host_cpus": os.cpu_count(),
        "blas_threads": threads,
    }


# ----------------------------------------------------------------------------- legs on the Wan layer

def backward_leg(layer, cfg, qd, vd, steps, warmup, torch):
    """The backward of the attention (plain ASA) on the same layer and mask: the key-to-query lists
    and the dQ / dK / dV kernels, timed back to back between two HIP events.  Q, V (rows) and dO are
    reordered and the forward's output and lse computed beforehand, outside the timed region."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    q_r = ops.reorder(qd, layer.perm, sp.Npad, sp.b, "rows")
    v_r = ops.reorder(vd, layer.perm, sp.Npad, sp.b, "rows")
    gen = torch.Generator(device=qd.device).manual_seed(7)
    do = torch.randn(qd.shape, generator=gen, device=qd.device, dtype=torch.float32).to(torch.bfloat16)
    do_r = ops.reorder(do, layer.perm, sp.Npad, sp.b, "rows")
    o_r, lse = ops.sparse_attn_fwd(q_r, layer.k_r, layer.v_t, sp.N, sp.b, sp.scale, layer.kv_count,
                                   layer.kv_idx, want_lse=True)
    ws = torch.empty(ops.attn_bwd_workspace_bytes(1, sp.heads, sp.Npad, sp.d), dtype=torch.uint8,
                     device=qd.device)

    def one():
        kc, ki = ops.transpose_lists(layer.kv_count, layer.kv_idx)
        ops.sparse_attn_bwd(q_r, layer.k_r, v_r, o_r, do_r, lse, sp.N, sp.b, sp.scale, layer.kv_count,
                            layer.kv_idx, kc, ki, workspace=ws)
    ms = _timed(one, steps, torch, warm=warmup)
    cnt, idx = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy()
    pairs = kept_pair_tokens(cnt, idx, sp.N, sp.b)
    alg = 10.0 * sp.d * pairs        # five products over the kept pairs (S, dP, dV, dQ, dK)
    executed = 14.0 * sp.d * pairs   # S and dP are computed in both kernels
    return {
        "ms": round(ms, 4),
        "what": "dbs_transpose_lists + dbs_sparse_attn_bwd (dQ, dK/dV kernels), "
                "tau %.2f mask of the Wan-shaped layer" % sp.tau,
        "algorithmic_flop": alg,
        "executed_flop": executed,
        "algorithmic_tflops": round(alg / (ms * 1e-3) / 1e12, 1),
        "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 1),
        "executed_frac_of_bf16_peak": round(executed / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
    }


def mask_rules_leg(layer, steps, torch):
    """The alternative selection rules on the layer's P_imp: the kept-block lists under the
    cumulative threshold (tau 0.9), top-k (k = 16) and the statistical cutoff expecting 16 of nb
    blocks (the library computes u = U(1 - 16/nb)), each launched `steps` times back to back."""
    from dynamic_block_sparse_gilbert_amd import ops
    nb = layer.p_imp.shape[-1]
    out = {}
    for name, rule, param in (("cumulative_tau0.9", "cumulative", 0.9), ("topk_16", "topk", 16),
                              ("stat_k16", "stat_k", 16)):
        t = _timed(lambda: ops.build_mask_rule(layer.p_imp, rule, param, kv_count=layer.kv_count,
                                               kv_idx=layer.kv_idx), steps, torch)
        cnt = layer.kv_count.cpu().numpy()
        out[name] = {"us": round(t * 1e3, 2), "block_sparsity": round(float(1.0 - cnt.sum() / (cnt.size * nb)), 4)}
    return out


def query_pruning_leg(layer, cfg, qd, steps, torch, r=0.5, win=(2, 2, 2), tau=None):
    """BSA query pruning on the layer and mask: the kept rows (centres of 2 x 2 x 2 windows plus
    the most distinct tokens, keep ratio r), the attention over them with token filling, against the
    unpruned attention on the same lists; each timed back to back between two HIP events."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    perm_h = layer.perm.cpu().numpy()
    anc = torch.from_numpy(ops.prune_anchors(cfg.T, cfg.H, cfg.W, win, perm_h)).to(qd.device)
    out = torch.empty_like(qd)

    def prune():
        return ops.query_prune(qd, layer.perm, anc, sp.Npad, sp.b, r)

    qc, rs, kp = prune()

    def pruned():
        ops.sparse_attn_fwd_pruned_tok(qd, layer.perm, layer.k_r, layer.v_t, sp.N, sp.b, sp.scale, layer.kv_count,
                                       layer.kv_idx, qc, rs, anc, kp, out=out, order=layer.order)

    def full():
        ops.sparse_attn_fwd_tok(qd, layer.perm, layer.k_r, layer.v_t, sp.N, sp.b, sp.scale, layer.kv_count,
                                layer.kv_idx, out=out, order=layer.order)

    t_prune, t_pruned, t_full = (_timed(f, steps, torch, warm=3) for f in (prune, pruned, full))
    cnt, idx, qch = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy(), qc.cpu().numpy()
    kept_q = float(qch.sum()) / (qch.shape[0] * qch.shape[1] * sp.N)
    nb = cnt.shape[-1]
    c2, i2 = cnt.reshape(-1, nb), idx.reshape(-1, nb, nb)
    own = float(c2.sum())
    union = 0.0
    for r_ in range(c2.shape[0]):
        for I in range(0, nb - 1, 2):
            union += len(set(i2[r_, I, :c2[r_, I]].tolist()) | set(i2[r_, I + 1, :c2[r_, I + 1]].tolist()))
    ef = 4.0 * sp.d * kept_pair_tokens(cnt, idx, sp.N, sp.b, q_rows=qch)
    kv_keep = float(cnt.sum() / (cnt.size * cnt.shape[-1]))
    return {
        "what": "dbs_query_prune + dbs_sparse_attn_fwd_pruned_tok (attention over the kept rows with token "
                "filling), 2x2x2 centre windows, keep ratio %.2f, on the tau %.6g mask of the %s layer"
                % (r, sp.tau if tau is None else tau, cfg.name),
        "query_keep": round(kept_q, 4),
        "kv_block_keep": round(kv_keep, 4),
        "combined_sparsity": round(1.0 - kept_q * kv_keep, 4),
        "prune_us": round(t_prune * 1e3, 2),
        "pruned_attn_ms": round(t_pruned, 4),
        "prune_plus_pruned_attn_ms": round(t_prune + t_pruned, 4),
        "unpruned_attn_ms": round(t_full, 4),
        "pruned_attn_executed_tflops": round(ef / (t_pruned * 1e-3) / 1e12, 2),
        "pair_union_over_own_blocks": round(2.0 * union / own, 4),
    }


def pooled_leg(layer, cfg, qd, steps, torch):
    """The pooled estimates (MEAN, TRIP) on the layer, each timed back to back between two HIP
    events, with the cumulative mask they give at the layer's tau."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    out = {}
    ws = torch.empty(max(16, ops.lib().dbs_pooled_workspace_bytes(1, sp.heads, sp.N, sp.d, sp.b)), dtype=torch.uint8,
                     device=qd.device)
    for kind in ("mean", "trip"):
        t = _timed(lambda: ops.estimate_pooled(qd, layer.perm, layer.k_r, sp.N, sp.b, kind, p_imp=layer.p_imp,
                                               workspace=ws), steps, torch)
        cnt, _, _ = ops.build_mask(layer.p_imp, sp.tau)
        c = cnt.cpu().numpy()
        out[kind] = {"us": round(t * 1e3, 2), "block_sparsity_at_tau": round(float(1 - c.sum() / (c.size * sp.nb)), 4)}
    return out


def sics_leg(cfg, qd, kd, steps, torch, step_ms=None):
    """SPADE's scheme choice on the 720p layer: every candidate block shape of the config scored by
    the SICS aggregation score of Q and K in one call (candidate permutations uploaded once), and
    the per-head choice; timed back to back between two HIP events."""
    from dynamic_block_sparse_gilbert_amd.layer import SicsChooser
    ch = SicsChooser(cfg.T, cfg.H, cfg.W, cfg.cuboid_choices, cfg.b, prefix=cfg.text_prefix, device=qd.device)
    t0 = time.perf_counter()
    ch.choose(qd, kd)
    torch.cuda.synchronize()
    first = (time.perf_counter() - t0) * 1e3
    t = _timed(lambda: ch.choose(qd, kd), steps, torch)
    choice = ch.choice.cpu().numpy()[0].tolist()
    res = {"candidates": [list(c) for c in cfg.cuboid_choices], "choice_per_head": choice,
           "ms_all_candidates": round(t, 4), "first_call_wall_ms": round(first, 2),
           "what": "dbs_sics_choose: SICS of Q and K for every candidate cuboid order and the per-head argmax, "
                   "one call"}
    if step_ms:
        res["share_of_layer_step"] = round(t / step_ms, 4)
    return res


# ----------------------------------------------------------------------------- driver

def sustain_leg(layer, tens, tau, secs, torch):
    """Each stage of the step alone, then the whole step, launched back to back for about `secs`
    seconds of wall time, with 3 s idle gaps between them; per stage the mean time per call
    (HIP events) and the Unix times it started and ended (for sampling the board's power and clock
    beside the run)."""
    qd, kd, vd = tens
    out = torch.empty_like(qd)
    stages = [("attention", lambda: layer.attend(out)),
              ("estimate_mask", lambda: layer.mask(tau)),
              ("reorder_kv", lambda: layer._reorder_kv(kd, vd)),
              ("layer_step", lambda: layer.forward(qd, kd, vd, out=out, tau=tau))]
    layer.forward(qd, kd, vd, out=out, tau=tau)
    res = {}
    for name, fn in stages:
        torch.cuda.synchronize()
        time.sleep(3.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.time()
        e0.record()
        calls = 0
        while calls == 0 or time.time() - t0 < secs:
            for _ in range(10):
                fn()
            calls += 10
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        res[name] = {"ms_per_call": round(e0.elapsed_time(e1) / calls, 4), "calls": calls,
                     "start_unix": round(t0, 3), "end_unix": round(t1, 3)}
        log(f"sustain {name} start {t0:.3f} end {t1:.3f} ms/call {res[name]['ms_per_call']}")
    return res


def load_inputs(cfg, torch, dev):
    from workloads import make_inputs
    t0 = time.perf_counter()
    q, k, v = make_inputs(cfg, workers=16)
    t_gen = time.perf_counter() - t0
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    to = lambda a: torch.from_numpy(a).to(dt).to(dev)
    return (q, k, v), (to(q), to(k), to(v)), t_gen


def resolve_tau(layer, qd, kd, vd, out, mode, val):
    if mode == "tau":
        return float(val), {"tau_rule": "fixed by the workload"}
    # P_imp alone (the estimate and a mask at tau 1): the bisection needs no attention
    layer.prepare(qd, kd, vd)
    layer.mask(1.0, keep_p_imp=True)
    tau, s = layer.tune_tau(val)
    return tau, {"tau_rule": f"largest float32 tau with block sparsity >= {val} (bisection with dbs_build_mask "
                             "on the layer's P_imp, outside the timed region)", "target_sparsity": val}


def run_config(cid, rules, args, torch, dev, cpu=True):
    import numpy as np
    from workloads import get_config
    cfg = get_config(cid)
    log(f"config {cid}: inputs")
    host, (qd, kd, vd), t_gen = load_inputs(cfg, torch, dev)
    layer = make_layer(cfg, dev, fused=not args.unfused)
    out = torch.empty_like(qd)
    torch.cuda.synchronize()
    results = []
    for mode, val in rules:
        tau, info = resolve_tau(layer, qd, kd, vd, out, mode, val)
        log(f"config {cid}: tau {tau:.6g}, timing")
        res = measure(layer, cfg, qd, kd, vd, out, tau, args.steps, args.warmup, torch)
        res.update(info)
        res["input_gen_s"] = round(t_gen, 2)
        log(f"config {cid}: {res['ms_per_step']} ms/step, sparsity {res['block_sparsity']}")
        if cpu:
            log(f"config {cid}: cpu baseline")
            heads, blocks = CPU_SAMPLE[cid]
            res["cpu_baseline"] = cpu_baseline(cfg, *host, np.asarray(layer.perm.cpu().numpy()), tau, heads, blocks)
        results.append(res)
    return cfg, layer, (qd, kd, vd), results


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): every step of the path is "
              "independent per head, so several GPUs would each run a share of the heads; the library "
              "has no multi-GPU launch.", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.tau is not None:
        rule = ("tau", args.tau)
    elif args.target is not None:
        rule = ("target", args.target)
    elif args.config == HEADLINE[0]:
        rule = HEADLINE[1:]
    else:
        rule = EXTRA_RUNS.get(args.config, [("tau", 0.9)])[0]
    cfg, layer, tens, (head,) = run_config(args.config, [rule], args, torch, dev, cpu=not args.no_cpu_baseline)
    sustained = sustain_leg(layer, tens, head["tau"], args.sustain, torch) if args.sustain > 0 else None
    # BSA query pruning on the headline layer and mask (the Wan layer's leg runs under extra)
    qp_head = None
    if not args.no_legs and cfg.dtype == "bf16" and not cfg.global_pool:
        layer.mask(head["tau"])
        qp_head = query_pruning_leg(layer, cfg, tens[0], 10, torch, tau=head["tau"])
    del layer, tens
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "dense-equiv TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "fp32" else "bf16",
        "data": "synthetic (seeded smooth-field Q/K, iid V; no model weights)",
        "config": {
            "workload": head["workload"],
            "tau": head["tau"],
            "tau_rule": head["tau_rule"],
            "block_sparsity": head["block_sparsity"],
            "token_pairs_kept": head["token_pairs_kept"],
            "executed_attn_flop": head["executed_attn_flop"],
            "dense_equiv_flop": head["dense_equiv_flop"],
        },
        "roofline": head["roofline"],
        "stage_rooflines": head["stage_rooflines"],
        "stages_ms": head["stages_ms"],
        "step_streams": head["step_streams"],
        "step_ms_events": head["step_ms_events"],
        "graph_ms_per_step": head["graph_ms_per_step"],
        "graph_value": head["graph_value"],
        "input_gen_s": head["input_gen_s"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if sustained is not None:
        line["sustained"] = sustained
    if qp_head is not None:
        line["query_pruning"] = qp_head

    if not args.no_extra:
        extra = {"configs": {}}
        wan_layer = None
        for cid in [int(c) for c in args.configs.split(",") if c.strip()]:
            if cid == args.config or cid not in EXTRA_RUNS:
                continue
            c, lay, tens, results = run_config(cid, EXTRA_RUNS[cid], args, torch, dev, cpu=not args.no_cpu_baseline)
            for (mode, val), r in zip(EXTRA_RUNS[cid], results):
                extra["configs"][f"config{cid}_{'tau' if mode == 'tau' else 's'}{val:.2f}"] = r
            if not args.no_legs and cid == 2:
                lay.spec.tau = 0.90
                lay.forward(*tens, tau=0.90, keep_p_imp=True)
                torch.cuda.synchronize()
                extra["backward"] = backward_leg(lay, c, tens[0], tens[2], 10, 3, torch)
                extra["mask_rules"] = mask_rules_leg(lay, 20, torch)
                lay.mask(0.90)
                extra["query_pruning"] = query_pruning_leg(lay, c, tens[0], 20, torch)
                extra["pooled_estimates"] = pooled_leg(lay, c, tens[0], 20, torch)
                lay.mask(0.90)
                other = make_layer(c, dev, fused=args.unfused)
                ms_o, _ = run_steps(other, *tens, torch.empty_like(tens[0]), 0.90, args.steps, args.warmup, torch)
                extra["wan_tau0.90_unfused_ms_per_step" if not args.unfused else "wan_tau0.90_fused_ms_per_step"] = \
                    round(ms_o, 4)
                del other
            if not args.no_legs and cid == 5:
                step = results[0]["ms_per_step"] if results else None
                extra["sics_scheme_choice"] = sics_leg(c, tens[0], tens[1], 10, torch, step)
            del lay, tens
            torch.cuda.empty_cache()
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
