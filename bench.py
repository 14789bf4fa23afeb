#!/usr/bin/env python3
"""Benchmark: one ASA attention layer forward on one MI355X.

Workload: the Wan2.1-1.3B-shaped self-attention layer -- batch 1, 12 heads,
head dim 128, bf16, latent 21 x 30 x 52 = 32,760 tokens (padded to 32,768),
smooth-field Q/K (sigma 4) + 0.3 noise, iid V; b = 128, k = 16, Gilbert-curve
reorder, threshold tau = 0.90 (tau = 0.95 is measured as well and reported
under "extra", and so is the backward of the attention at tau = 0.90).
Synthetic inputs stand in for the model's activations.

A step is one pass of the whole hot path over that batch, all on one stream:
reorder K, V -> estimate_mask (the sampled estimate, sampled Q rows read in
token order, with the cumulative-threshold selection fused into its final
launch, so P_imp never reaches HBM) -> sparse_attn_fwd (Q read and the output
written in token order, so the return to token order is part of that launch).
With --unfused the estimate and the mask run as two calls (estimate_blocks,
build_mask), the layout the unfused time under "extra" is measured with.  Inputs are resident in
HBM before timing starts; buffers and the permutation are set up once outside
the timed region.

value = dense-equivalent TFLOP/s = 4 * B * H * N^2 * d / (seconds per step).
The timed region holds HIP events at its two ends only; the per-stage
breakdown ("stages_ms") comes from a separate untimed pass of the same steps
with HIP events between the stages on the launch stream.
roofline = the attention kernel (the dominant one): executed FLOP (4 * d *
sum over kept block pairs of |I| * |J|) / its mean launch time from that
breakdown pass, against the bf16 dense MFMA peak.  cpu_baseline = the CPU oracle on a bounded sample of the
same layer (two of the twelve heads in full), scaled to the whole layer.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan_traffic.json")
ATTN_SRC = os.path.join(ROOT, "dynamic_block_sparse_gilbert_amd", "csrc", "kernels", "attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--tau", type=float, default=0.90)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="estimate and mask as two calls")
    ap.add_argument("--no-extra", action="store_true", help="skip the tau=0.95 and backward measurements")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def src_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kept_pair_tokens(cnt, idx, N, b, q_rows=None):
    """sum over kept (I, J) of |I| * |J| with valid-token block sizes; q_rows (same shape as cnt):
    the query rows computed per block instead of |I| (pruned queries)."""
    import numpy as np
    nb = cnt.shape[-1]
    L = np.array([min(b, N - J * b) for J in range(nb)], dtype=np.float64)
    c = cnt.reshape(-1, nb)
    ix = idx.reshape(-1, nb, nb)
    qr = None if q_rows is None else q_rows.reshape(-1, nb)
    total = 0.0
    for r in range(c.shape[0]):
        for I in range(nb):
            total += (L[I] if qr is None else qr[r, I]) * L[ix[r, I, :c[r, I]]].sum()
    return total


def run_steps(layer, q, k, v, out, tau, steps, warmup, torch):
    """The timed region: `steps` whole layer steps, back to back on one stream, with HIP events
    only at its two ends (an event between kernels costs a cache write-back of its own).
    Returns (host ms per step between synchronisations, event ms per step)."""
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


def stage_times(layer, q, k, v, out, tau, steps, torch):
    """Per-stage breakdown in a separate, untimed pass over the same steps: HIP events on the
    launch stream between the stages of each step (each stage time carries one event's cost).
    The attention entry is the mean attention launch duration used for the roofline."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    names = ["reorder_kv", "estimate_mask", "attn"] if layer.fused else ["reorder_kv", "estimate", "mask", "attn"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for s in range(steps):
        e = ev[s]
        e[0].record()
        layer.prepare(q, k, v)
        e[1].record()
        if layer.fused:
            layer.mask(tau)
        else:
            ops.estimate_blocks_tok(q, layer.perm, layer.k_r, sp.N, sp.b, sp.k, sp.scale, p_imp=layer.p_imp,
                                    workspace=layer.ws)
            e[2].record()
            ops.build_mask(layer.p_imp, tau, kv_count=layer.kv_count, kv_idx=layer.kv_idx, order=layer.order)
        e[len(names) - 1].record()
        layer.wait_v()   # V is reordered on a side stream
        ops.sparse_attn_fwd_tok(q, layer.perm, layer.k_r, layer.v_t, sp.N, sp.b, sp.scale, layer.kv_count,
                                layer.kv_idx, layer.k_g, layer.v_g, layer.Ng, sp.n_pool, out=out,
                                order=layer.order)
        e[len(names)].record()
    torch.cuda.synchronize()
    return {n: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
            for i, n in enumerate(names)}


def backward_leg(layer, cfg, qd, vd, steps, warmup, torch):
    """The backward of the attention (plain ASA) on the same layer and mask: the key-to-query lists
    and the dQ / dK / dV kernels, timed back to back between two HIP events.  Q, V (rows) and dO are
    reordered and the forward's output and lse computed beforehand, outside the timed region."""
    import numpy as np
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
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    cnt, idx = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy()
    pairs = kept_pair_tokens(cnt, idx, sp.N, sp.b)
    alg = 10.0 * sp.d * pairs        # five products over the kept pairs (S, dP, dV, dQ, dK)
    executed = 14.0 * sp.d * pairs   # S and dP are computed in both kernels
    return {
        "ms": round(ms, 4),
        "what": "dbs_transpose_lists + dbs_sparse_attn_bwd (rows -> tiles copies, dQ, dK/dV kernels), "
                "tau 0.9 mask of the timed layer",
        "algorithmic_flop": alg,
        "executed_flop": executed,
        "algorithmic_tflops": round(alg / (ms * 1e-3) / 1e12, 1),
        "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 1),
        "executed_frac_of_bf16_peak": round(executed / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
    }


def mask_rules_leg(layer, steps, torch):
    """The alternative selection rules on the timed layer's P_imp: the kept-block lists under the
    cumulative threshold (tau 0.9), top-k (k = 16) and the statistical cutoff (u = U(1 - 16/nb)),
    each launched `steps` times back to back between two HIP events."""
    from dynamic_block_sparse_gilbert_amd import ops
    nb = layer.p_imp.shape[-1]
    out = {}
    for name, rule, param in (("cumulative_tau0.9", "cumulative", 0.9), ("topk_16", "topk", 16),
                              ("stat_k16", "stat", ops.stat_quantile(16, nb))):
        ops.build_mask_rule(layer.p_imp, rule, param, kv_count=layer.kv_count, kv_idx=layer.kv_idx)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            ops.build_mask_rule(layer.p_imp, rule, param, kv_count=layer.kv_count, kv_idx=layer.kv_idx)
        e1.record()
        torch.cuda.synchronize()
        cnt = layer.kv_count.cpu().numpy()
        out[name] = {"us": round(e0.elapsed_time(e1) / steps * 1e3, 2),
                     "block_sparsity": round(float(1.0 - cnt.sum() / (cnt.size * nb)), 4)}
    return out


def query_pruning_leg(layer, cfg, qd, steps, torch, r=0.5, win=(2, 2, 2)):
    """BSA query pruning on the timed layer and mask: the kept rows (centres of 2 x 2 x 2 windows plus
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

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    t_prune, t_pruned, t_full = timed(prune), timed(pruned), timed(full)
    cnt, idx, qch = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy(), qc.cpu().numpy()
    kept_q = float(qch.sum()) / (qch.shape[0] * qch.shape[1] * sp.N)
    # key blocks streamed by the paired work items (blocks 2P, 2P + 1 over the union of their lists)
    # against the two lists' own lengths
    nb = cnt.shape[-1]
    c2, i2 = cnt.reshape(-1, nb), idx.reshape(-1, nb, nb)
    own = float(c2.sum())
    union = 0.0
    for r_ in range(c2.shape[0]):
        for I in range(0, nb - 1, 2):
            union += len(set(i2[r_, I, :c2[r_, I]].tolist()) | set(i2[r_, I + 1, :c2[r_, I + 1]].tolist()))
    ef = 4.0 * sp.d * kept_pair_tokens(cnt, idx, sp.N, sp.b, q_rows=qch)
    kv_keep = 1.0 - float(1.0 - cnt.sum() / (cnt.size * cnt.shape[-1]))
    return {
        "what": "dbs_query_prune + dbs_sparse_attn_fwd_pruned_tok (64-row work items, then token filling), "
                "2x2x2 centre windows, keep ratio %.2f, on the tau %.2f mask of the timed layer" % (r, sp.tau),
        "query_keep": round(kept_q, 4),
        "kv_block_keep": round(kv_keep, 4),
        "combined_sparsity": round(1.0 - kept_q * kv_keep, 4),
        "prune_us": round(t_prune * 1e3, 2),
        "pruned_attn_ms": round(t_pruned, 4),
        "unpruned_attn_ms": round(t_full, 4),
        "pruned_attn_executed_tflops": round(ef / (t_pruned * 1e-3) / 1e12, 2),
        "pair_union_over_own_blocks": round(2.0 * union / own, 4),
    }


def pooled_leg(layer, cfg, qd, steps, torch):
    """The pooled estimates (MEAN, TRIP) on the timed layer, each timed back to back between two HIP
    events with the cumulative mask they give at the layer's tau, and the SICS aggregation score of
    four cuboid block shapes (one call each)."""
    from dynamic_block_sparse_gilbert_amd import ops
    sp = layer.spec
    out = {}
    ws = torch.empty(max(16, ops.lib().dbs_pooled_workspace_bytes(1, sp.heads, sp.N, sp.d, sp.b)), dtype=torch.uint8,
                     device=qd.device)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    for kind in ("mean", "trip"):
        t = timed(lambda: ops.estimate_pooled(qd, layer.perm, layer.k_r, sp.N, sp.b, kind, p_imp=layer.p_imp,
                                              workspace=ws))
        cnt, _, _ = ops.build_mask(layer.p_imp, sp.tau)
        c = cnt.cpu().numpy()
        out[kind] = {"us": round(t * 1e3, 2), "block_sparsity_at_tau": round(float(1 - c.sum() / (c.size * sp.nb)), 4)}
    cands = [(1, 8, 16), (2, 8, 8), (4, 4, 8), (1, 4, 32)]
    t0 = time.perf_counter()
    choice, scores = ops.choose_cuboids_sics(qd, cfg.T, cfg.H, cfg.W, cands, sp.b)
    torch.cuda.synchronize()
    out["sics"] = {"candidates": [list(c) for c in cands], "choice_per_head": choice.cpu().numpy()[0].tolist(),
                   "wall_ms_4_candidates": round((time.perf_counter() - t0) * 1e3, 2)}
    return out


def cpu_baseline(cfg, q, k, v, perm, tau, heads=2):
    """The oracle, as it stands, on a bounded sample of the same layer: the first
    `heads` heads in full (estimator, mask, attention over every query block),
    scaled to all heads."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.attention import masked_attention
    from oracle.estimator import p_imp
    from oracle.mask import build_mask
    from oracle.reorder import reorder_fast

    t_est = t_mask = t_attn = 0.0
    for h in range(heads):
        x = [reorder_fast(t[:, :, h:h + 1], perm, cfg.Npad)[0, 0] for t in (q, k, v)]
        t0 = time.perf_counter()
        P = p_imp(x[0], x[1], cfg.N, cfg.b, cfg.k, cfg.scale).astype(np.float32)
        t_est += time.perf_counter() - t0
        t0 = time.perf_counter()
        cnt, idx, _, _ = build_mask(P, tau)
        t_mask += time.perf_counter() - t0
        kept = [idx[I, :cnt[I]].tolist() for I in range(cfg.nb)]
        t0 = time.perf_counter()
        masked_attention(x[0], x[1], x[2], cfg.N, cfg.b, kept, cfg.scale)
        t_attn += time.perf_counter() - t0
    sample = t_est + t_mask + t_attn
    total = sample * cfg.heads / heads
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": cfg.dense_flop() / total / 1e12,
        "unit": "dense-equiv TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"heads 0-{heads - 1} of {cfg.heads} in full: estimator {t_est:.2f} s, mask {t_mask:.2f} s, "
                   f"attention over all {cfg.nb} query blocks {t_attn:.2f} s ({sample:.1f} s of CPU work); "
                   f"scaled x{cfg.heads / heads:g} heads -> {total:.1f} s per layer"),
        "host_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): every step of the path is "
              "independent per head, so several GPUs would each run a share of the heads; that "
              "configuration is not part of this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    from workloads import get_config, make_inputs

    cfg = get_config(2)
    t_gen = time.perf_counter()
    q, k, v = make_inputs(cfg)                    # bf16-representable float32 [1, N, 12, 128]
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    qd, kd, vd = to(q), to(k), to(v)
    out = torch.empty_like(qd)
    spec = LayerSpec(T=cfg.T, H=cfg.H, W=cfg.W, heads=cfg.heads, d=cfg.d, b=cfg.b, k=cfg.k, tau=args.tau)
    layer = AsaLayer(spec, device=dev, fused=not args.unfused)
    torch.cuda.synchronize()

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms, ms_ev = run_steps(layer, qd, kd, vd, out, args.tau, args.steps, args.warmup, torch)
    stage = stage_times(layer, qd, kd, vd, out, args.tau, args.steps, torch)
    attn_ms = stage["attn"]
    cnt, idx = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy()
    nb = cfg.nb
    sparsity = 1.0 - cnt.sum() / (cnt.size * nb)
    pairs = kept_pair_tokens(cnt, idx, cfg.N, cfg.b)
    exec_flop = 4.0 * cfg.d * pairs
    attn_tflops = exec_flop / (attn_ms * 1e-3) / 1e12
    dense = cfg.dense_flop()

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tj = json.load(open(TRAFFIC_FILE))
            if tj.get("attn_src_sha256_16") == src_hash(ATTN_SRC) and abs(tj.get("tau", -1) - args.tau) < 1e-9:
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    # byte passes: reorder of K, V (read + write) and P_imp read / kv lists write
    e = 2
    reorder_bytes = 2.0 * 2 * cfg.heads * cfg.N * cfg.d * e
    mask_bytes = 4.0 * cfg.heads * nb * nb + 4.0 * cfg.heads * (nb + cnt.sum())
    byte_passes = {"reorder_kv_GBs": round(reorder_bytes / (stage["reorder_kv"] * 1e-3) / 1e9, 1)}
    if "mask" in stage:
        byte_passes["mask_GBs"] = round(mask_bytes / (stage["mask"] * 1e-3) / 1e9, 1)
    byte_passes["hbm_peak_GBs"] = HBM_PEAK_GBS

    extra = {}
    if not args.no_extra:
        n95 = max(5, args.steps // 2)
        ms95, _ = run_steps(layer, qd, kd, vd, out, 0.95, n95, 2, torch)
        stage95 = stage_times(layer, qd, kd, vd, out, 0.95, n95, torch)
        attn95 = stage95["attn"]
        c95, i95 = layer.kv_count.cpu().numpy(), layer.kv_idx.cpu().numpy()
        ef95 = 4.0 * cfg.d * kept_pair_tokens(c95, i95, cfg.N, cfg.b)
        extra["tau_0.95"] = {
            "ms_per_step": round(ms95, 4),
            "value": round(dense / (ms95 * 1e-3) / 1e12, 2),
            "block_sparsity": round(float(1.0 - c95.sum() / (c95.size * nb)), 4),
            "stages_ms": {kk: round(vv, 4) for kk, vv in stage95.items()},
            "attn_executed_tflops": round(ef95 / (attn95 * 1e-3) / 1e12, 2),
        }
        layer.forward(qd, kd, vd, out=out, tau=args.tau)   # the timed mask again
        layer.mask(args.tau, keep_p_imp=True)              # and its P_imp, for the rule comparison
        torch.cuda.synchronize()
        extra["backward"] = backward_leg(layer, cfg, qd, vd, max(5, args.steps // 5), 3, torch)
        extra["mask_rules"] = mask_rules_leg(layer, 20, torch)
        layer.mask(args.tau)
        extra["query_pruning"] = query_pruning_leg(layer, cfg, qd, 20, torch)
        extra["pooled_estimates"] = pooled_leg(layer, cfg, qd, 20, torch)
        layer.mask(args.tau)
        other = AsaLayer(spec, device=dev, fused=args.unfused)
        ms_o, _ = run_steps(other, qd, kd, vd, out, args.tau, args.steps, args.warmup, torch)
        extra["unfused_ms_per_step" if not args.unfused else "fused_ms_per_step"] = round(ms_o, 4)
        del other

    line = {
        "metric": "ms/layer + dense-equiv TFLOP/s, block-sparse attn at 90-95% sparsity, 1 GPU",
        "value": round(dense / (ms * 1e-3) / 1e12, 3),
        "unit": "dense-equiv TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth-field Q/K, iid V; no model weights)",
        "config": {
            "workload": "wan2.1-1.3b-shaped ASA layer: B=1, 12 heads, d=128, 21x30x52 = 32,760 tokens, "
                        "b=128, k=16, Gilbert reorder",
            "tau": args.tau,
            "block_sparsity": round(float(sparsity), 4),
            "token_pairs_kept": pairs,
            "executed_attn_flop": exec_flop,
            "dense_equiv_flop": dense,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel<128,128>",
            "achieved": round(attn_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "launch_ms": round(attn_ms, 4),
        },
        "stages_ms": {kk: round(vv, 4) for kk, vv in stage.items()},
        "byte_passes": byte_passes,
        "step_ms_events": round(ms_ev, 4),
        "input_gen_s": round(t_gen, 2),
    }
    if extra:
        line["extra"] = extra
    if not args.no_cpu_baseline:
        perm = layer.perm.cpu().numpy()
        line["cpu_baseline"] = cpu_baseline(cfg, q, k, v, perm, args.tau)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
