"""GPU: the layer step recorded as a HIP graph (AsaLayer.capture) replays bit for bit like the
eager step. Each case replays the graph three times, with its bound buffers refilled in place
between replays and with eager work and synchronisations of the program in between; every
replay's output and kept-block lists are compared with an eager forward pass of a second layer
on the same inputs. The eager path itself is checked against the oracle by the layer tests."""
import numpy as np
import pytest
import torch

from gpu_helpers import say
from workloads import get_config, make_inputs
from workloads.generator import head_cuboid

pytestmark = pytest.mark.gpu


def _layer(cfg, nheads, tau):
    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    cub = [head_cuboid(cfg, h) for h in range(nheads)] if cfg.reorder == "cuboid_per_head" else None
    spec = LayerSpec(T=cfg.T, H=cfg.H, W=cfg.W, heads=nheads, d=cfg.d, b=cfg.b, k=cfg.k, tau=tau,
                     prefix=cfg.text_prefix, order=cfg.reorder, cuboid=cfg.cuboid, cuboids=cub,
                     n_pool=cfg.global_pool, dtype=cfg.dtype)
    return AsaLayer(spec)


def _inputs(cfg, heads):
    dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
    return [torch.from_numpy(a).to(dt).cuda() for a in make_inputs(cfg, heads=heads, workers=4)]


# the tiny float32 layer, the Wan and CogVideoX shapes (register-sorted masks, a work order, ASA_G),
# and the long layers (radix-selected masks over 1,200 and 872 blocks, per-head orders at 720p)
@pytest.mark.parametrize("cid,nheads,tau", [(1, 1, 0.9), (2, 2, 0.9), (3, 2, 0.95), (4, 1, 0.86), (5, 2, 0.9)])
def test_graph_replay_equals_eager(cid, nheads, tau):
    say("graph replay", cid, nheads, tau)
    cfg = get_config(cid)
    a = _inputs(cfg, list(range(nheads)))
    b = _inputs(cfg, list(range(nheads, 2 * nheads)))
    g_layer, e_layer = _layer(cfg, nheads, tau), _layer(cfg, nheads, tau)
    qg, kg, vg = (x.clone() for x in a)
    out_g = torch.empty_like(qg)
    graph = g_layer.capture(qg, kg, vg, out_g, tau=tau)
    out_e = torch.empty_like(qg)
    scratch = torch.empty_like(qg)

    def check(src, what):
        e_layer.forward(*src, out=out_e, tau=tau, out_dtype=out_e.dtype)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"{what}: output differs from the eager step"
        assert torch.equal(g_layer.kv_count, e_layer.kv_count), f"{what}: kv_count differs"
        cnt = e_layer.kv_count.cpu().numpy().reshape(-1)
        ig = g_layer.kv_idx.cpu().numpy().reshape(cnt.size, -1)
        ie = e_layer.kv_idx.cpu().numpy().reshape(cnt.size, -1)
        for r in range(cnt.size):
            assert np.array_equal(ig[r, :cnt[r]], ie[r, :cnt[r]]), f"{what}: kv_idx row {r} differs"

    graph.replay()
    check(a, "replay 1")
    for x, y in zip((qg, kg, vg), b):   # refill the bound inputs in place
        x.copy_(y)
    graph.replay()
    check(b, "replay 2")
    # eager work of the program on the graph's own layer between replays
    g_layer.forward(*a, out=scratch, tau=tau, out_dtype=scratch.dtype)
    torch.cuda.synchronize()
    graph.replay()
    check(b, "replay 3")
    assert torch.isfinite(out_g.float()).all()


def test_capture_rejects_two_stream_layer():
    from dynamic_block_sparse_gilbert_amd.layer import AsaLayer, LayerSpec
    cfg = get_config(2)
    spec = LayerSpec(T=cfg.T, H=cfg.H, W=cfg.W, heads=1, d=cfg.d, b=cfg.b, k=cfg.k, tau=0.9,
                     order=cfg.reorder, dtype=cfg.dtype)
    layer = AsaLayer(spec, overlap=True)
    x = torch.zeros((1, cfg.N, 1, cfg.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="one-stream"):
        layer.capture(x, x, x, torch.empty_like(x))
