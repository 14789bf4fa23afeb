"""Pins for sparsity/work accounting and the generator's determinism."""
import json
import os

import numpy as np

from oracle.accounting import (block_sparsity, combined_sparsity, dense_flop, executed_flop,
                               token_sparsity)
from workloads import get_config, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bsa_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "bsa_example.json")))
    assert round(g["tokens"] * g["query_keep"]) == g["queries_kept"]
    assert abs(combined_sparsity(g["query_keep"], g["kv_keep"]) - g["sparsity"]) < 1e-12


def test_block_and_token_sparsity():
    nb, N, b = 4, 60, 16            # last block holds 12 tokens
    cnt = np.array([[4, 4, 4, 4]])
    idx = np.tile(np.arange(4), (1, 4, 1))
    assert block_sparsity(cnt, nb) == 0.0
    assert abs(token_sparsity(cnt, idx, N, b)) < 1e-12
    cnt1 = np.array([[1, 1, 1, 1]])
    idx1 = np.tile(np.arange(4)[:, None], (1, 1, 4))
    assert block_sparsity(cnt1, nb) == 0.75
    kept = 3 * 16 * 16 + 12 * 12
    assert abs(token_sparsity(cnt1, idx1, N, b) - (1 - kept / 3600)) < 1e-12
    assert executed_flop(cnt1, idx1, N, b, 8, 1) == 4 * 8 * kept
    assert executed_flop(cnt1, idx1, N, b, 8, 1, Ng=2) == 4 * 8 * kept + 4 * 8 * 60 * 2


def test_dense_flop_wan():
    assert abs(dense_flop(1, 12, 32760, 128) - 6.594e12) / 6.594e12 < 1e-3
    assert get_config(2).dense_flop() == dense_flop(1, 12, 32760, 128)


def test_generator_deterministic_and_bf16():
    cfg = get_config(1)
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    cfg3 = get_config(3)
    q, k, v = make_inputs(cfg3, heads=[0])
    bits = q.view(np.uint32)
    assert (bits & 0xFFFF == 0).all()          # bf16-representable
    assert q.shape == (1, 17776, 1, 64)
    # text prefix is iid: no correlation between neighbouring text tokens
    t = q[0, :226, 0]
    assert abs(np.mean(np.sum(t[1:] * t[:-1], axis=1))) / 64 < 0.2
    # video tokens: neighbours strongly correlated (smooth field)
    vq = q[0, 226:, 0]
    assert np.mean(np.sum(vq[1:] * vq[:-1], axis=1)) / 64 > 0.5
