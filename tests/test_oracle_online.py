"""The tiled online-softmax recurrence (the algorithm the kernels implement)
reaches the plain definition: a float64 CPU model of it, block by block with
the pages' update rules, against the materialised oracle, for many block
shapes, ragged sizes, causal or not, large logits, and the lazy refresh of
the running maximum that the kernels use (refresh only when the block
maximum exceeds it by more than 8 in base-2 units)."""
import math

import numpy as np
import pytest

import oracle
from oracle import oracle_np


def _inputs(seed, b, h, sq, sk, d, big_rows=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, h, sq, d))
    k = rng.standard_normal((b, h, sk, d))
    v = rng.standard_normal((b, h, sk, d))
    if big_rows:
        idx = rng.choice(sk, size=big_rows, replace=False)
        k[:, :, idx] *= 8.0
    return q, k, v


@pytest.mark.parametrize("block_m,block_n", [(1, 1), (3, 3), (16, 16), (64, 64), (128, 64),
                                             (3, 128), (128, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_matches_definition(block_m, block_n, causal):
    q, k, v = _inputs(1, 1, 2, 131, 157, 24, big_rows=4)
    scale = 1 / math.sqrt(24)
    o_ref, lse_ref = oracle.forward(q, k, v, scale, causal)
    o, lse = oracle_np.attention_forward_tiled(q, k, v, scale, causal, block_m, block_n)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,sk", [(1, 1), (5, 200), (200, 5), (257, 300)])
def test_lazy_max_refresh_is_exact(causal, sq, sk):
    # the kernels' threshold: 8 in base-2 units = 8 ln 2 natural-log units
    q, k, v = _inputs(2, 2, 1, sq, sk, 16, big_rows=min(sk, 6))
    scale = 0.7
    o_ref, lse_ref = oracle.forward(q, k, v, scale, causal)
    o, lse = oracle_np.attention_forward_tiled(q, k, v, scale, causal, 128, 64,
                                               lazy_threshold=8 * math.log(2.0))
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


def test_lazy_refresh_is_exercised():
    # rising scores along the keys: every block max exceeds the previous one,
    # so a refresh threshold of 8 ln 2 skips some refreshes and takes others
    sk, d = 256, 4
    q = np.ones((1, 1, 1, d))
    k = np.zeros((1, 1, sk, d))
    k[0, 0, :, 0] = np.linspace(0.0, 30.0, sk)
    v = np.random.default_rng(3).standard_normal((1, 1, sk, d))
    o_ref, lse_ref = oracle.forward(q, k, v, 1.0, False)
    for thr in (0.0, 8 * math.log(2.0), 100.0):
        o, lse = oracle_np.attention_forward_tiled(q, k, v, 1.0, False, 1, 16, lazy_threshold=thr)
        assert np.max(np.abs(o - o_ref)) <= 1e-12
        assert abs(lse[0, 0, 0] - lse_ref[0, 0, 0]) <= 1e-12


@pytest.mark.parametrize("block_m,block_n", [(1, 1), (3, 5), (16, 64), (128, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_two_phase_backward_matches_definition(block_m, block_n, causal):
    # the kernels' backward split (dQ per query block, dK/dV per key block,
    # P recomputed from L in both) against the materialised gradients
    q, k, v = _inputs(4, 1, 2, 70, 93, 12, big_rows=3)
    dout = np.random.default_rng(5).standard_normal(q.shape)
    scale = -0.4 if causal else 0.3
    ref = oracle_np.attention_backward(q, k, v, dout, scale, causal)
    got = oracle_np.attention_backward_tiled(q, k, v, dout, scale, causal, block_m, block_n)
    for g, r in zip(got, ref[:3]):
        assert np.max(np.abs(g - r)) <= 1e-12 * max(1.0, np.max(np.abs(r)))
