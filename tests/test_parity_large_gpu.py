"""Tensors larger than 4 GiB: every entry point addresses them with 64-bit
offsets.

Each case draws its inputs on the device (seeded, synth.device_normal) so
that one operand spans more than 2^32 bytes, runs the HIP path, and compares
whole heads chosen to sit before, across and past the 2^31 and 2^32 byte
marks with the CPU oracle, which gets host copies of those heads.  Heads are
independent in attention, so a head's oracle result needs only its own
slices.  Tolerances are the ones of the targeted tests (forward: max-abs 1e-4
fp32, 2e-2 / mean 2e-3 for 16-bit; backward: the gradient-scaled bounds;
e5m2: the rigorous bound of test_parity_e5m2_gpu.py).
"""
import gc
import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from tiled_attention_04_amd import synth  # noqa: E402
from gpu_cases import compare, say  # noqa: E402
import test_parity_bwd_gpu as bwd  # noqa: E402
import test_parity_e5m2_gpu as e8  # noqa: E402

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def heads_across(n_heads, head_bytes, extra_seed):
    """Heads whose first byte lies just before / at / after 2^31 and 2^32,
    the first and last head, and two more at random."""
    picks = {0, n_heads - 1}
    for mark in (1 << 31, 1 << 32):
        h = mark // head_bytes
        picks.update(x for x in (h - 1, h, h + 1) if 0 <= x < n_heads)
    rng = np.random.default_rng(extra_seed)
    picks.update(int(x) for x in rng.integers(0, n_heads, 2))
    return sorted(picks)


def host_heads(t, heads, layout="bhsd"):
    """float64 [n, 1, S, D] copies of heads of a [1, H, S, D] (or [1, S, H, D]) tensor."""
    import torch
    pick = (lambda h: t[0, :, h]) if layout == "bshd" else (lambda h: t[0, h])
    rows = [pick(h).to(torch.float32).cpu().numpy().astype(np.float64) for h in heads]
    return np.stack(rows)[:, None]


def free_device():
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_bf16():
    """bf16 q, k, v of [1, 33000, 512, 128]: 4.03 GiB each."""
    shape = (1, 33000, 512, 128)
    say(f"[gpu] large bf16 inputs {shape}")
    q = synth.device_normal(shape, "bf16", 9101)
    k = synth.device_normal(shape, "bf16", 9102)
    v = synth.device_normal(shape, "bf16", 9103)
    assert q.numel() * q.element_size() > 4 * GIB
    yield q, k, v
    del q, k, v
    free_device()


def test_forward_bf16_past_4gib(big_bf16):
    import torch
    import tiled_attention_04_amd as fa
    q, k, v = big_bf16
    scale = 1.0 / math.sqrt(128)
    say("[gpu] large fwd bf16 [1,33000,512,128] causal")
    o, lse = fa.forward(q, k, v, causal=True, sm_scale=scale)
    torch.cuda.synchronize()
    heads = heads_across(q.shape[1], 512 * 128 * 2, 1)
    o_ref, lse_ref = oracle.forward(host_heads(q, heads), host_heads(k, heads),
                                    host_heads(v, heads), scale, True)
    compare(f"large fwd heads {heads}", "bf16", host_heads(o, heads),
            lse[0, heads].double().cpu().numpy()[:, None], o_ref, lse_ref)
    del o, lse


def test_backward_bf16_past_4gib(big_bf16):
    import torch
    import tiled_attention_04_amd as fa
    q, k, v = big_bf16
    scale = 1.0 / math.sqrt(128)
    say("[gpu] large bwd bf16 [1,33000,512,128] causal")
    do = synth.device_normal(q.shape, "bf16", 9104)
    o, lse = fa.forward(q, k, v, causal=True, sm_scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, sm_scale=scale)
    torch.cuda.synchronize()
    del o, lse
    heads = heads_across(q.shape[1], 512 * 128 * 2, 2)
    refs = oracle.backward(host_heads(q, heads), host_heads(k, heads), host_heads(v, heads),
                           host_heads(do, heads), scale, True)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs[:3]):
        bwd.check(f"large bwd {name} heads {heads}", host_heads(g, heads), r)
    del do, dq, dk, dv
    free_device()


def test_forward_fp16_bshd_past_4gib():
    """[b, s, h, d] layout: a seq stride of 4.2M elements, so one 64-row tile
    spans 0.5 GiB and the tensor 4.03 GiB."""
    import torch
    import tiled_attention_04_amd as fa
    shape = (1, 512, 33000, 128)
    say(f"[gpu] large fwd fp16 bshd {shape} non-causal")
    q = synth.device_normal(shape, "fp16", 9111, std=0.5)
    k = synth.device_normal(shape, "fp16", 9112, std=0.5)
    v = synth.device_normal(shape, "fp16", 9113, std=0.5)
    o, lse = fa.forward(q, k, v, causal=False, sm_scale=0.3, layout="bshd")
    torch.cuda.synchronize()
    heads = heads_across(33000, 128 * 2, 3)
    o_ref, lse_ref = oracle.forward(host_heads(q, heads, "bshd"), host_heads(k, heads, "bshd"),
                                    host_heads(v, heads, "bshd"), 0.3, False)
    compare(f"large fwd bshd heads {heads}", "fp16", host_heads(o, heads, "bshd"),
            lse[0, heads].double().cpu().numpy()[:, None], o_ref, lse_ref)
    del q, k, v, o, lse
    free_device()


def test_forward_fp32_past_4gib():
    import torch
    import tiled_attention_04_amd as fa
    shape = (1, 16500, 512, 128)
    say(f"[gpu] large fwd fp32 {shape} causal")
    q = synth.device_normal(shape, "fp32", 9121, std=0.5)
    k = synth.device_normal(shape, "fp32", 9122, std=0.5)
    v = synth.device_normal(shape, "fp32", 9123, std=0.5)
    assert q.numel() * 4 > 4 * GIB
    scale = 1.0 / math.sqrt(128)
    o, lse = fa.forward(q, k, v, causal=True, sm_scale=scale)
    torch.cuda.synchronize()
    heads = heads_across(shape[1], 512 * 128 * 4, 4)
    o_ref, lse_ref = oracle.forward(host_heads(q, heads), host_heads(k, heads),
                                    host_heads(v, heads), scale, True)
    compare(f"large fwd fp32 heads {heads}", "fp32", host_heads(o, heads),
            lse[0, heads].double().cpu().numpy()[:, None], o_ref, lse_ref)
    del q, k, v, o, lse
    free_device()


def test_splitk_bf16_past_4gib():
    """16 queries per head against 4096 keys (K and V of 4.1 GiB each), keys
    split four ways."""
    import torch
    import tiled_attention_04_amd as fa
    H = 4200
    say(f"[gpu] large splitk bf16 q [1,{H},16,128] k/v [1,{H},4096,128]")
    q = synth.device_normal((1, H, 16, 128), "bf16", 9131)
    k = synth.device_normal((1, H, 4096, 128), "bf16", 9132)
    v = synth.device_normal((1, H, 4096, 128), "bf16", 9133)
    assert k.numel() * 2 > 4 * GIB
    scale = 1.0 / math.sqrt(128)
    o, lse = fa.forward_splitk(q, k, v, causal=False, sm_scale=scale, num_splits=4)
    torch.cuda.synchronize()
    heads = heads_across(H, 4096 * 128 * 2, 5)
    o_ref, lse_ref = oracle.forward(host_heads(q, heads), host_heads(k, heads),
                                    host_heads(v, heads), scale, False)
    compare(f"large splitk heads {heads}", "bf16", host_heads(o, heads),
            lse[0, heads].double().cpu().numpy()[:, None], o_ref, lse_ref)
    del q, k, v, o, lse
    free_device()


def test_e5m2_past_4gib():
    """float8 e5m2 q, k of [1, 66000, 512, 128] and key-major V [1, 66000, 128, 512]:
    4.03 GiB each."""
    import torch
    import tiled_attention_04_amd as fa
    H, S, D = 66000, 512, 128
    say(f"[gpu] large fwd e5m2 [1,{H},{S},{D}] non-causal")
    q = synth.device_normal((1, H, S, D), "e5m2", 9141)
    k = synth.device_normal((1, H, S, D), "e5m2", 9142)
    vt = synth.device_normal((1, H, D, S), "e5m2", 9143)
    assert q.numel() > 4 * GIB
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.forward(q, k, vt, causal=False, sm_scale=scale)
    torch.cuda.synchronize()
    heads = heads_across(H, S * D, 6)
    q64, k64 = host_heads(q, heads), host_heads(k, heads)
    v64 = np.stack([vt[0, h].to(torch.float32).cpu().numpy().astype(np.float64).T
                    for h in heads])[:, None]
    o_ref, lse_ref = oracle.forward(q64, k64, v64, scale, False)
    o_abs, _ = oracle.forward(q64, k64, np.abs(v64), scale, False)
    vsum = np.abs(v64).sum(axis=2, keepdims=True)
    delta = e8.score_delta(q64, k64, scale, False)
    e8.check_bound(f"large e5m2 heads {heads}", host_heads(o, heads),
                   lse[0, heads].double().cpu().numpy()[:, None], o_ref, o_abs, vsum, lse_ref,
                   delta)
    del q, k, vt, o, lse
    free_device()
