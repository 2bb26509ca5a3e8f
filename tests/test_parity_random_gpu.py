"""Seeded random configurations through every entry point, against the oracle.

Each case draws, from its own seed, a dtype, batch, heads, sequence lengths
(including 1 and lengths that are no multiple of any tile), a head_dim the
dtype allows, the layout, causal or not and a scale of either sign, then
compares the HIP path with the CPU oracle at the same bounds as the targeted
tests: the forward's tolerances for fa_fwd and fa_fwd_splitk, the
gradient-scaled bounds for fa_bwd (see test_parity_bwd_gpu.py).  The draws
are fixed by the seeds, so a failure names a reproducible case.
"""
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
from gpu_cases import compare, device_to_f64, gpu_bhsd_f64, run_gpu, say  # noqa: E402
import test_parity_bwd_gpu as bwd  # noqa: E402

pytestmark = pytest.mark.gpu


def draw_case(seed, backward=False):
    rng = np.random.default_rng(1000 + seed)
    dtype = str(rng.choice(["bf16", "fp16", "fp32"]))
    layout = str(rng.choice(["bhsd", "shd"]))
    batch = 1 if layout == "shd" else int(rng.integers(1, 4))
    heads = int(rng.integers(1, 5))
    seq_q = int(rng.choice([1, int(rng.integers(2, 80)), int(rng.integers(80, 400))]))
    seq_k = int(rng.choice([1, int(rng.integers(2, 80)), int(rng.integers(80, 500))]))
    step = 4 if dtype == "fp32" else 8
    d_max = 128 if (backward and dtype == "fp32") else 256
    head_dim = int(rng.integers(1, d_max // step + 1)) * step
    causal = bool(rng.integers(0, 2))
    scale = float(rng.choice([-1.0, 1.0]) * rng.uniform(0.05, 1.5) / math.sqrt(head_dim))
    name = (f"rand{seed} {dtype} {layout} B{batch} H{heads} Sq{seq_q} Sk{seq_k} D{head_dim} "
            f"causal={causal} scale={scale:.4f}")
    return synth.custom(name, dtype, layout, batch, heads, seq_q, seq_k, head_dim, std=1.0,
                        sm_scale=scale, causal=causal, seed=2000 + seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_forward(seed):
    w = draw_case(seed)
    inp = synth.make_inputs(w)
    say(f"[gpu] {w.name}")
    o, lse = run_gpu(inp)
    o_ref, lse_ref = oracle.forward(inp.as_bhsd_f64("q"), inp.as_bhsd_f64("k"),
                                    inp.as_bhsd_f64("v"), w.sm_scale, w.causal)
    compare(w.name, w.dtype, gpu_bhsd_f64(o, w.layout), device_to_f64(lse), o_ref, lse_ref)


@pytest.mark.parametrize("seed", range(12))
def test_random_splitk(seed):
    import torch
    import tiled_attention_04_amd as fa
    w = draw_case(100 + seed)
    if w.dtype == "fp32":  # key splitting takes 16-bit inputs only
        w = synth.custom(w.name.replace("fp32", "bf16"), "bf16", w.layout, w.batch, w.heads,
                         w.seq_q, w.seq_k, (w.head_dim + 7) // 8 * 8, sm_scale=w.sm_scale,
                         causal=w.causal, seed=w.seed)
    splits = int(np.random.default_rng(3000 + seed).integers(0, 17))
    inp = synth.make_inputs(w)
    say(f"[gpu] splitk {w.name} splits={splits}")
    q, k, v = (bwd.to_device(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    layout = "shd" if w.layout == "shd" else "bhsd"
    o, lse = fa.forward_splitk(q, k, v, causal=w.causal, sm_scale=w.sm_scale, layout=layout,
                               num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(inp.as_bhsd_f64("q"), inp.as_bhsd_f64("k"),
                                    inp.as_bhsd_f64("v"), w.sm_scale, w.causal)
    compare(f"splitk {w.name}", w.dtype, gpu_bhsd_f64(o, w.layout), device_to_f64(lse), o_ref,
            lse_ref)


@pytest.mark.parametrize("seed", range(16))
def test_random_backward(seed):
    w = draw_case(200 + seed, backward=True)
    bwd.full_bwd_parity(w)
