"""GPU parity of the key-split forward (fa_fwd_splitk) against the CPU oracle.

Same tolerances as the forward (the target's: bf16/fp16 max-abs 2e-2 and
mean-abs 2e-3 for O and lse).  Covers explicit and automatic split counts,
ragged key tails, causal shares that are empty for some query tiles, the
fp16 [seq, heads, d] workload (16 heads, 1000 queries x 1537 keys) and short-query workloads with few query
tiles per head, equality with fa_fwd for one split, and workspace reuse.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from tiled_attention_04_amd import synth  # noqa: E402
from gpu_cases import compare, device_to_f64, gpu_bhsd_f64, say, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


def run_splitk(inp, num_splits, workspace=None):
    import torch
    import tiled_attention_04_amd as fa
    w = inp.workload
    q, k, v = (to_device(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    layout = "shd" if w.layout == "shd" else "bhsd"
    o, lse = fa.forward_splitk(q, k, v, causal=w.causal, sm_scale=w.sm_scale, layout=layout,
                               num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def splitk_parity(w, num_splits, workspace=None):
    inp = synth.make_inputs(w)
    import tiled_attention_04_amd as fa
    chosen = num_splits or fa.fa_fwd_splitk_choose(w.batch, w.heads, w.seq_q, w.seq_k,
                                                    w.head_dim, w.causal)
    say(f"[gpu] splitk {w.name}: {w.dtype} {w.layout} B={w.batch} H={w.heads} Sq={w.seq_q} "
        f"Sk={w.seq_k} D={w.head_dim} causal={w.causal} splits={chosen}")
    o, lse = run_splitk(inp, num_splits, workspace)
    o_ref, lse_ref = oracle.forward(inp.as_bhsd_f64("q"), inp.as_bhsd_f64("k"),
                                    inp.as_bhsd_f64("v"), w.sm_scale, w.causal)
    compare(f"splitk {w.name} s={chosen}", w.dtype, gpu_bhsd_f64(o, w.layout),
            device_to_f64(lse), o_ref, lse_ref)
    return chosen


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [2, 3, 5, 16])
def test_splitk_explicit(dtype, causal, splits):
    w = synth.custom("splitk ragged", dtype, "bhsd", 2, 3, 129, 700, 64, causal=causal, seed=31)
    splitk_parity(w, splits)


@pytest.mark.parametrize("head_dim", [32, 80, 128, 144, 192, 200, 256])
def test_splitk_head_dims(head_dim):
    w = synth.custom(f"splitk d{head_dim}", "bf16", "bhsd", 1, 4, 200, 1000, head_dim,
                     causal=True, seed=32)
    splitk_parity(w, 4)


@pytest.mark.parametrize("dtype,causal,splits", [("fp16", False, 3), ("bf16", True, 16)])
def test_splitk_head_dim_256_shares(dtype, causal, splits):
    # head_dim 256 with ragged shares; 16 splits leave most causal shares empty
    w = synth.custom("splitk d256 shares", dtype, "bhsd", 1, 3, 300, 650, 256, causal=causal,
                     seed=34)
    splitk_parity(w, splits)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_splitk_large_grid_shares(head_dim):
    # 1024 query tiles: 8-wave workgroups, whose shares of 5-6 key tiles
    # end inside the loop unrolled by four
    w = synth.custom(f"splitk large grid d{head_dim}", "bf16", "bhsd", 1, 1024, 100, 1000,
                     head_dim, causal=False, seed=36)
    splitk_parity(w, 3)


def test_splitk_more_splits_than_tiles():
    # causal, 2 key tiles per query tile at most: most shares are empty
    w = synth.custom("splitk empty shares", "bf16", "bhsd", 1, 2, 100, 100, 64, causal=True,
                     seed=33)
    splitk_parity(w, 8)


def test_splitk_c2_auto():
    # the choice for 16 heads of 1000 queries x 1537 keys is 1: the unsplit small-grid kernel splits its keys between
    # two wave groups of each workgroup instead
    assert splitk_parity(synth.WORKLOADS["c2"], 0) == 1
    assert splitk_parity(synth.WORKLOADS["c2"], 2) == 2


@pytest.mark.parametrize("seq_q", [10, 100])
def test_splitk_short_queries(seq_q):
    # few query rows against a long key sequence, [seq, heads, d] layout
    w = synth.custom(f"short q{seq_q}", "fp16", "shd", 1, 12, seq_q, 4096, 64, sm_scale=0.5,
                     seed=34)
    assert splitk_parity(w, 0) > 1


def test_splitk_one_split_equals_fa_fwd():
    import torch
    import tiled_attention_04_amd as fa
    w = synth.custom("splitk one", "bf16", "bhsd", 2, 4, 300, 500, 128, causal=True, seed=35)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    o1, l1 = fa.forward_splitk(q, k, v, causal=True, num_splits=1)
    o2, l2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitk_workspace_reuse_and_determinism():
    import torch
    import tiled_attention_04_amd as fa
    ws = torch.empty(fa.fa_fwd_splitk_workspace(1, 16, 1000, 64, 6), dtype=torch.uint8,
                     device="cuda")
    big = synth.custom("splitk reuse big", "fp16", "bhsd", 1, 16, 1000, 1537, 64, seed=36)
    small = synth.custom("splitk reuse small", "fp16", "bhsd", 1, 4, 300, 900, 64, causal=True,
                         seed=37)
    splitk_parity(big, 6, workspace=ws)
    splitk_parity(small, 3, workspace=ws)
    a = run_splitk(synth.make_inputs(small), 3, workspace=ws)
    b = run_splitk(synth.make_inputs(small), 3, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
