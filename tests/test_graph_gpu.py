"""The entry points under HIP graph capture.

The library enqueues kernels on the caller's stream and never allocates,
frees, clears memory or synchronises, so a captured sequence of fa_fwd,
fa_fwd_splitk (with a caller workspace) and fa_bwd must replay to the same
bits as eager calls.  Each replay here runs on fresh inputs copied into the
captured buffers, with eager work and synchronisation between replays, and
is compared bit for bit with eager calls on the same inputs; the first
replay is also checked against the oracle.
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
from gpu_cases import compare, device_to_f64, say, to_device  # noqa: E402

pytestmark = pytest.mark.gpu

REPLAYS = 4


def draw(seed, dtype="bf16"):
    w = synth.custom(f"graph seed {seed}", dtype, "bhsd", 2, 4, 300, 333, 128, causal=True,
                     seed=seed)
    inp = synth.make_inputs(w)
    return w, inp, synth.make_dout(w)


def run_all(fa, q, k, v, do, scale, ws, outs=None):
    """Forward, key-split forward and backward; into `outs` when given."""
    import torch
    o_out = outs["o"] if outs else None
    lse_out = outs["lse"] if outs else None
    o, lse = fa.forward(q, k, v, causal=True, sm_scale=scale, out=o_out, lse=lse_out)
    so, slse = fa.forward_splitk(q, k, v, causal=True, sm_scale=scale, num_splits=3,
                                 workspace=ws, out=outs["so"] if outs else None,
                                 lse=outs["slse"] if outs else None)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, sm_scale=scale,
                             dq=outs["dq"] if outs else None, dk=outs["dk"] if outs else None,
                             dv=outs["dv"] if outs else None,
                             delta=outs["delta"] if outs else None)
    res = {"o": o, "lse": lse, "so": so, "slse": slse, "dq": dq, "dk": dk, "dv": dv}
    if outs is None:
        res["delta"] = torch.empty_like(lse)
    return res


def test_graph_replays_match_eager():
    import torch
    import tiled_attention_04_amd as fa
    w, inp, dout = draw(700)
    q, k, v, do = (to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, dout))
    scale = w.sm_scale
    need = fa.fa_fwd_splitk_workspace(w.batch, w.heads, w.seq_q, w.head_dim, 3)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    # warm up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        outs = run_all(fa, q, k, v, do, scale, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all(fa, q, k, v, do, scale, ws, outs)
    torch.cuda.synchronize()

    for rep in range(REPLAYS):
        w_r, inp_r, dout_r = draw(710 + rep)
        for dst, src in zip((q, k, v, do), (inp_r.q, inp_r.k, inp_r.v, dout_r)):
            dst.copy_(to_device(src, "bf16"))
        torch.cuda.synchronize()
        say(f"[gpu] graph replay {rep} (inputs seed {710 + rep})")
        graph.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in outs.items()}
        # eager calls on the same inputs, between the replays
        ref = run_all(fa, q, k, v, do, scale, torch.empty_like(ws))
        torch.cuda.synchronize()
        for name in ("o", "lse", "so", "slse", "dq", "dk", "dv"):
            assert torch.equal(got[name], ref[name]), f"replay {rep}: {name} differs from eager"
        if rep == 0:
            o_ref, lse_ref = oracle.forward(inp_r.as_bhsd_f64("q"), inp_r.as_bhsd_f64("k"),
                                            inp_r.as_bhsd_f64("v"), scale, True)
            compare("graph replay 0", "bf16", device_to_f64(got["o"]), device_to_f64(got["lse"]),
                    o_ref, lse_ref)
            compare("graph replay 0 splitk", "bf16", device_to_f64(got["so"]),
                    device_to_f64(got["slse"]), o_ref, lse_ref)
        say(f"graph replay {rep}: all outputs bitwise equal to eager")


def test_graph_e5m2_and_fp32_forward():
    """The float8 e5m2 and fp32 forwards captured and replayed the same way."""
    import torch
    import tiled_attention_04_amd as fa
    shape = (2, 3, 200, 64)
    bufs = {
        "e5m2": [synth.device_normal(shape, "e5m2", 720 + i) for i in range(2)]
        + [synth.device_normal((2, 3, 64, 208), "e5m2", 722)],
        "fp32": [synth.device_normal(shape, "fp32", 730 + i, std=0.5) for i in range(3)],
    }
    for dtype, (q, k, v) in bufs.items():
        torch.cuda.synchronize()
        o, lse = fa.forward(q, k, v, causal=True)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fa.forward(q, k, v, causal=True, out=o, lse=lse)
        for rep in range(REPLAYS):
            for i, t in enumerate((q, k, v)):
                t.copy_(synth.device_normal(tuple(t.shape), dtype, 800 + 10 * rep + i,
                                            std=1.0 if dtype == "e5m2" else 0.5))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got_o, got_l = o.clone(), lse.clone()
            ref_o, ref_l = fa.forward(q, k, v, causal=True)
            torch.cuda.synchronize()
            assert torch.equal(got_o.view(torch.uint8) if dtype == "e5m2" else got_o,
                               ref_o.view(torch.uint8) if dtype == "e5m2" else ref_o), \
                f"{dtype} replay {rep}: O differs from eager"
            assert torch.equal(got_l, ref_l), f"{dtype} replay {rep}: lse differs from eager"
        say(f"graph {dtype}: {REPLAYS} replays bitwise equal to eager")
