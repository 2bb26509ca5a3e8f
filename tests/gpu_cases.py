"""Shared helpers of the GPU parity tests: upload seeded inputs, call the HIP
path through its C ABI binding, and compare with the CPU oracle."""
import sys

import numpy as np

import oracle
from tiled_attention_04_amd import synth

# Tolerances for O and lse, as the target states them.
TOL = {"fp32": {"max": 1e-4, "mean": None},
       "fp16": {"max": 2e-2, "mean": 2e-3},
       "bf16": {"max": 2e-2, "mean": 2e-3}}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def device_to_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def run_gpu(inp, causal=None, sm_scale=None, with_lse=True, views=None):
    """Run the HIP path on the inputs; returns (o, lse) as torch tensors."""
    import tiled_attention_04_amd as fa
    w = inp.workload
    q = to_device(inp.q, w.dtype)
    k = to_device(inp.k, w.dtype)
    v = to_device(inp.v, w.dtype)
    if views is not None:
        q, k, v = views(q, k, v)
    layout = "shd" if w.layout == "shd" else "bhsd"
    res = fa.forward(q, k, v, causal=w.causal if causal is None else causal,
                     sm_scale=w.sm_scale if sm_scale is None else sm_scale, layout=layout,
                     return_lse=with_lse)
    import torch
    torch.cuda.synchronize()
    return res


def gpu_bhsd_f64(o, layout):
    """GPU output to float64 in [B, H, S, D] order."""
    x = device_to_f64(o)
    if layout == "shd":
        x = np.transpose(x, (1, 0, 2))[None]
    return x


def compare(name, dtype, o_gpu, lse_gpu, o_ref, lse_ref):
    tol = TOL[dtype]
    assert np.all(np.isfinite(o_gpu)), f"{name}: non-finite O"
    err_o = np.abs(o_gpu - o_ref)
    msg = f"{name}: O max {err_o.max():.3e} mean {err_o.mean():.3e}"
    if lse_gpu is not None:
        assert np.all(np.isfinite(lse_gpu)), f"{name}: non-finite lse"
        err_l = np.abs(lse_gpu - lse_ref)
        msg += f" | lse max {err_l.max():.3e} mean {err_l.mean():.3e}"
    say(msg)
    assert err_o.max() <= tol["max"], msg
    if tol["mean"] is not None:
        assert err_o.mean() <= tol["mean"], msg
    if lse_gpu is not None:
        assert err_l.max() <= tol["max"], msg
        if tol["mean"] is not None:
            assert err_l.mean() <= tol["mean"], msg
    return msg


def full_parity(inp, causal=None, sm_scale=None, views=None, with_lse=True, name=None):
    """Whole-output comparison (sizes the oracle finishes in seconds)."""
    w = inp.workload
    causal = w.causal if causal is None else causal
    sm_scale = w.sm_scale if sm_scale is None else sm_scale
    name = name or w.name
    say(f"[gpu] {name}: dtype={w.dtype} layout={w.layout} B={w.batch} H={w.heads} "
        f"Sq={w.seq_q} Sk={w.seq_k} D={w.head_dim} causal={causal} scale={sm_scale}")
    res = run_gpu(inp, causal=causal, sm_scale=sm_scale, with_lse=with_lse, views=views)
    o, lse = (res if with_lse else (res, None))
    o_ref, lse_ref = oracle.forward(inp.as_bhsd_f64("q"), inp.as_bhsd_f64("k"),
                                    inp.as_bhsd_f64("v"), sm_scale, causal)
    lse_g = device_to_f64(lse) if lse is not None else None
    return compare(name, w.dtype, gpu_bhsd_f64(o, w.layout), lse_g, o_ref, lse_ref)


def sampled_rows(w, rng, n_random, extra=()):
    """Flat row ids ((b*H + h)*Sq + i) covering tile edges, the ends and random rows."""
    S = w.seq_q
    picks = set()
    bhs = [(0, 0), (w.batch - 1, w.heads - 1), (w.batch // 2, w.heads // 2)]
    for (b, h) in bhs:
        base = (b * w.heads + h) * S
        for i in [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 255, 256, S // 2, S - 129, S - 128,
                  S - 65, S - 64, S - 2, S - 1]:
            if 0 <= i < S:
                picks.add(base + i)
    for i in extra:
        picks.add(int(i))
    picks.update(rng.choice(w.batch * w.heads * S, size=n_random, replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def sampled_parity(inp, rows, name=None):
    """Full-size run on the GPU, oracle on the sampled rows only."""
    w = inp.workload
    name = name or w.name
    say(f"[gpu] {name} (sampled {rows.size} rows): B={w.batch} H={w.heads} Sq={w.seq_q} "
        f"Sk={w.seq_k} D={w.head_dim} causal={w.causal}")
    o, lse = run_gpu(inp)
    import torch
    # properties that hold at any size: finite, and O inside the per-(b,h,dim)
    # range of V (each output row is a convex combination of V rows)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), f"{name}: non-finite"
    o_flat = o.float().reshape(w.batch * w.heads, w.seq_q, w.head_dim)
    v_dev = to_device(inp.v, w.dtype).float().reshape(w.batch * w.heads, w.seq_k, w.head_dim)
    vmin, vmax = v_dev.amin(dim=1, keepdim=True), v_dev.amax(dim=1, keepdim=True)
    slack = 2e-2
    assert bool((o_flat >= vmin - slack).all()) and bool((o_flat <= vmax + slack).all()), \
        f"{name}: O leaves the convex hull of V"
    del v_dev, o_flat
    bh_needed = sorted({int(r) // w.seq_q for r in rows})
    heads = [(bh // w.heads, bh % w.heads) for bh in bh_needed]
    q64 = inp.as_bhsd_f64("q", heads)
    k64 = inp.as_bhsd_f64("k", heads)
    v64 = inp.as_bhsd_f64("v", heads)
    # re-index rows into the reduced (len(heads), 1, Sq) problem
    pos = {bh: n for n, bh in enumerate(bh_needed)}
    local = np.array([pos[int(r) // w.seq_q] * w.seq_q + int(r) % w.seq_q for r in rows])
    o_ref, lse_ref = oracle.forward_rows(q64, k64, v64, w.sm_scale, w.causal, rows=local)
    o_all = device_to_f64(o).reshape(-1, w.head_dim)
    lse_all = device_to_f64(lse).reshape(-1)
    return compare(name, w.dtype, o_all[rows], lse_all[rows], o_ref, lse_ref)


def whole_parity_chunked(inp, name=None, heads_per_chunk=2, record=None):
    """Full-size run on the GPU, then the oracle over EVERY output row, a few
    (batch, head) pairs at a time so host memory stays bounded.  Max-abs and
    mean-abs are taken over all elements of O and lse; the per-config figures
    are printed and, when `record` is a dict, stored in it."""
    import time
    w = inp.workload
    name = name or w.name
    say(f"[gpu] {name} (whole output, oracle in chunks of {heads_per_chunk} heads): B={w.batch} "
        f"H={w.heads} Sq={w.seq_q} Sk={w.seq_k} D={w.head_dim} causal={w.causal}")
    o, lse = run_gpu(inp)
    o_all = device_to_f64(o)          # [B, H, Sq, D] for the bhsd layouts used here
    lse_all = device_to_f64(lse)      # [B, H, Sq]
    del o, lse
    assert np.all(np.isfinite(o_all)) and np.all(np.isfinite(lse_all)), f"{name}: non-finite"
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    o_max = l_max = 0.0
    o_sum = l_sum = 0.0
    worst = "-"
    t0 = time.time()
    for c in range(0, len(pairs), heads_per_chunk):
        chunk = pairs[c:c + heads_per_chunk]
        q64 = inp.as_bhsd_f64("q", chunk)
        k64 = inp.as_bhsd_f64("k", chunk)
        v64 = inp.as_bhsd_f64("v", chunk)
        o_ref, lse_ref = oracle.forward(q64, k64, v64, w.sm_scale, w.causal)
        o_g = np.stack([o_all[b, h] for (b, h) in chunk])[:, None]
        l_g = np.stack([lse_all[b, h] for (b, h) in chunk])[:, None]
        eo = np.abs(o_g - o_ref)
        el = np.abs(l_g - lse_ref)
        if float(eo.max()) > o_max:
            n, _, i, d = np.unravel_index(int(np.argmax(eo)), eo.shape)
            worst = (f"(b, h) {chunk[n]} row {i} dim {d}: gpu {o_g[n, 0, i, d]:.6f} "
                     f"oracle {o_ref[n, 0, i, d]:.6f}")
        o_max, o_sum = max(o_max, float(eo.max())), o_sum + float(eo.sum())
        l_max, l_sum = max(l_max, float(el.max())), l_sum + float(el.sum())
        say(f"  {name}: heads {c}..{c + len(chunk) - 1} of {len(pairs)} checked "
            f"({time.time() - t0:.0f} s), O max so far {o_max:.3e}")
    o_mean = o_sum / o_all.size
    l_mean = l_sum / lse_all.size
    tol = TOL[w.dtype]
    msg = (f"{name} (whole output): O max {o_max:.3e} mean {o_mean:.3e} | "
           f"lse max {l_max:.3e} mean {l_mean:.3e}; largest O error at {worst}")
    say(msg)
    if record is not None:
        record.update(o_max_abs=o_max, o_mean_abs=o_mean, lse_max_abs=l_max, lse_mean_abs=l_mean,
                      rows=int(lse_all.size))
    assert o_max <= tol["max"] and l_max <= tol["max"], msg
    if tol["mean"] is not None:
        assert o_mean <= tol["mean"] and l_mean <= tol["mean"], msg
    return msg
