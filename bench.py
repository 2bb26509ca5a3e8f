"""Benchmark of the MI355X fused attention forward.

Default workload: bf16 [batch 1, heads 16, seq 32768, head_dim 128], causal,
sm_scale 1/sqrt(128), Q/K/V ~ N(0, 1) with 1% of the K rows of every head
scaled by 8 (seeded synthetic inputs).  One step is one call of fa_fwd over
that batch (the whole forward: O and the logsumexp).  Inputs are resident in
HBM before the timed region starts.

Prints one JSON line:
  value      attention TFLOP/s = 4*b*h*s_q*s_k*d (halved for causal) / time
  roofline   the kernel's achieved TFLOP/s against the MI355X dense MFMA
             peak of the input type, with HBM traffic from rocprofv3 counters
             when they were taken on the current kernel source; a workload
             whose algorithmic bytes (Q, K, V read once, O and lse written
             once) take longer at 8 TB/s than its FLOPs at that peak (the
             short-query shapes) reports GB/s against the HBM bound instead
  cpu_baseline  the CPU oracle (C, double, OpenMP) timed on a bounded sample
             of the same workload on this host

The default line also carries `parity`: the max-abs and mean-abs error of the
timed run's O and lse against the oracle on the rows the CPU baseline ran.

Other modes:
  --all-configs         one JSON line per workload C1..C5 (the five configs:
                        ms, TFLOP/s, % of peak, HBM traffic when counted on the
                        current source, and the error of that run's output
                        against the oracle over EVERY row; C5's oracle runs in
                        chunks of heads, about a minute on 16 host cores)
  --workload c1|c2|c3|c4   time another workload (not the default line); also
                        short100 / short10 (few queries against 4096 keys),
                        short10_h800 (the same with 800 heads) and
                        c5_e5m2 (the default workload in float8 e5m2, V passed
                        key-major; roofline against the dense fp8 MFMA peak)
                        and hd256 (bf16 [1,16,8192,256] causal: the kernel of
                        head_dim 129..256)
  --splits S            forward through fa_fwd_splitk with S key splits (0: the
                        library's choice)
  --copy-calib          also run a plain device copy of 1 GiB (for counter
                        calibration under rocprofv3 --pmc)
  --summarize-pmc DIR   reduce rocprofv3 --pmc output under DIR to a summary
  --write-traffic F W   profiles/traffic_<workload>.json from a FETCH_SIZE and a
                        WRITE_SIZE rocprofv3 --pmc pass (with --copy-calib)
  --pass bwd            time the backward (fa_bwd: delta, dQ and dK/dV launches)
                        on the same workload instead; FLOPs counted as 2.5x the
                        forward's (the five products of the backward), so the
                        recomputation of P in both phases is extra work
"""
import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA: 256 CU x 2.4 GHz x 8192 FLOP/clk
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 matrix (MFMA) peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E bandwidth
METRIC = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak (1 GPU)"
KERNEL_SOURCES = ["tiled_attention_04_amd/csrc/fa_fwd_kernels.hpp",
                  "tiled_attention_04_amd/csrc/fa_fwd_ks2.hpp",
                  "tiled_attention_04_amd/csrc/fa_fwd_wide.hpp",
                  "tiled_attention_04_amd/csrc/fa_mfma_asm.hpp",
                  "tiled_attention_04_amd/csrc/fa_api.hip"]
PROFILES = os.path.join(ROOT, "profiles")
# context only: the pages' unfused attention timings on an RTX 3090 (fp32,
# d_model 768, 12 heads, batch 4; sequence length not stated)
CONTEXT_RTX3090 = {"qk_matmul_ms": 0.1428, "pv_matmul_ms": 0.0759, "softmax_ms": 0.0314,
                   "source": "[CS336] Assignment 2: Systems, Nsight Systems Profile (unfused)"}


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(key="c5"):
    """HBM bytes per launch of workload `key` from the committed counter
    summary profiles/traffic_<key>.json, if it matches the current kernel
    source; otherwise None."""
    try:
        with open(os.path.join(PROFILES, f"traffic_{key}.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, target_s=15.0):
    """Time the C oracle on a bounded sample of query rows of the workload.

    A 64-row pilot sizes the sample to about target_s seconds; the rows are
    evenly spaced over the first few (batch, head) pairs, so their causal
    lengths average like the full workload's."""
    import numpy as np
    import oracle

    w = inp.workload
    S = w.seq_q

    def row_flops(rows):
        i = rows % S
        keys = np.minimum(i + 1, w.seq_k) if w.causal else np.full(rows.shape, w.seq_k)
        return float(np.sum(4.0 * keys * w.head_dim))

    ref = {}

    def run(n_heads, n_rows):
        heads = [(bh // w.heads, bh % w.heads) for bh in range(n_heads)]
        q64 = inp.as_bhsd_f64("q", heads)
        k64 = inp.as_bhsd_f64("k", heads)
        v64 = inp.as_bhsd_f64("v", heads)
        rows = np.unique(np.linspace(0, n_heads * S - 1, n_rows).astype(np.int64))
        t0 = time.perf_counter()
        ref["o"], ref["lse"] = oracle.forward_rows(q64, k64, v64, w.sm_scale, w.causal, rows=rows)
        return rows, time.perf_counter() - t0

    mean_row = 4.0 * w.head_dim * ((w.seq_k + 1) / 2 if w.causal else w.seq_k)
    max_rows = w.batch * w.heads * S
    n_rows = 256
    for _ in range(4):  # grow the sample until it takes at least two thirds of target_s
        n_heads = int(min(w.batch * w.heads, max(1, -(-n_rows // S))))
        rows, dt = run(n_heads, min(n_rows, n_heads * S))
        if dt >= (2.0 / 3.0) * target_s or rows.size >= max_rows:
            break
        rate = row_flops(rows) / max(dt, 1e-3)  # oracle FLOP/s on this host
        n_rows = int(min(max_rows, max(2 * n_rows, rate * target_s / mean_row)))
    out = {"value": row_flops(rows) / dt / 1e12, "unit": "TFLOP/s",
           "cores": oracle.max_threads(), "kind": "oracle",
           "sample": f"{rows.size} evenly spaced query rows of the first {n_heads} (batch, head) "
                     f"pairs of the same workload (fp64 C oracle, materialised softmax), "
                     f"{dt:.1f} s wall"}
    out["numpy_oracle"] = numpy_oracle_rate(inp)
    # rows are flat ids of the first n_heads (batch, head) pairs, hence of the
    # whole problem too: the caller compares the GPU output on them
    return out, rows, ref["o"], ref["lse"]


def numpy_oracle_rate(inp, max_rows=8192):
    """The NumPy float64 oracle (BLAS matmuls) on the first rows of one head:
    with a causal mask, query rows 0..n-1 see only keys 0..n-1, so the
    sample is exact with K and V cut to n keys."""
    import numpy as np
    from oracle import oracle_np
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except ImportError:
        threads = 0
    w = inp.workload
    n = min(w.seq_q, max_rows)
    nk = n if w.causal else w.seq_k
    q = inp.as_bhsd_f64("q", [(0, 0)])[:, :, :n]
    k = inp.as_bhsd_f64("k", [(0, 0)])[:, :, :nk]
    v = inp.as_bhsd_f64("v", [(0, 0)])[:, :, :nk]
    t0 = time.perf_counter()
    oracle_np.attention_forward(q, k, v, w.sm_scale, w.causal)
    dt = time.perf_counter() - t0
    i = np.arange(n)
    keys = np.minimum(i + 1, nk) if w.causal else np.full(n, nk)
    return {"value": float(np.sum(4.0 * keys * w.head_dim)) / dt / 1e12, "unit": "TFLOP/s",
            "blas_threads": threads,
            "sample": f"first {n} query rows of (batch 0, head 0), float64 NumPy oracle "
                      f"(materialised softmax in row blocks), {dt:.1f} s wall"}


def summarize_pmc(d):
    """Reduce rocprofv3 --pmc counter CSVs under d: per-kernel mean of each counter."""
    import csv
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                k = row.get("Kernel_Name", "?")
                c = row.get("Counter_Name", "?")
                v = float(row.get("Counter_Value", "nan"))
                key = (k, c)
                n, s = out.get(key, (0, 0.0))
                out[key] = (n + 1, s + v)
    res = {}
    for (k, c), (n, s) in sorted(out.items()):
        res.setdefault(k, {})[c] = {"mean": s / n, "samples": n}
    return res


def write_traffic(key, fetch_dir, write_dir, command):
    """profiles/traffic_<key>.json from two rocprofv3 --pmc passes (FETCH_SIZE,
    then WRITE_SIZE) of `bench.py --copy-calib` runs: the forward kernel's
    per-dispatch KiB, each scaled by what the same counter read for the plain
    1 GiB device copy the run makes (its bytes over the counter's bytes)."""
    fetch, write = summarize_pmc(fetch_dir), summarize_pmc(write_dir)

    def pick(res, counter, needle):
        hits = [(k, v[counter]["mean"]) for k, v in res.items() if needle in k and counter in v]
        assert len(hits) == 1, (needle, [h[0] for h in hits])
        return hits[0]
    kname, f_kib = pick(fetch, "FETCH_SIZE", "fa_fwd")
    _, w_kib = pick(write, "WRITE_SIZE", "fa_fwd")
    _, f_copy = pick(fetch, "FETCH_SIZE", "copyBuffer")
    _, w_copy = pick(write, "WRITE_SIZE", "copyBuffer")
    n = 1 << 30
    f_fac, w_fac = n / (f_copy * 1024), n / (w_copy * 1024)
    out = {"kernel": kname, "workload_key": key, "kernel_source_hash": kernel_source_hash(),
           "fetch_size_kib": f_kib, "write_size_kib": w_kib,
           "copy_calibration": {"bytes_read_and_written": n, "fetch_size_kib": f_copy,
                                "write_size_kib": w_copy, "fetch_factor": round(f_fac, 4),
                                "write_factor": round(w_fac, 4)},
           "hbm_bytes_per_launch": int(round(f_kib * 1024 * f_fac + w_kib * 1024 * w_fac)),
           "command": command}
    path = os.path.join(PROFILES, f"traffic_{key}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return path


def bench_bwd(args, w, inp, up, q, k, v, o, lse, layout, stream):
    """Time fa_bwd on the workload (inputs, O, lse and dO resident before timing)."""
    import torch
    import tiled_attention_04_amd as fa
    from tiled_attention_04_amd import synth

    fa.forward(q, k, v, causal=w.causal, sm_scale=w.sm_scale, layout=layout, out=o, lse=lse)
    do = up(synth.make_dout(w))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)

    def step():
        fa.backward(q, k, v, o, do, lse, causal=w.causal, sm_scale=w.sm_scale, layout=layout,
                    dq=dq, dk=dk, dv=dv, delta=delta)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s0, s1 in ev:
        s0.record(stream)
        step()
        s1.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms = sum(per) / len(per)
    flops = 2.5 * w.flops()
    value = flops / (ms * 1e-3) / 1e12
    print(f"[bench] bwd {args.steps} steps: avg {ms:.4f} ms, median {per[len(per) // 2]:.4f}, "
          f"min {per[0]:.4f}", file=sys.stderr, flush=True)
    out = {"metric": "attention bwd TFLOP/s (2.5x forward FLOPs) and % of MI355X bf16 MFMA peak",
           "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "pass": "bwd", "flops_per_step": flops},
           "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
           "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                        "traffic": None, "kernel_ms_avg": round(ms, 5),
                        "kernel_ms_min": round(per[0], 5)}}
    print(json.dumps(out), flush=True)
    return 0


def upload(w, a, dev):
    import numpy as np
    import torch
    if w.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    if w.dtype == "e5m2":
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e5m2).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_bhsd_f64(t, layout):
    """A device output ([B,H,S,...] or [S,H,...] for "shd") as float64 [B,H,S,...]."""
    import numpy as np
    import torch
    x = t.detach().to(torch.float64).cpu().numpy()
    if layout == "shd":
        x = np.moveaxis(x, 0, 1)[None] if x.ndim == 3 else x
    return x


def error_summary(o_gpu, lse_gpu, o_ref, lse_ref, rows, how):
    """Max-abs and mean-abs errors of O and lse (float64 arrays of equal shape)."""
    import numpy as np
    eo, el = np.abs(o_gpu - o_ref), np.abs(lse_gpu - lse_ref)
    return {"o_max_abs": float(eo.max()), "o_mean_abs": float(eo.mean()),
            "lse_max_abs": float(el.max()), "lse_mean_abs": float(el.mean()),
            "rows": int(rows), "finite": bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all()),
            "against": how}


def whole_output_errors(w, inp, o, lse, layout, heads_per_chunk):
    """Error of the GPU output over every row, the oracle run a few heads at a time."""
    import numpy as np
    import oracle
    o_all = to_bhsd_f64(o, layout)
    lse_all = lse.detach().double().cpu().numpy()
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    acc = {"o_max": 0.0, "o_sum": 0.0, "l_max": 0.0, "l_sum": 0.0}
    t0 = time.perf_counter()
    for c in range(0, len(pairs), heads_per_chunk):
        chunk = pairs[c:c + heads_per_chunk]
        o_ref, lse_ref = oracle.forward(inp.as_bhsd_f64("q", chunk), inp.as_bhsd_f64("k", chunk),
                                        inp.as_bhsd_f64("v", chunk), w.sm_scale, w.causal)
        eo = np.abs(np.stack([o_all[b, h] for (b, h) in chunk])[:, None] - o_ref)
        el = np.abs(np.stack([lse_all[b, h] for (b, h) in chunk])[:, None] - lse_ref)
        acc["o_max"], acc["o_sum"] = max(acc["o_max"], float(eo.max())), acc["o_sum"] + float(eo.sum())
        acc["l_max"], acc["l_sum"] = max(acc["l_max"], float(el.max())), acc["l_sum"] + float(el.sum())
        print(f"[bench] {w.name}: oracle over heads {c}..{c + len(chunk) - 1} of {len(pairs)} "
              f"({time.perf_counter() - t0:.0f} s)", file=sys.stderr, flush=True)
    return {"o_max_abs": acc["o_max"], "o_mean_abs": acc["o_sum"] / o_all.size,
            "lse_max_abs": acc["l_max"], "lse_mean_abs": acc["l_sum"] / lse_all.size,
            "rows": int(lse_all.size),
            "finite": bool(np.isfinite(o_all).all() and np.isfinite(lse_all).all()),
            "against": "fp64 C oracle, every row", "oracle_s": round(time.perf_counter() - t0, 1)}


def time_launches(step, stream, steps, warmup):
    """W untimed launches, then K timed ones: events around the region and
    around every launch.  Returns (ms per step over the region, sorted
    per-launch ms, wall seconds)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    region0.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    per_launch = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    return region0.elapsed_time(region1) / steps, per_launch, t_wall


def algorithmic_bytes(w):
    """HBM bytes a launch must move at least: Q, K, V read once and O written
    once in the storage type, the fp32 lse written once."""
    eb = {"fp32": 4, "fp16": 2, "bf16": 2, "e5m2": 1}[w.dtype]
    return w.batch * w.heads * ((2 * w.seq_q + 2 * w.seq_k) * w.head_dim * eb + 4 * w.seq_q)


def roofline(w, key, splits, per_launch, peak):
    """The bound of the launch (HBM bytes or MFMA FLOPs, whichever takes
    longer at the MI355X peaks) and the achieved fraction of it."""
    flops, nbytes = w.flops(), algorithmic_bytes(w)
    ms_avg = sum(per_launch) / len(per_launch)
    timing = {"kernel_ms_avg": round(ms_avg, 5),
              "kernel_ms_median": round(per_launch[len(per_launch) // 2], 5),
              "kernel_ms_min": round(per_launch[0], 5)}
    traffic = load_traffic(key) if splits == 1 else None
    if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12):
        achieved = nbytes / (ms_avg * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": nbytes, **timing}
    achieved = flops / (ms_avg * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, **timing}


def bench_line(w, key, steps, warmup, splits, ms_per_step, per_launch, peak):
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    return {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "key_splits": splits, "batch": w.batch, "heads": w.heads,
                   "seq_q": w.seq_q, "seq_k": w.seq_k, "head_dim": w.head_dim,
                   "causal": w.causal, "sm_scale": w.sm_scale, "flops_per_step": flops},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": roofline(w, key, splits, per_launch, peak),
        "context": {"rtx3090_unfused_per_call": CONTEXT_RTX3090},
    }


class Setup:
    """Seeded inputs of one workload, resident on the device, and its step."""

    def __init__(self, key, dev, splits=1):
        import torch
        import tiled_attention_04_amd as fa
        from tiled_attention_04_amd import synth
        w = synth.WORKLOADS.get(key) or synth.EXTRA_WORKLOADS[key]
        print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
        self.key, self.w, self.inp = key, w, synth.make_inputs(w)
        q, k = upload(w, self.inp.q, dev), upload(w, self.inp.k, dev)
        if w.dtype == "e5m2":
            import numpy as np
            # the fp8 path takes V key-major: [B, H, D, Sk] (Sk is a multiple of 16 here)
            v = upload(w, np.transpose(self.inp.v, (0, 1, 3, 2)), dev)
        else:
            v = upload(w, self.inp.v, dev)
        self.q, self.k, self.v = q, k, v
        self.peak = {"e5m2": PEAK_FP8_TFLOPS, "fp32": PEAK_FP32_TFLOPS}.get(w.dtype, PEAK_BF16_TFLOPS)
        self.layout = layout = "shd" if w.layout == "shd" else "bhsd"
        self.o = o = torch.empty_like(q)
        self.lse = lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.splits = 1
        if splits != 1:
            self.splits = splits or fa.fa_fwd_splitk_choose(w.batch, w.heads, w.seq_q, w.seq_k,
                                                            w.head_dim, w.causal)
            ws = torch.empty(max(1, fa.fa_fwd_splitk_workspace(w.batch, w.heads, w.seq_q,
                                                               w.head_dim, self.splits)),
                             dtype=torch.uint8, device=dev)
            n = self.splits

            def step():
                fa.forward_splitk(q, k, v, causal=w.causal, sm_scale=w.sm_scale, layout=layout,
                                  num_splits=n, out=o, lse=lse, workspace=ws)
        else:
            def step():
                fa.forward(q, k, v, causal=w.causal, sm_scale=w.sm_scale, layout=layout, out=o,
                           lse=lse)
        self.step = step


def all_configs(args, dev):
    """One line per workload C1..C5, each with the whole-output error of its run."""
    import torch
    for key in ("c1", "c2", "c3", "c4", "c5"):
        st = Setup(key, dev)
        ms, per, _ = time_launches(st.step, st.stream, args.steps, args.warmup)
        out = bench_line(st.w, key, args.steps, args.warmup, 1, ms, per, st.peak)
        print(f"[bench] {key}: {ms:.4f} ms/step, kernel min {per[0]:.4f} ms",
              file=sys.stderr, flush=True)
        # the output of the last timed launch, against the oracle over every row
        out["parity"] = whole_output_errors(st.w, st.inp, st.o, st.lse, st.layout,
                                            heads_per_chunk=2 if key == "c5" else 16)
        print(json.dumps(out), flush=True)
        del st
        torch.cuda.empty_cache()
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5",
                    choices=["c1", "c2", "c3", "c4", "c5", "short100", "short10", "short10_h800",
                             "c5_e5m2", "hd256"])
    ap.add_argument("--all-configs", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--summarize-pmc", default=None)
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "output directories (FETCH_SIZE pass, WRITE_SIZE pass)")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"])
    ap.add_argument("--splits", type=int, default=1,
                    help="forward through fa_fwd_splitk with this many key splits "
                         "(0: the library's choice; 1: plain fa_fwd)")
    args = ap.parse_args()

    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc), indent=1))
        return 0
    if args.write_traffic:
        cmd = (f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- "
               f"python -u bench.py --workload {args.workload} --no-cpu-baseline --steps 3 "
               f"--warmup 1 --copy-calib")
        print(write_traffic(args.workload, *args.write_traffic, cmd))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (heads would shard across GPUs with no exchange)",
              file=sys.stderr)
        return 2

    import torch

    import tiled_attention_04_amd as fa

    fa.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all_configs:
        return all_configs(args, dev)

    st = Setup(args.workload, dev, splits=args.splits if args.which == "fwd" else 1)
    w = st.w
    if args.which == "bwd":
        return bench_bwd(args, w, st.inp, lambda a: upload(w, a, dev), st.q, st.k, st.v, st.o,
                         st.lse, st.layout, st.stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    ms_per_step, per_launch, t_wall = time_launches(st.step, st.stream, args.steps, args.warmup)
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (events), wall {t_wall:.3f} s, "
          f"kernel avg {sum(per_launch) / len(per_launch):.4f} ms, "
          f"median {per_launch[len(per_launch)//2]:.4f}, min {per_launch[0]:.4f}",
          file=sys.stderr, flush=True)

    if args.copy_calib:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 copies of {n} bytes", file=sys.stderr, flush=True)
        del src, dst

    out = bench_line(w, args.workload, args.steps, args.warmup, st.splits, ms_per_step,
                     per_launch, st.peak)
    if not args.no_cpu_baseline and args.workload == "c5":
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        base, rows, o_ref, lse_ref = cpu_baseline(st.inp)
        out["cpu_baseline"] = base
        # the timed run's output on the same rows (flat ids over [B*H*Sq])
        o_g = to_bhsd_f64(st.o, st.layout).reshape(-1, w.head_dim)[rows]
        l_g = st.lse.detach().double().cpu().numpy().reshape(-1)[rows]
        out["parity"] = error_summary(o_g, l_g, o_ref, lse_ref, rows.size,
                                      "fp64 C oracle on the cpu_baseline sample rows")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
