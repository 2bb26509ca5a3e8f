"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, so both the GPU path's tests and
the CPU oracle can take their inputs from it without sharing any method code.

Recipe (a reading: the pages only say the inputs are random normals with a
given standard deviation -- "Understanding Triton Tutorials Part 2", section
"Fused Attention 2", and the test of "BUG in flash attention kernel"):
  * one NumPy PCG64 generator per workload, seeded with ``seed``;
  * Q, K, V drawn in that order as float64 standard normals, in the C order of
    the workload's logical shape, times ``std``;
  * each value rounded once, round-to-nearest-even, to the storage dtype;
  * large-logit stress (long-sequence workload only): afterwards, for every
    (batch, head) in order, ``round(frac * seq_k)`` distinct key rows are drawn
    without replacement and those K rows are multiplied by ``factor`` (a power
    of two, so the scaling is exact).
Storage: fp32 -> np.float32, fp16 -> np.float16, bf16 -> np.uint16 holding the
bf16 bit pattern, e5m2 -> np.uint8 holding the float8 e5m2 bit pattern (OCP:
sign, 5 exponent bits with bias 15, 2 mantissa bits -- the upper byte of an
IEEE binary16; NumPy has neither type).
"""
from dataclasses import dataclass, field
import math

import numpy as np

DTYPES = ("fp32", "fp16", "bf16", "e5m2")
LAYOUTS = ("shd", "bhsd")  # [seq, heads, d] (batch 1) or [batch, heads, seq, d]


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    layout: str
    batch: int
    heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    std: float
    sm_scale: float
    causal: bool
    seed: int
    stress_frac: float = 0.0
    stress_factor: float = 1.0

    def flops(self):
        """Attention FLOPs by the convention 4*b*h*s_q*s_k*d, halved when causal."""
        f = 4.0 * self.batch * self.heads * self.seq_q * self.seq_k * self.head_dim
        return f / 2 if self.causal else f

    def shape(self, which):
        s = self.seq_q if which == "q" else self.seq_k
        if self.layout == "shd":
            assert self.batch == 1
            return (s, self.heads, self.head_dim)
        return (self.batch, self.heads, s, self.head_dim)

    def strides(self, which):
        """Element strides in the order (batch, head, seq, dim)."""
        s = self.seq_q if which in ("q", "o") else self.seq_k
        H, D = self.heads, self.head_dim
        if self.layout == "shd":
            return (s * H * D, D, H * D, 1)
        return (H * s * D, s * D, D, 1)


WORKLOADS = {
    "c1": Workload("fp32 [128,1,64] seq-heads-d, non-causal", "fp32", "shd", 1, 1, 128, 128, 64,
                   0.5, 1.0 / 8.0, False, seed=21),
    "c2": Workload("fp16 s_q=1000 s_k=1537 h=16 d=64 seq-heads-d, non-causal", "fp16", "shd", 1, 16,
                   1000, 1537, 64, 0.5, 0.5, False, seed=22),
    "c3": Workload("bf16 [4,12,2048,64] causal", "bf16", "bhsd", 4, 12, 2048, 2048, 64,
                   1.0, 1.0 / 8.0, True, seed=23),
    "c4": Workload("bf16 [4,32,4096,80] causal", "bf16", "bhsd", 4, 32, 4096, 4096, 80,
                   1.0, 1.0 / math.sqrt(80.0), True, seed=24),
    "c5": Workload("bf16 [1,16,32768,128] causal, 1% of K rows x8", "bf16", "bhsd", 1, 16, 32768,
                   32768, 128, 1.0, 1.0 / math.sqrt(128.0), True, seed=25,
                   stress_frac=0.01, stress_factor=8.0),
}

# Short-query / cross-attention shapes of the form the triton issue's test
# matrix uses (few query rows against 4096 keys, [seq, heads, d], fp16):
# timing cases for the key-split forward, not target configurations.
EXTRA_WORKLOADS = {
    "short100": Workload("fp16 s_q=100 s_k=4096 h=12 d=64 seq-heads-d, non-causal", "fp16",
                         "shd", 1, 12, 100, 4096, 64, 1.0, 0.5, False, seed=41),
    "short10": Workload("fp16 s_q=10 s_k=4096 h=12 d=64 seq-heads-d, non-causal", "fp16",
                        "shd", 1, 12, 10, 4096, 64, 1.0, 0.5, False, seed=42),
    # the issue's largest head count: each head's 4096 keys read for 10 queries
    "short10_h800": Workload("fp16 s_q=10 s_k=4096 h=800 d=64 seq-heads-d, non-causal", "fp16",
                             "shd", 1, 800, 10, 4096, 64, 1.0, 0.5, False, seed=43),
    # the long causal workload with every input stored in float8 e5m2 (the
    # fp8 variant of the tutorial's kernel): same draws, rounded to e5m2
    "c5_e5m2": Workload("e5m2 [1,16,32768,128] causal, 1% of K rows x8", "e5m2", "bhsd", 1, 16,
                        32768, 32768, 128, 1.0, 1.0 / math.sqrt(128.0), True, seed=25,
                        stress_frac=0.01, stress_factor=8.0),
    # the widest head_dim of the forward (its one-pass kernel), long causal
    # rows with the same key stress as the 32768-token workload
    "hd256": Workload("bf16 [1,16,8192,256] causal, 1% of K rows x8", "bf16", "bhsd", 1, 16,
                      8192, 8192, 256, 1.0, 1.0 / 16.0, True, seed=26,
                      stress_frac=0.01, stress_factor=8.0),
}

_CHUNK = 1 << 22


def round_to_dtype(x, dtype):
    """Round float64 values once (RNE) to the storage representation of dtype."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp32":
        return x.astype(np.float32)
    if dtype == "fp16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return _f64_to_bf16_bits(x)
    if dtype == "e5m2":
        return _f64_to_e5m2_bits(x)
    raise ValueError(dtype)


E5M2_MAX = 57344.0  # 1.75 * 2^15


def _f64_to_e5m2_bits(x):
    """RNE to the e5m2 grid: 3 significant bits for |x| >= 2^-14, a fixed
    quantum of 2^-16 below (subnormals); the rounded value is exact in
    binary16, whose upper byte is the e5m2 code."""
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no e5m2 code here")
    a = np.abs(x)
    _, ex = np.frexp(a)  # a = m 2^ex, 0.5 <= m < 1
    quantum = np.where(a >= 2.0 ** -14, np.ldexp(1.0, ex - 3), 2.0 ** -16)
    r = np.rint(a / quantum) * quantum  # np.rint: ties to even
    if np.any(r > E5M2_MAX):
        raise ValueError("value outside the e5m2 range")
    h = np.copysign(r, x).astype(np.float16)  # exact
    return (np.ascontiguousarray(h).view(np.uint16) >> np.uint16(8)).astype(np.uint8)


def _f64_to_bf16_bits(x):
    a = np.abs(x)
    if np.any((a > 0) & (a < 2.0 ** -126)) or np.any(a > 3.0e38) or np.any(np.isnan(x)):
        raise ValueError("value outside the bf16 normal range")
    bits = np.ascontiguousarray(x).view(np.uint64)
    drop = np.uint64(45)  # 52 float64 mantissa bits -> 7 bf16 mantissa bits
    lsb = (bits >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    kept = (bits + half + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = kept.view(np.float64).astype(np.float32)  # exact: value is bf16-representable
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def widen(stored, dtype):
    """Exact float64 values of a stored array."""
    if dtype == "bf16":
        u = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "e5m2":
        u = np.asarray(stored, dtype=np.uint8).astype(np.uint16) << np.uint16(8)
        return u.view(np.float16).astype(np.float64)
    return np.asarray(stored).astype(np.float64)


def _draw(rng, shape, std, dtype):
    n = int(np.prod(shape))
    out_dtype = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16,
                 "e5m2": np.uint8}[dtype]
    out = np.empty(n, dtype=out_dtype)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = round_to_dtype(rng.standard_normal(e - s) * std, dtype)
    return out.reshape(shape)


def device_normal(shape, dtype, seed, std=1.0, device="cuda"):
    """Seeded N(0, std^2) values drawn on the device by torch's generator and
    rounded to ``dtype`` (torch's own round-to-nearest-even conversion), for
    inputs too large to draw on the host.  Both sides of a comparison read the
    same tensor: the GPU path directly, the oracle through host copies of the
    slices it checks."""
    import torch
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16,
           "e5m2": torch.float8_e5m2}[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=tdt, device=device)
    flat = out.view(-1)
    step = 1 << 28  # draw in fp32 chunks of 1 GiB
    for s in range(0, flat.numel(), step):
        e = min(flat.numel(), s + step)
        flat[s:e] = (torch.randn(e - s, generator=gen, device=device) * std).to(tdt)
    return out


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    stressed_rows: dict = field(default_factory=dict)  # (b, h) -> key indices scaled

    def as_bhsd_f64(self, which, heads=None):
        """float64 copy in [B, H, S, D] order (optionally only some (b, h) pairs)."""
        arr = {"q": self.q, "k": self.k, "v": self.v}[which]
        if self.workload.layout == "shd":
            arr = np.transpose(arr, (1, 0, 2))[None]
        if heads is not None:
            arr = np.stack([arr[b, h] for (b, h) in heads])[:, None]
        return widen(arr, self.workload.dtype)


def make_inputs(w, seq_q=None, seq_k=None):
    """Draw the inputs of workload ``w`` (a Workload or a key of WORKLOADS)."""
    if isinstance(w, str):
        w = WORKLOADS[w] if w in WORKLOADS else EXTRA_WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    q = _draw(rng, w.shape("q"), w.std, w.dtype)
    k = _draw(rng, w.shape("k"), w.std, w.dtype)
    v = _draw(rng, w.shape("v"), w.std, w.dtype)
    stressed = {}
    if w.stress_frac > 0:
        n_rows = int(round(w.stress_frac * w.seq_k))
        for b in range(w.batch):
            for h in range(w.heads):
                idx = np.sort(rng.choice(w.seq_k, size=n_rows, replace=False))
                stressed[(b, h)] = idx
                if w.layout == "shd":
                    rows = k[idx, h, :]
                else:
                    rows = k[b, h, idx, :]
                scaled = round_to_dtype(widen(rows, w.dtype) * w.stress_factor, w.dtype)
                if w.layout == "shd":
                    k[idx, h, :] = scaled
                else:
                    k[b, h, idx, :] = scaled
    return Inputs(w, q, k, v, stressed)


def make_integer_score_inputs(w, nonzeros=4):
    """Inputs whose scores Q K^T are small integers: every Q row holds
    ``nonzeros`` entries +-1 at distinct random dims (zeros elsewhere) and K
    holds integers in [-2, 2]; V is drawn as in ``make_inputs``.  A row's
    scores then span at most 4 * nonzeros, so with a scale of +-ln 2 every
    softmax weight relative to the row maximum is an exact power of two no
    smaller than 2^-16 (exact in every storage type here, e5m2 included)."""
    rng = np.random.default_rng(w.seed)
    qshape, kshape = w.shape("q"), w.shape("k")
    rows = int(np.prod(qshape[:-1]))
    q = np.zeros((rows, w.head_dim))
    cols = np.argsort(rng.random((rows, w.head_dim)), axis=1)[:, :nonzeros]
    signs = rng.choice([-1.0, 1.0], size=(rows, nonzeros))
    np.put_along_axis(q, cols, signs, axis=1)
    k = rng.integers(-2, 3, size=kshape).astype(np.float64)
    v = _draw(rng, w.shape("v"), w.std, w.dtype)
    return Inputs(w, round_to_dtype(q.reshape(qshape), w.dtype), round_to_dtype(k, w.dtype), v, {})


def make_dout(w):
    """The upstream gradient dO of workload ``w`` for the backward: N(0, 1)
    draws in the shape (and layout) of q, rounded once to the dtype, from its
    own stream (seed + 7919) so the forward inputs are unchanged."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed + 7919)
    return _draw(rng, w.shape("q"), 1.0, w.dtype)


def dout_bhsd_f64(w, dout):
    """dO as float64 in [B, H, S, D] order."""
    arr = np.transpose(dout, (1, 0, 2))[None] if w.layout == "shd" else dout
    return widen(arr, w.dtype)


def custom(name, dtype, layout, batch, heads, seq_q, seq_k, head_dim, std=1.0, sm_scale=None,
           causal=False, seed=0, stress_frac=0.0, stress_factor=1.0):
    """A Workload for edge-case tests (same recipe, other sizes)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return Workload(name, dtype, layout, batch, heads, seq_q, seq_k, head_dim, std, sm_scale,
                    causal, seed, stress_frac, stress_factor)
