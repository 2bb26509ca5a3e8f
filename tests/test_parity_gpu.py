"""Parity of the HIP attention forward with the CPU oracle (MI355X only).

Every case calls the library through its C ABI binding and compares O and
the logsumexp with the oracle at the stated tolerances: max-abs 1e-4 for
fp32; max-abs 2e-2 and mean-abs 2e-3 for fp16/bf16.
"""
import math

import numpy as np
import pytest

from tiled_attention_04_amd import synth
from gpu_cases import (full_parity, sampled_parity, sampled_rows, say, run_gpu, to_device,
                       whole_parity_chunked)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_attention_04_amd as fa
    fa.lib()  # fail loudly if the HIP library is missing


# ---- the five workloads ------------------------------------------------------

@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_workload_full(key):
    full_parity(synth.make_inputs(key), name=key)


def test_workload_c4_whole_output():
    """Every row of C4 (bf16 [4,32,4096,80] causal) against the oracle."""
    whole_parity_chunked(synth.make_inputs("c4"), name="c4", heads_per_chunk=16)


def test_workload_c5_whole_output():
    """Every row of C5 (bf16 [1,16,32768,128] causal, 1% of K rows x8)."""
    whole_parity_chunked(synth.make_inputs("c5"), name="c5", heads_per_chunk=2)


def test_workload_c4_sampled():
    inp = synth.make_inputs("c4")
    rows = sampled_rows(inp.workload, np.random.default_rng(4), 1500)
    sampled_parity(inp, rows, name="c4")


def test_workload_c5_sampled():
    inp = synth.make_inputs("c5")
    w = inp.workload
    # rows that see a stressed (x8) key on or after it, for head (0, 0) and (0, 15)
    extra = []
    for (b, h) in [(0, 0), (0, 15)]:
        idx = inp.stressed_rows[(b, h)]
        base = (b * w.heads + h) * w.seq_q
        extra += [base + int(j) for j in idx[:40]] + [base + int(j) + 1 for j in idx[:20]]
    rows = sampled_rows(w, np.random.default_rng(5), 400, extra=extra)
    sampled_parity(inp, rows, name="c5")


# ---- edges -------------------------------------------------------------------

EDGE_SEQ = [(1, 1), (1, 64), (10, 63), (100, 65), (129, 127), (64, 129), (77, 300), (300, 77)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,sk", EDGE_SEQ)
def test_ragged_sequences(dtype, causal, sq, sk):
    w = synth.custom("ragged", dtype, "bhsd", 2, 3, sq, sk, 64, causal=causal,
                     seed=100 + sq * 7 + sk)
    full_parity(synth.make_inputs(w), name=f"ragged {dtype} sq={sq} sk={sk} causal={causal}")


@pytest.mark.parametrize("d", [8, 16, 24, 32, 40, 64, 72, 80, 96, 112, 128, 136, 160, 192, 200, 256])
def test_head_dims_bf16(d):
    w = synth.custom("hd", "bf16", "bhsd", 1, 2, 150, 190, d, causal=(d % 16 == 0), seed=200 + d)
    full_parity(synth.make_inputs(w), name=f"head_dim bf16 d={d}")


@pytest.mark.parametrize("d", [8, 64, 80, 128, 248])
def test_head_dims_fp16(d):
    w = synth.custom("hd", "fp16", "bhsd", 1, 2, 150, 190, d, causal=True, seed=300 + d)
    full_parity(synth.make_inputs(w), name=f"head_dim fp16 d={d}")


@pytest.mark.parametrize("d", [4, 12, 32, 60, 64, 100, 128, 256])
def test_head_dims_fp32(d):
    w = synth.custom("hd", "fp32", "bhsd", 1, 2, 150, 190, d, causal=(d % 8 == 0), seed=400 + d)
    full_parity(synth.make_inputs(w), name=f"head_dim fp32 d={d}")


def test_seq_heads_dim_layout_cross_attention():
    """[seq, heads, d] with seq_q != seq_k (the layout family of the issue)."""
    w = synth.custom("shd", "fp16", "shd", 1, 8, 100, 700, 32, std=0.5, sm_scale=0.5, seed=500)
    full_parity(synth.make_inputs(w), name="shd fp16 q_ctx=100")


def test_heads_seq_dim_layout_distinct_head_strides():
    """(heads, seq, d) with q_ctx != seqlen: Q/O and K/V head strides differ, the
    case the "BUG in flash attention kernel" issue got wrong."""
    import torch
    w = synth.custom("hsd", "fp16", "bhsd", 1, 8, 4095, 4096, 32, std=0.5, sm_scale=0.5, seed=501)
    full_parity(synth.make_inputs(w), name="hsd fp16 q_ctx=4095 vs 4096")
    w2 = synth.custom("hsd", "fp16", "bhsd", 1, 16, 10, 4096, 32, std=0.5, sm_scale=0.5, seed=502)
    full_parity(synth.make_inputs(w2), name="hsd fp16 q_ctx=10")


def test_issue_matrix_800_heads():
    """q_ctx = 10 against 4096 keys with 800 heads, d = 32, [seq, heads, d]: the
    largest head count of the issue's test matrix (a grid of 800 one-wave-deep
    query tiles)."""
    w = synth.custom("issue h800", "fp16", "shd", 1, 800, 10, 4096, 32, std=0.5, sm_scale=0.5,
                     seed=510)
    full_parity(synth.make_inputs(w), name="shd fp16 q_ctx=10 heads=800")


def test_strided_views():
    """Inputs that are views with padded rows and a permuted layout."""
    import torch

    def views(q, k, v):
        # embed each tensor in a wider buffer (row stride 72 instead of 64)
        def widen(t):
            buf = torch.zeros(t.shape[:-1] + (t.shape[-1] + 8,), dtype=t.dtype, device=t.device)
            buf[..., : t.shape[-1]] = t
            return buf[..., : t.shape[-1]]
        return widen(q), widen(k), widen(v)

    w = synth.custom("views", "bf16", "bhsd", 2, 2, 130, 200, 64, causal=True, seed=503)
    full_parity(synth.make_inputs(w), views=views, name="strided views bf16")


def test_lse_null_path():
    w = synth.custom("nolse", "bf16", "bhsd", 1, 2, 70, 90, 64, seed=504)
    full_parity(synth.make_inputs(w), with_lse=False, name="lse=NULL")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
def test_scale_values(scale):
    w = synth.custom("scale", "bf16", "bhsd", 1, 2, 100, 150, 64, causal=True, seed=505)
    full_parity(synth.make_inputs(w), sm_scale=scale, name=f"sm_scale={scale}")


def test_large_logit_stress_small():
    w = synth.custom("stress", "bf16", "bhsd", 1, 4, 512, 512, 128, causal=True, seed=506,
                     stress_frac=0.02, stress_factor=8.0)
    full_parity(synth.make_inputs(w), name="stress x8 small")
    w2 = synth.custom("stress", "fp16", "bhsd", 1, 4, 300, 300, 64, std=1.0, sm_scale=0.25,
                      causal=False, seed=507, stress_frac=0.05, stress_factor=32.0)
    full_parity(synth.make_inputs(w2), name="stress x32 fp16")


def test_many_heads_xcd_mapping():
    """n_bh % 8 == 0 takes the XCD-grouped workgroup mapping; 7 heads does not."""
    for heads in (8, 7):
        w = synth.custom("xcd", "bf16", "bhsd", 2, heads, 300, 300, 64, causal=True,
                         seed=508 + heads)
        full_parity(synth.make_inputs(w), name=f"heads={heads} batch=2")


def test_empty_problems_are_noops():
    import torch
    import tiled_attention_04_amd as fa
    for shape_q in [(0, 2, 8, 64), (1, 0, 8, 64), (1, 2, 0, 64)]:
        q = torch.zeros(shape_q, dtype=torch.bfloat16, device="cuda")
        kv = torch.zeros((shape_q[0], shape_q[1], 8, 64), dtype=torch.bfloat16, device="cuda")
        o = torch.full_like(q, 3.0)
        fa.forward(q, kv, kv, out=o)
        torch.cuda.synchronize()
        assert bool((o == 3.0).all())


def test_repeat_is_bitwise_deterministic():
    import torch
    w = synth.custom("det", "bf16", "bhsd", 1, 8, 1000, 1000, 128, causal=True, seed=509)
    inp = synth.make_inputs(w)
    o1, l1 = run_gpu(inp)
    o2, l2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- large grids: 8-wave workgroups (at head_dim 64 and 128 with four LDS
# stages and loads two tiles ahead, a loop unrolled by four key tiles) ----

LARGE_GRID = [
    # (dtype, heads, seq_q, seq_k, head_dim, causal)
    ("bf16", 1024, 200, 333, 128, False),   # one query tile per head, ragged keys
    ("bf16", 1024, 100, 100, 128, False),   # two key tiles
    ("bf16", 1024, 256, 500, 128, False),   # eight key tiles: two whole unrolled rounds
    ("bf16", 1024, 200, 333, 64, True),     # head_dim 64
    ("fp16", 1024, 250, 777, 48, False),    # head_dim 48 in the 64 slots, 13 key tiles
    ("bf16", 1024, 200, 333, 128, True),
    ("bf16", 512, 300, 129, 128, False),    # a ragged second query tile, 3 key tiles
    ("bf16", 512, 300, 300, 128, True),
    ("bf16", 256, 700, 1000, 120, True),    # head_dim padding inside the 128 slots
    ("bf16", 1024, 64, 64, 104, False),     # one key tile
    ("bf16", 1024, 17, 1, 112, False),      # a single key
    ("fp16", 512, 300, 517, 128, True),
    ("fp16", 256, 1000, 200, 128, False),
]


@pytest.mark.parametrize("dtype,heads,sq,sk,d,causal", LARGE_GRID)
def test_large_grid_head_dim_128(dtype, heads, sq, sk, d, causal):
    w = synth.custom("large grid", dtype, "bhsd", 1, heads, sq, sk, d, causal=causal,
                     seed=600 + sq + sk + d)
    full_parity(synth.make_inputs(w), name=f"large grid {dtype} h={heads} sq={sq} sk={sk} d={d} "
                                           f"causal={causal}")


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_large_grid_scales(scale):
    w = synth.custom("large grid scale", "bf16", "bhsd", 2, 512, 256, 400, 128, causal=True,
                     seed=650)
    full_parity(synth.make_inputs(w), sm_scale=scale, name=f"large grid sm_scale={scale}")


# ---- 4-wave workgroups whose last query tile leaves waves without rows (they
# load their share of the tiles and skip the compute) ----

ROWLESS_WAVES = [
    # (dtype, heads, seq_q, seq_k, head_dim, causal)
    ("bf16", 300, 200, 333, 80, True),     # tile 1: wave 2 has 8 rows, wave 3 none
    ("fp16", 400, 40, 500, 64, False),     # waves 2 and 3 without rows in every workgroup
    ("bf16", 280, 100, 64, 96, True),      # one key tile, wave 3 without rows
    ("fp16", 300, 33, 700, 32, True),      # causal, 33 queries: one row in wave 1
]


@pytest.mark.parametrize("dtype,heads,sq,sk,d,causal", ROWLESS_WAVES)
def test_rowless_waves(dtype, heads, sq, sk, d, causal):
    w = synth.custom("rowless waves", dtype, "bhsd", 1, heads, sq, sk, d, causal=causal,
                     std=0.5 if dtype == "fp16" else 1.0, seed=690 + sq + sk + d)
    full_parity(synth.make_inputs(w), name=f"rowless waves {dtype} h={heads} sq={sq} sk={sk} "
                                           f"d={d} causal={causal}")


# ---- small grids (at most 256 query tiles of 128 rows): the key tiles of a
# query tile split between two wave groups of one workgroup, merged at the end ----

KEY_GROUPS = [
    # (dtype, heads, seq_q, seq_k, head_dim, causal)
    ("bf16", 2, 100, 65, 128, False),     # two key tiles, the second with one key
    ("bf16", 2, 300, 200, 64, True),      # causal, fewer keys than queries: 2, 4, 4 tiles
    ("fp16", 3, 129, 1000, 80, True),     # row-sum column; 2 and 3 tiles (group 1 idles)
    ("bf16", 4, 257, 777, 96, False),     # 13 tiles, the last ragged
    ("fp16", 2, 64, 4096, 32, False),     # 64 tiles
    ("bf16", 3, 200, 130, 48, True),      # head_dim 48 in the 64 slots, 3 tiles
]


@pytest.mark.parametrize("dtype,heads,sq,sk,d,causal", KEY_GROUPS)
def test_key_groups_in_workgroup(dtype, heads, sq, sk, d, causal):
    w = synth.custom("key groups", dtype, "bhsd", 1, heads, sq, sk, d, causal=causal,
                     seed=680 + sq + sk + d)
    full_parity(synth.make_inputs(w), name=f"key groups {dtype} h={heads} sq={sq} sk={sk} d={d} "
                                           f"causal={causal}")


def test_key_groups_stress_rescales():
    """Keys scaled x32: the two groups' running maxima drift apart before the merge."""
    w = synth.custom("key groups stress", "bf16", "bhsd", 1, 4, 256, 2048, 128, causal=False,
                     seed=690, stress_frac=0.03, stress_factor=32.0)
    full_parity(synth.make_inputs(w), name="key groups stress x32")


# ---- head_dim 193..256: the widest paddings, several key and query tiles ----

HEAD_DIM_256 = [
    # (dtype, heads, seq_q, seq_k, head_dim, causal)
    ("bf16", 4, 300, 333, 256, True),
    ("bf16", 4, 300, 333, 256, False),
    ("fp16", 2, 129, 700, 248, True),      # head_dim padding inside the last block
    ("bf16", 2, 1000, 64, 200, False),     # one key tile
    ("bf16", 2, 1, 1, 256, False),         # a single query and key
    ("fp16", 3, 700, 129, 256, True),      # causal with fewer keys than queries
    ("bf16", 1, 513, 1025, 224, True),
]


@pytest.mark.parametrize("dtype,heads,sq,sk,d,causal", HEAD_DIM_256)
def test_head_dim_256_tiles(dtype, heads, sq, sk, d, causal):
    w = synth.custom("head_dim 256", dtype, "bhsd", 1, heads, sq, sk, d, causal=causal,
                     seed=700 + sq + sk + d)
    full_parity(synth.make_inputs(w), name=f"head_dim {d} {dtype} h={heads} sq={sq} sk={sk} "
                                           f"causal={causal}")


def test_head_dim_256_stress_rescales():
    """head_dim 256 with keys scaled x32: many rescales of the 256-wide accumulator."""
    w = synth.custom("head_dim 256 stress", "bf16", "bhsd", 1, 8, 1024, 1024, 256, causal=True,
                     seed=760, stress_frac=0.03, stress_factor=32.0)
    full_parity(synth.make_inputs(w), name="head_dim 256 stress x32")


def test_large_grid_stress_rescales():
    """Keys scaled x32 in a long causal row: the running maximum is raised
    (and the accumulators rescaled) many times per row."""
    w = synth.custom("large grid stress", "bf16", "bhsd", 1, 128, 2048, 2048, 128, causal=True,
                     seed=651, stress_frac=0.03, stress_factor=32.0)
    full_parity(synth.make_inputs(w), name="large grid stress x32")
