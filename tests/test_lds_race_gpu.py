"""LDS race check: the parity cases run through a debug build of the
library (tests/libfa_lds_poison.so, built with FA_LDS_POISON) in which every
kernel fills each double-buffer stage with NaN as soon as the barrier that
ends its last read has passed, just before the stage's next tile is loaded.
Stage use, per kernel:
  forward (16-bit): step t reads K(t + 1) (stage (t + 1) & 1) and V(t)
    (stage t & 1); after the barrier that closes step t - 1, K(t) and
    V(t - 1) are free and receive K(t + 2) and V(t + 1);
  forward, head_dim > 128: step t reads V(t) and K(t + 2) and, with three V
    stages, V(t + 1); after the barrier that opens it, K(t + 1) and V(t - 1)
    are free and receive K(t + 3) and V(t + 2) (three V stages) or V(t + 1);
  dQ: step t reads K/V tile t from one stage while tile t + 1 loads into the
    other, freed by the barrier that closed step t - 1;
  dK/dV: the same with Q/dO tiles (and their L, D values).
A read outside its window (a missing or misplaced barrier or wait) would see
NaN or the next tile's data: the outputs must still match the oracle at the
usual bounds, with no NaN.  The production library does not carry this code.
"""
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

from tiled_attention_04_amd import synth  # noqa: E402
from gpu_cases import full_parity  # noqa: E402
import test_parity_bwd_gpu as bwd  # noqa: E402
import test_parity_splitk_gpu as splitk  # noqa: E402

pytestmark = pytest.mark.gpu
POISON_LIB = os.path.join(HERE, "libfa_lds_poison.so")


@pytest.fixture(autouse=True)
def poisoned_library():
    """Route the binding to the race-check build for the duration of a test."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_attention_04_amd as fa
    if not os.path.exists(POISON_LIB):
        raise ImportError(f"{POISON_LIB} is missing: run __graft_entry__.build()")
    saved_path, saved_lib = fa.LIB_PATH, fa._lib
    fa.LIB_PATH, fa._lib = POISON_LIB, None
    try:
        fa.lib()
        yield
    finally:
        fa.LIB_PATH, fa._lib = saved_path, saved_lib


FWD = [
    ("bf16", "bhsd", 2, 3, 300, 333, 64, True),      # 4-wave workgroups, ragged tails
    ("fp16", "bhsd", 1, 4, 700, 1100, 128, False),   # many key tiles
    ("bf16", "bhsd", 4, 64, 512, 512, 128, True),    # 4-wave workgroups, 8 key tiles
    # 8-wave workgroups (>= 1024 of them): four stages, loads two tiles ahead
    ("bf16", "bhsd", 4, 128, 512, 600, 128, True),   # 4 and 8 key tiles
    ("fp16", "bhsd", 2, 512, 256, 900, 64, False),   # 15 key tiles, head_dim 64
    # 8-wave workgroups, two stages (head_dim 80: the row-sum column)
    ("bf16", "bhsd", 1, 1024, 200, 333, 80, True),
    ("bf16", "bhsd", 1, 2, 150, 190, 80, True),      # head_dim 80 (padded V blocks)
    ("bf16", "bhsd", 1, 2, 150, 190, 256, True),     # head_dim 256 (wide kernel, two V stages)
    ("fp16", "bhsd", 1, 2, 300, 700, 192, False),    # head_dim 192 (wide kernel, three V stages)
    ("bf16", "bhsd", 1, 3, 400, 900, 160, True),     # head_dim 160 (wide kernel, three V stages)
    ("fp16", "shd", 1, 800, 10, 4096, 32, False),    # the issue's 800-head case
]


@pytest.mark.parametrize("dtype,layout,b,h,sq,sk,d,causal", FWD)
def test_forward_with_poisoned_stages(dtype, layout, b, h, sq, sk, d, causal):
    w = synth.custom("lds race fwd", dtype, layout, b, h, sq, sk, d, causal=causal,
                     std=0.5 if dtype == "fp16" else 1.0, seed=700 + sq + d)
    full_parity(synth.make_inputs(w), name=f"poisoned LDS fwd {dtype} {layout} h={h} sq={sq} "
                                           f"sk={sk} d={d} causal={causal}")


@pytest.mark.parametrize("d", [128, 256])
def test_splitk_with_poisoned_stages(d):
    # key shares that start past the first tile (t0 > 0) and one-tile shares
    w = synth.custom("lds race splitk", "bf16", "bhsd", 1, 3, 300, 900, d, causal=True,
                     seed=790 + d)
    splitk.splitk_parity(w, 5)


def test_forward_c3_with_poisoned_stages():
    full_parity(synth.make_inputs("c3"), name="poisoned LDS fwd c3")


BWD = [
    ("bf16", 2, 3, 129, 200, 64, True),
    ("fp16", 2, 4, 700, 1100, 128, False),   # several dQ query blocks and dK/dV key blocks
    ("bf16", 1, 2, 300, 420, 256, True),     # head_dim 256 kernels
    ("bf16", 2, 3, 129, 200, 80, False),
]


@pytest.mark.parametrize("dtype,b,h,sq,sk,d,causal", BWD)
def test_backward_with_poisoned_stages(dtype, b, h, sq, sk, d, causal):
    w = synth.custom(f"lds race bwd {dtype} d{d}", dtype, "bhsd", b, h, sq, sk, d, causal=causal,
                     seed=750 + d)
    bwd.full_bwd_parity(w, tag=" (poisoned LDS)")
