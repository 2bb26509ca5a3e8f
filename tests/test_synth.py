"""The seeded input generator: determinism, rounding and the stress recipe."""
import numpy as np
import torch

from tiled_attention_04_amd import synth


def test_same_seed_same_bits():
    a = synth.make_inputs("c1")
    b = synth.make_inputs("c1")
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_chunked_draw_equals_single_draw():
    rng1 = np.random.default_rng(5)
    rng2 = np.random.default_rng(5)
    n = synth._CHUNK + 12345
    whole = rng1.standard_normal(n)
    parts = np.concatenate([rng2.standard_normal(synth._CHUNK), rng2.standard_normal(12345)])
    assert np.array_equal(whole, parts)


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal(100000) * 4).astype(np.float32)
    ours = synth.round_to_dtype(x32.astype(np.float64), "bf16")
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert synth.round_to_dtype(np.array([1.0 + 2.0 ** -8]), "bf16")[0] == 0x3F80
    assert synth.round_to_dtype(np.array([1.0 + 3 * 2.0 ** -8]), "bf16")[0] == 0x3F82
    # widening is exact
    assert np.array_equal(synth.widen(ref, "bf16"), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).double().numpy())


def test_workload_shapes_and_distribution():
    w = synth.WORKLOADS["c2"]
    x = synth.make_inputs("c2")
    assert x.q.shape == (1000, 16, 64) and x.k.shape == (1537, 16, 64) and x.q.dtype == np.float16
    vals = synth.widen(x.k, "fp16")
    assert abs(vals.std() - w.std) < 0.01 and abs(vals.mean()) < 0.01
    assert w.strides("q") == (1000 * 16 * 64, 64, 16 * 64, 1)
    assert w.strides("k") == (1537 * 16 * 64, 64, 16 * 64, 1)


def test_stress_rows_are_scaled_exactly():
    w = synth.custom("stress", "bf16", "bhsd", 1, 2, 64, 300, 16, causal=True, seed=9,
                     stress_frac=0.01, stress_factor=8.0)
    plain = synth.custom("plain", "bf16", "bhsd", 1, 2, 64, 300, 16, causal=True, seed=9)
    a, b = synth.make_inputs(w), synth.make_inputs(plain)
    assert len(a.stressed_rows) == 2
    for (bb, h), idx in a.stressed_rows.items():
        assert len(idx) == 3 and len(set(idx.tolist())) == 3
        ka = synth.widen(a.k[bb, h], "bf16")
        kb = synth.widen(b.k[bb, h], "bf16")
        mask = np.zeros(300, bool)
        mask[idx] = True
        assert np.array_equal(ka[mask], 8.0 * kb[mask])
        assert np.array_equal(ka[~mask], kb[~mask])


def test_flop_convention():
    assert synth.WORKLOADS["c5"].flops() == 4.0 * 16 * 32768 * 32768 * 128 / 2
    assert synth.WORKLOADS["c2"].flops() == 4.0 * 16 * 1000 * 1537 * 64


def test_e5m2_rounding_matches_torch_and_round_trips():
    # RNE to e5m2 agrees with torch's float32 -> float8_e5m2 conversion over
    # normals, subnormals, ties and the largest finite value
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000) * np.exp2(rng.uniform(-20, 15, 50000))
    x = np.concatenate([x, [0.0, 2.0 ** -17, 3 * 2.0 ** -18, 2.0 ** -16, 1.125, 1.375, 2.5,
                            -3.5 * 2.0 ** -16, 57344.0, -57344.0]])
    x = x[np.abs(x) <= 57344.0].astype(np.float32).astype(np.float64)
    mine = synth.round_to_dtype(x, "e5m2")
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    # every finite code decodes exactly and rounds back to itself (-0 aside)
    codes = np.arange(256, dtype=np.uint8)
    vals = synth.widen(codes, "e5m2")
    fin = np.isfinite(vals) & (codes != 0x80)
    assert np.array_equal(synth.round_to_dtype(vals[fin], "e5m2"), codes[fin])
    assert vals[0x3C] == 1.0 and vals[0x7B] == 57344.0 and vals[0x01] == 2.0 ** -16


def test_integer_score_inputs_give_small_integer_scores():
    w = synth.custom("int scores", "e5m2", "bhsd", 1, 2, 40, 70, 64, seed=4)
    inp = synth.make_integer_score_inputs(w)
    q, k = inp.as_bhsd_f64("q"), inp.as_bhsd_f64("k")
    assert np.all(np.count_nonzero(q, axis=-1) == 4)
    s = q @ np.swapaxes(k, -1, -2)
    assert np.array_equal(s, np.rint(s))
    span = s.max(axis=-1) - s.min(axis=-1)
    assert span.max() <= 16
