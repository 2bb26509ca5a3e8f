"""Pins for the CPU oracle: checks against what the mathematics fixes.

None of these re-types the oracle's own loop.  Each pin compares the oracle
with something independent of it: a 50-digit decimal brute force of the
definition without the max shift, closed forms, invariants, scipy's
logsumexp/softmax on the scores, a hand-derived worked example, and the
independent NumPy oracle.  ``PINS`` is also run against deliberately broken
builds of the C oracle (planted mistakes, on the CPU) to show that each
plausible mistake fails at least one pin.
"""
import decimal
import math
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import oracle_np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _visible(i, sk, causal):
    return [j for j in range(sk) if (not causal or j <= i)]


# ----------------------------------------------------------------------------
# pins: each takes fwd(q, k, v, sm_scale, causal) -> (o, lse) and raises on
# disagreement
# ----------------------------------------------------------------------------

def pin_decimal_bruteforce(fwd):
    """Tiny random cases against a 50-digit decimal evaluation of
    P = exp(S) / sum exp(S) (no max shift), O = P V, L = ln sum exp(S)."""
    ctx = decimal.Context(prec=50)
    rng = np.random.default_rng(7)
    for (B, H, sq, sk, d, causal) in [(1, 1, 3, 4, 2, False), (1, 2, 5, 3, 3, True),
                                      (2, 1, 4, 6, 5, True), (1, 1, 6, 6, 4, False),
                                      (1, 1, 2, 7, 8, False)]:
        q, k, v = _rand(rng, B, H, sq, d), _rand(rng, B, H, sk, d), _rand(rng, B, H, sk, d)
        scale = 0.7
        o, lse = fwd(q, k, v, scale, causal)
        for b in range(B):
            for h in range(H):
                for i in range(sq):
                    vis = _visible(i, sk, causal)
                    e = []
                    for j in vis:
                        dot = sum((decimal.Decimal(float(q[b, h, i, t])) *
                                   decimal.Decimal(float(k[b, h, j, t])) for t in range(d)),
                                  decimal.Decimal(0))
                        e.append(ctx.exp(ctx.multiply(decimal.Decimal(scale), dot)))
                    z = sum(e, decimal.Decimal(0))
                    ref_lse = float(ctx.ln(z))
                    assert abs(lse[b, h, i] - ref_lse) < 1e-13, (b, h, i, lse[b, h, i], ref_lse)
                    for t in range(d):
                        acc = sum((e[n] * decimal.Decimal(float(v[b, h, j, t]))
                                   for n, j in enumerate(vis)), decimal.Decimal(0))
                        ref = float(acc / z)
                        assert abs(o[b, h, i, t] - ref) < 1e-13, (b, h, i, t, o[b, h, i, t], ref)


def pin_zero_queries(fwd):
    """Q = 0: every visible score is 0, so O_i = mean of the visible V rows and
    L_i = ln |visible(i)|; |visible(i)| = min(i+1, s_k) causal, s_k otherwise."""
    rng = np.random.default_rng(11)
    for (sq, sk, causal) in [(9, 9, True), (5, 12, True), (12, 5, True), (7, 13, False)]:
        v = _rand(rng, 1, 2, sk, 3)
        q = np.zeros((1, 2, sq, 3))
        k = _rand(rng, 1, 2, sk, 3)
        o, lse = fwd(q, k, v, 1.3, causal)
        for h in range(2):
            for i in range(sq):
                n = min(i + 1, sk) if causal else sk
                np.testing.assert_allclose(o[0, h, i], v[0, h, :n].mean(axis=0), atol=1e-14)
                assert abs(lse[0, h, i] - math.log(n)) < 1e-14


def pin_causal_row0(fwd):
    """Causal row 0 sees key 0 only: O_0 = V_0 and L_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 2, 3, 6, 4), _rand(rng, 2, 3, 9, 4), _rand(rng, 2, 3, 9, 4)
    o, lse = fwd(q, k, v, 0.9, True)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.9 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               atol=1e-14)


def pin_single_key(fwd):
    """s_k = 1: every row returns V_0, and L_i = scale * q_i . k_0."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 2, 5, 3), _rand(rng, 1, 2, 1, 3), _rand(rng, 1, 2, 1, 3)
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, np.broadcast_to(v[:, :, :1], o.shape), atol=1e-15)
        np.testing.assert_allclose(lse, 0.5 * (q @ k[:, :, 0, :, None])[..., 0], atol=1e-14)


def pin_constant_values(fwd):
    """All V rows equal c: O_i = c whatever the weights."""
    rng = np.random.default_rng(14)
    q, k = _rand(rng, 1, 1, 7, 5, std=3.0), _rand(rng, 1, 1, 11, 5, std=3.0)
    c = np.array([1.5, -2.0, 0.25, 7.0, -0.125])
    v = np.broadcast_to(c, (1, 1, 11, 5)).copy()
    for causal in (False, True):
        o, _ = fwd(q, k, v, 0.8, causal)
        np.testing.assert_allclose(o[0, 0], np.broadcast_to(c, (7, 5)), atol=1e-13)


def pin_identical_keys(fwd):
    """All K rows equal: scores are equal along a row, so O_i is the mean of
    the visible V rows and L_i = scale * q_i . k + ln |visible(i)|."""
    rng = np.random.default_rng(15)
    krow = _rand(rng, 4)
    q = _rand(rng, 1, 1, 8, 4, std=2.0)
    k = np.broadcast_to(krow, (1, 1, 10, 4)).copy()
    v = _rand(rng, 1, 1, 10, 4)
    for causal in (False, True):
        o, lse = fwd(q, k, v, 1.1, causal)
        for i in range(8):
            n = min(i + 1, 10) if causal else 10
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-13)
            assert abs(lse[0, 0, i] - (1.1 * q[0, 0, i] @ krow + math.log(n))) < 1e-13


def pin_identity_values(fwd):
    """V = identity (d = s_k) makes O the probability matrix itself: rows sum
    to 1, hidden keys get exactly 0, and ln P_ij + L_i equals the score
    scale * q_i . k_j for every visible key."""
    rng = np.random.default_rng(16)
    sk = 6
    for (sq, causal) in [(6, True), (4, False), (9, True)]:
        q, k = _rand(rng, 1, 1, sq, sk), _rand(rng, 1, 1, sk, sk)
        v = np.eye(sk)[None, None]
        p, lse = fwd(q, k, v, 0.6, causal)
        p = p[0, 0]
        s = 0.6 * (q[0, 0] @ k[0, 0].T)
        np.testing.assert_allclose(p.sum(axis=1), np.ones(sq), atol=1e-14)
        for i in range(sq):
            for j in range(sk):
                if causal and j > i:
                    assert p[i, j] == 0.0
                else:
                    assert p[i, j] > 0.0
                    assert abs(math.log(p[i, j]) + lse[0, 0, i] - s[i, j]) < 1e-12


def pin_scipy_routines(fwd):
    """L = scipy.special.logsumexp of the masked scores and O = softmax(S) V
    with scipy.special.softmax, on a ragged causal and a non-causal case."""
    rng = np.random.default_rng(17)
    for (sq, sk, causal) in [(13, 13, True), (7, 19, False), (19, 7, True)]:
        q, k, v = _rand(rng, 1, 1, sq, 8), _rand(rng, 1, 1, sk, 8), _rand(rng, 1, 1, sk, 8)
        o, lse = fwd(q, k, v, 0.35, causal)
        s = 0.35 * (q[0, 0] @ k[0, 0].T)
        if causal:
            s = np.where(np.arange(sk)[None, :] > np.arange(sq)[:, None], -np.inf, s)
        np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(s, axis=1), atol=1e-13)
        np.testing.assert_allclose(o[0, 0], scipy.special.softmax(s, axis=1) @ v[0, 0], atol=1e-13)


def pin_invariances(fwd):
    """Non-causal: permuting keys (K and V rows together) changes nothing;
    permuting queries permutes the outputs; adding one vector w to every key
    shifts each row's scores by a constant, leaving O and adding scale*q_i.w
    to L_i; sm_scale = 0 gives the plain mean of V."""
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 1, 2, 6, 5), _rand(rng, 1, 2, 9, 5), _rand(rng, 1, 2, 9, 5)
    o, lse = fwd(q, k, v, 0.45, False)
    perm = rng.permutation(9)
    o2, lse2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.45, False)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    qp = rng.permutation(6)
    o3, lse3 = fwd(q[:, :, qp], k, v, 0.45, False)
    np.testing.assert_allclose(o3, o[:, :, qp], atol=1e-13)
    np.testing.assert_allclose(lse3, lse[:, :, qp], atol=1e-13)
    w = _rand(rng, 5)
    o4, lse4 = fwd(q, k + w, v, 0.45, False)
    np.testing.assert_allclose(o4, o, atol=1e-12)
    np.testing.assert_allclose(lse4, lse + 0.45 * (q @ w), atol=1e-12)
    o5, lse5 = fwd(q, k, v, 0.0, False)
    np.testing.assert_allclose(o5, np.broadcast_to(v.mean(axis=2, keepdims=True), o5.shape),
                               atol=1e-14)
    np.testing.assert_allclose(lse5, np.full(lse5.shape, math.log(9)), atol=1e-14)


def pin_golden_worked_example(fwd):
    """The hand-derived example in tests/golden/worked_example.txt."""
    q = np.array([1.0, 1.0, 0.0]).reshape(1, 1, 3, 1)
    k = np.array([0.0, math.log(2.0), math.log(3.0)]).reshape(1, 1, 3, 1)
    v = np.array([6.0, 0.0, -6.0]).reshape(1, 1, 3, 1)
    consts = {"0": 0.0, "ln3": math.log(3.0), "ln6": math.log(6.0)}
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 6
    out = {c: fwd(q, k, v, 1.0, bool(c)) for c in (0, 1)}
    for causal, row, o_ref, l_ref in rows:
        o, lse = out[int(causal)]
        assert abs(o[0, 0, int(row), 0] - float(o_ref)) < 1e-14
        assert abs(lse[0, 0, int(row)] - consts[l_ref]) < 1e-14


def pin_matches_numpy_oracle(fwd):
    """The independent NumPy float64 oracle, on ragged shapes, both masks."""
    rng = np.random.default_rng(19)
    for (B, H, sq, sk, d, causal) in [(2, 3, 37, 53, 16, False), (1, 2, 70, 45, 24, True),
                                      (1, 1, 129, 129, 8, True)]:
        q, k, v = _rand(rng, B, H, sq, d), _rand(rng, B, H, sk, d), _rand(rng, B, H, sk, d)
        o, lse = fwd(q, k, v, 0.3, causal)
        o_np, lse_np = oracle_np.attention_forward(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, o_np, atol=1e-12)
        np.testing.assert_allclose(lse, lse_np, atol=1e-12)


PINS = [pin_decimal_bruteforce, pin_zero_queries, pin_causal_row0, pin_single_key,
        pin_constant_values, pin_identical_keys, pin_identity_values, pin_scipy_routines,
        pin_invariances, pin_golden_worked_example, pin_matches_numpy_oracle]


def _c_fwd(lib=None):
    def fwd(q, k, v, sm_scale, causal):
        return oracle.forward(q, k, v, sm_scale, causal, lib=lib)
    return fwd


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_oracle_pin(pin):
    pin(_c_fwd())


@pytest.mark.parametrize("pin", [p for p in PINS if p is not pin_matches_numpy_oracle],
                         ids=lambda p: p.__name__)
def test_numpy_oracle_pin(pin):
    pin(lambda q, k, v, s, c: oracle_np.attention_forward(q, k, v, s, c))


def test_rows_entry_matches_full():
    rng = np.random.default_rng(20)
    q, k, v = _rand(rng, 2, 3, 17, 8), _rand(rng, 2, 3, 23, 8), _rand(rng, 2, 3, 23, 8)
    o, lse = oracle.forward(q, k, v, 0.4, True)
    rows = rng.choice(2 * 3 * 17, size=40, replace=False)
    o_r, lse_r = oracle.forward_rows(q, k, v, 0.4, True, rows=rows)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(lse_r, lse.reshape(-1)[rows])


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 1, 2, 2))
    k = np.zeros((1, 1, 0, 2))
    with pytest.raises(ValueError):
        oracle.forward(q, k, k, 1.0, False)
    with pytest.raises(ValueError):
        oracle.forward_rows(q, np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), 1.0, False,
                            rows=[5])


# ----------------------------------------------------------------------------
# planted mistakes: each edit of fa_oracle.c below is a plausible bug; the pin
# suite must reject every one of them.
# ----------------------------------------------------------------------------
MUTANTS = {
    "diagonal_excluded": ("n_visible = i + 1;", "n_visible = (i > 0) ? i : 1;"),
    "scale_dropped": ("score[j] = sm_scale * dot;", "score[j] = dot;"),
    "k_transposed": ("dot += q_row[t] * k_row[t];", "dot += q_row[t] * k_head[t * seq_k + j];"),
    "lse_missing_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "exponent_sign": ("score[j] = exp(score[j] - m);", "score[j] = exp(m - score[j]);"),
    "not_normalised": ("const double p = score[j] / l;", "const double p = score[j];"),
    "last_key_dropped": ("int64_t n_visible = seq_k;",
                         "int64_t n_visible = seq_k > 1 ? seq_k - 1 : 1;"),
    "v_row_from_query": ("const double* v_row = v_head + j * head_dim;",
                         "const double* v_row = v_head + (i % seq_k) * head_dim;"),
    "causal_ignored": ("if (causal && i + 1 < n_visible)", "if (causal < 0 && i + 1 < n_visible)"),
    "k_head_offset_shared": ("k + bh * seq_k * head_dim,", "k,"),
    "lse_log2": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, mutant_dir):
    src = open(os.path.join(ROOT, "oracle", "fa_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"anchor for {name} not found exactly once"
    mutated = src.replace(old, new)
    c_path = os.path.join(mutant_dir, f"{name}.c")
    so_path = os.path.join(mutant_dir, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-w", c_path, "-o",
                           so_path, "-lm"])
    lib = oracle.load_variant(so_path)
    fwd = _c_fwd(lib)
    failed = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
