"""Pins of the gradient oracle (oracle/fa_oracle_bwd.c and the NumPy twin).

Each pin checks the backward against something other than itself:
  * central finite differences of the (separately pinned) forward oracle;
  * torch autograd on the CPU in float64 (an independent implementation);
  * closed forms and invariants of the softmax gradient:
      - a softmax row is unchanged when one vector is added to every key, so
        the sum over keys of dK is 0;
      - every visible row of P sums to 1, so the sum over keys of dV equals
        the sum over queries of dO;
      - identical keys, or identical value rows, make every dS row sum to
        zero against a constant, so dQ = 0 (and dK = 0 for constant values);
      - a single key gives P = 1: dQ = dK = 0 and dV_0 = sum_i dO_i;
      - dO = 0 gives zero gradients;
  * the C and NumPy oracles agree.
The planted-mistake tests at the end edit fa_oracle_bwd.c in plausible ways
and require every edit to fail at least one pin.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import oracle_np  # noqa: E402


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _inputs(seed, B, H, Sq, Sk, D):
    rng = np.random.default_rng(seed)
    return (_rand(rng, B, H, Sq, D), _rand(rng, B, H, Sk, D), _rand(rng, B, H, Sk, D),
            _rand(rng, B, H, Sq, D))


def pin_finite_differences(bwd):
    """Central differences of sum(dO * O(q, k, v)) through the forward oracle."""
    for causal, scale, (Sq, Sk) in [(False, 0.8, (5, 7)), (True, 0.8, (6, 4)),
                                    (True, -0.6, (5, 7))]:
        q, k, v, do = _inputs(11, 1, 2, Sq, Sk, 3)
        dq, dk, dv = bwd(q, k, v, do, scale, causal)[:3]

        def loss(q_, k_, v_):
            o, _ = oracle.forward(q_, k_, v_, scale, causal)
            return float(np.sum(do * o))

        h = 1e-5
        for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.empty_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                saved = arr[idx]
                arr[idx] = saved + h
                fp = loss(q, k, v)
                arr[idx] = saved - h
                fm = loss(q, k, v)
                arr[idx] = saved
                num[idx] = (fp - fm) / (2 * h)
            err = np.max(np.abs(num - grad))
            assert err < 1e-7, f"d{name} vs finite differences: {err:.3e} (causal={causal})"


def pin_torch_autograd(bwd):
    """torch autograd on the CPU in float64 on the materialised definition."""
    torch = pytest.importorskip("torch")
    for causal, (Sq, Sk) in [(False, (19, 23)), (True, (19, 23)), (True, (23, 19))]:
        q, k, v, do = _inputs(12, 2, 2, Sq, Sk, 8)
        scale = 0.35
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        if causal:
            mask = torch.arange(Sk)[None, :] > torch.arange(Sq)[:, None]
            s = s.masked_fill(mask, float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), tv)
        o.backward(torch.tensor(do, dtype=torch.float64))
        dq, dk, dv = bwd(q, k, v, do, scale, causal)[:3]
        for name, mine, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
            err = np.max(np.abs(mine - ref.numpy()))
            assert err < 1e-10, f"d{name} vs torch autograd: {err:.3e} (causal={causal})"


def pin_dk_sums_to_zero(bwd):
    for causal in (False, True):
        q, k, v, do = _inputs(13, 2, 3, 17, 17, 6)
        dk = bwd(q, k, v, do, 0.5, causal)[1]
        tot = dk.sum(axis=2)
        assert np.max(np.abs(tot)) < 1e-10 * max(1.0, np.max(np.abs(dk))), tot


def pin_dv_sums_to_dout_sum(bwd):
    for causal in (False, True):
        q, k, v, do = _inputs(14, 2, 3, 17, 21, 6)
        dv = bwd(q, k, v, do, 0.5, causal)[2]
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-11)


def pin_identical_keys_zero_dq(bwd):
    q, k, v, do = _inputs(15, 1, 2, 9, 12, 5)
    k[:] = k[:, :, :1, :]
    for causal in (False, True):
        dq = bwd(q, k, v, do, 0.9, causal)[0]
        assert np.max(np.abs(dq)) < 1e-12


def pin_constant_values_zero_qk_grads(bwd):
    q, k, v, do = _inputs(16, 1, 2, 9, 12, 5)
    v[:] = v[:, :, :1, :]
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.9, causal)[:3]
        assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
        assert np.max(np.abs(dv)) > 1e-3  # P^T dO itself is not trivial


def pin_single_key(bwd):
    q, k, v, do = _inputs(17, 2, 2, 7, 1, 4)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 1.3, causal)[:3]
        assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
        np.testing.assert_allclose(dv[:, :, 0], do.sum(axis=2), rtol=0, atol=1e-12)


def pin_zero_dout(bwd):
    q, k, v, do = _inputs(18, 1, 2, 8, 8, 4)
    grads = bwd(q, k, v, np.zeros_like(do), 0.7, True)[:3]
    assert all(np.max(np.abs(g)) == 0.0 for g in grads)


def pin_matches_numpy_oracle(bwd):
    for causal, (Sq, Sk) in [(False, (33, 47)), (True, (47, 33)), (True, (40, 40))]:
        q, k, v, do = _inputs(19, 2, 3, Sq, Sk, 16)
        mine = bwd(q, k, v, do, 0.25, causal)[:3]
        ref = oracle_np.attention_backward(q, k, v, do, 0.25, causal)
        for a, b in zip(mine, ref):
            assert np.max(np.abs(a - b)) < 1e-12


PINS = [pin_finite_differences, pin_torch_autograd, pin_dk_sums_to_zero, pin_dv_sums_to_dout_sum,
        pin_identical_keys_zero_dq, pin_constant_values_zero_qk_grads, pin_single_key,
        pin_zero_dout, pin_matches_numpy_oracle]


def _c_bwd(lib=None):
    def bwd(q, k, v, do, scale, causal):
        return oracle.backward(q, k, v, do, scale, causal, lib=lib)
    return bwd


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_bwd_oracle_pin(pin):
    pin(_c_bwd())


@pytest.mark.parametrize("pin", [p for p in PINS if p is not pin_matches_numpy_oracle],
                         ids=lambda p: p.__name__)
def test_numpy_bwd_oracle_pin(pin):
    pin(lambda q, k, v, do, s, c: oracle_np.attention_backward(q, k, v, do, s, c))


def test_delta_is_rowsum_of_dout_times_o():
    q, k, v, do = _inputs(20, 2, 2, 13, 9, 6)
    delta = oracle.backward(q, k, v, do, 0.6, True)[3]
    o, _ = oracle.forward(q, k, v, 0.6, True)
    np.testing.assert_allclose(delta, np.sum(do * o, axis=-1), rtol=0, atol=1e-13)


def test_row_entries_match_full():
    q, k, v, do = _inputs(21, 2, 3, 17, 23, 8)
    for causal in (False, True):
        dq, dk, dv, _ = oracle.backward(q, k, v, do, 0.4, causal)
        rng = np.random.default_rng(22)
        rows = rng.choice(2 * 3 * 17, size=30, replace=False)
        keys = rng.choice(2 * 3 * 23, size=30, replace=False)
        np.testing.assert_allclose(oracle.backward_dq_rows(q, k, v, do, 0.4, causal, rows),
                                   dq.reshape(-1, 8)[rows], rtol=0, atol=1e-13)
        dk_r, dv_r = oracle.backward_dkv_rows(q, k, v, do, 0.4, causal, keys)
        np.testing.assert_allclose(dk_r, dk.reshape(-1, 8)[keys], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv_r, dv.reshape(-1, 8)[keys], rtol=0, atol=1e-13)


def test_bwd_oracle_rejects_bad_arguments():
    q, k, v, do = _inputs(23, 1, 1, 4, 4, 2)
    with pytest.raises(ValueError):
        oracle.backward(q, k[:, :, :0], v[:, :, :0], do, 1.0, False)
    with pytest.raises(ValueError):
        oracle.backward_dq_rows(q, k, v, do, 1.0, False, [4])
    with pytest.raises(ValueError):
        oracle.backward_dkv_rows(q, k, v, do, 1.0, False, [-1])


# ----------------------------------------------------------------------------
# planted mistakes in fa_oracle_bwd.c: every one must fail some pin
# ----------------------------------------------------------------------------
MUTANTS = {
    "delta_dropped": ("*ds_out = p * (dp - D);", "*ds_out = p * dp;"),
    "delta_sign": ("*ds_out = p * (dp - D);", "*ds_out = p * (dp + D);"),
    "dk_unscaled": ("dkh[j * head_dim + t] += sm_scale * ds * q_row[t];",
                    "dkh[j * head_dim + t] += ds * q_row[t];"),
    "dv_from_ds": ("dvh[j * head_dim + t] += p * do_row[t];",
                   "dvh[j * head_dim + t] += ds * do_row[t];"),
    "dq_from_v": ("dqh[i * head_dim + t] += sm_scale * ds * k_row[t];",
                  "dqh[i * head_dim + t] += sm_scale * ds * vh[j * head_dim + t];"),
    "lse_without_max": ("const double L = m + log(l);", "const double L = log(l);"),
    "causal_diagonal_dropped": ("if (causal && i + 1 < n) n = i + 1;",
                                "if (causal && i < n) n = i > 0 ? i : 1;"),
    "p_unscaled": ("const double p = exp(sm_scale * s - L);", "const double p = exp(s - L);"),
    "dp_from_k": ("dp += do_row[t] * v_row[t];", "dp += do_row[t] * k_row[t];"),
    "delta_from_q": ("D += do_row[t] * o_row[t];", "D += do_row[t] * q_row[t];"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="oracle_bwd_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_bwd_mistake_is_caught(name, mutant_dir):
    src = open(os.path.join(ROOT, "oracle", "fa_oracle_bwd.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"anchor for {name} not found exactly once"
    c_path = os.path.join(mutant_dir, f"{name}.c")
    so_path = os.path.join(mutant_dir, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-w", c_path, "-o",
                           so_path, "-lm"])
    bwd = _c_bwd(oracle.load_bwd_variant(so_path))
    failed = []
    for pin in PINS:
        try:
            pin(bwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
