"""The fp64 oracle, pinned to things other than itself (CPU only).

* every pin in ``tests/pins.py`` passes for the naive definition, for the
  row-subset entry point and for both online-softmax forms;
* each deliberately broken copy of the definition fails at least one pin;
* the online-softmax recurrence (page "flash.cu", forward_kernel: running
  max m from -inf, running sum l from 0, per-tile rescale) agrees with the
  naive definition by brute force over tiny shapes and tile sizes, including
  tiles that do not divide the sequence;
* the softmax matrix P has rows summing to 1, is zero above the causal
  diagonal and reproduces O = P V and P = exp(s - LSE).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from tests import pins


def naive(q, k, v, scale, causal):
    return oracle.attn(q, k, v, scale, causal)


def rows_form(q, k, v, scale, causal):
    b, h, sq, d = q.shape
    rows = np.arange(b * h * sq)[::-1].copy()  # reversed order on purpose
    o, lse = oracle.attn_rows(q, k, v, rows, scale, causal)
    o_full = np.empty((b * h * sq, d))
    lse_full = np.empty(b * h * sq)
    o_full[rows] = o
    lse_full[rows] = lse
    return o_full.reshape(b, h, sq, d), lse_full.reshape(b, h, sq)


def kv_outer(q, k, v, scale, causal):
    return oracle.attn_online_kv_outer(q, k, v, scale, causal, br=3, bc=2)


def q_outer(q, k, v, scale, causal):
    return oracle.attn_online_q_outer(q, k, v, scale, causal, br=2, bc=3)


FORMS = {"naive": naive, "rows": rows_form, "kv_outer": kv_outer, "q_outer": q_outer}


@pytest.mark.parametrize("pin", sorted(pins.PINS))
@pytest.mark.parametrize("form", sorted(FORMS))
def test_pin_holds(form, pin):
    err = pins.PINS[pin](FORMS[form])
    assert err <= pins.TOL, f"{form} violates pin {pin}: {err}"


@pytest.mark.parametrize("mutant", sorted(oracle.MUTANTS))
def test_each_mutant_fails_a_pin(mutant):
    def broken(q, k, v, scale, causal):
        return oracle.attn_mutant(q, k, v, scale, causal, mutant)
    failed = [name for name, pin in pins.PINS.items() if not pin(broken) <= pins.TOL]
    assert failed, f"mutant {mutant} passes every pin"


SIZES = [1, 2, 3, 5, 17, 63, 64, 65, 130]


@pytest.mark.parametrize("d", [1, 4, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_forms_match_naive_brute_force(d, causal):
    rng = np.random.default_rng(100 + d + 7 * causal)
    worst = 0.0
    for sq, sk in itertools.product(SIZES, SIZES):
        if sq * sk * d > 130 * 130 * 4 and (sq, sk) not in [(130, 130), (65, 64), (64, 65)]:
            continue  # keep the d = 64 sweep to a few large shapes
        q = rng.standard_normal((1, 2, sq, d)) * 1.5
        k = rng.standard_normal((1, 2, sk, d)) * 1.5
        v = rng.standard_normal((1, 2, sk, d))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attn(q, k, v, scale, causal)
        for br, bc in [(1, 1), (2, 3), (64, 64), (7, 5), (sq, sk)]:
            for form in (oracle.attn_online_kv_outer, oracle.attn_online_q_outer):
                o2, l2 = form(q, k, v, scale, causal, br=br, bc=bc)
                worst = max(worst, float(np.max(np.abs(o - o2))), float(np.max(np.abs(lse - l2))))
    assert worst <= 1e-12, worst


@pytest.mark.parametrize("causal", [False, True])
def test_probability_matrix(causal):
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 2, 9, 5)) * 2
    k = rng.standard_normal((2, 2, 11, 5)) * 2
    v = rng.standard_normal((2, 2, 11, 5))
    p, o, lse = oracle.attn_probs(q, k, v, 0.6, causal)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-14
    assert np.all(p >= 0)
    if causal:
        above = np.triu(np.ones((9, 11), bool), k=1)
        assert np.all(p[..., above] == 0.0)
    # O = P V with a library matmul
    assert np.max(np.abs(p @ v - o)) <= 1e-13
    # P = exp(scale q.k - LSE) on allowed entries
    s = 0.6 * (q @ np.swapaxes(k, -1, -2))
    allowed = p > 0
    ref = np.exp(s - lse[..., None])
    assert np.max(np.abs(np.where(allowed, ref, 0.0) - p)) <= 1e-13
    # the matrix entry point's O and LSE are the naive definition's
    o2, l2 = oracle.attn(q, k, v, 0.6, causal)
    assert np.max(np.abs(o - o2)) <= 1e-15 and np.max(np.abs(lse - l2)) <= 1e-15


def test_threads_do_not_change_results():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((2, 3, 50, 16))
    k = rng.standard_normal((2, 3, 70, 16))
    v = rng.standard_normal((2, 3, 70, 16))
    o1, l1 = oracle.attn(q, k, v, 0.25, True, nthreads=1)
    o8, l8 = oracle.attn(q, k, v, 0.25, True, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)


def test_low_precision_inputs_widen_exactly():
    import torch
    x = torch.randn(1, 1, 4, 8).to(torch.bfloat16)
    y = oracle._as_f64(x)
    assert np.array_equal(y, x.to(torch.float64).numpy())


def test_rejects_bad_arguments():
    q = np.zeros((1, 1, 2, 4))
    with pytest.raises(ValueError):
        oracle.attn(q, np.zeros((1, 1, 3, 5)), np.zeros((1, 1, 3, 5)), 1.0)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, q, q, [5], 1.0)
