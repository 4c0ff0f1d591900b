"""Pins for the oracle's backward (oracle.attn_bwd), all on the CPU.

The pages name a backward kernel class but print no gradient formula, so the
backward is the calculus of the forward definition (page "flash-attn 实现
prefill 阶段", section 问题分析).  It is pinned to things other than itself:

* central finite differences of the (already pinned) forward oracle;
* torch's fp64 CPU autograd through scaled_dot_product_attention;
* a two-key closed form (d = 1), derived by hand from the logistic form of a
  two-way softmax;
* invariants the forward fixes: adding one vector to every key leaves O
  unchanged (sum_j dK_j = 0); adding one vector to every value adds it to
  every O row (sum_j dV_j = sum_i dO_i); scores are bilinear in q and k
  (sum q.dQ = sum k.dK per head); a single key gives dQ = dK = 0.

Each deliberate mistake in oracle.BWD_MUTANTS fails at least one pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle


def _rand(seed, b, h, sq, sk, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, h, sq, d))
    k = rng.standard_normal((b, h, sk, d))
    v = rng.standard_normal((b, h, sk, d))
    g = rng.standard_normal((b, h, sq, d))
    return q, k, v, g


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


def pin_finite_differences(f):
    """Central differences of L = sum(O * dO) through the forward oracle."""
    worst = 0.0
    for causal in (False, True):
        q, k, v, g = _rand(11 + causal, 1, 2, 5, 7, 3)
        scale = 0.7
        dq, dk, dv = f(q, k, v, g, scale, causal)

        def loss(qq, kk, vv):
            o, _ = oracle.attn(qq, kk, vv, scale, causal, nthreads=1)
            return float(np.sum(o * g))

        eps = 1e-6
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            x = (q, k, v)[which]
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                plus = [q, k, v]
                minus = [q, k, v]
                plus[which] = x.copy()
                plus[which][idx] += eps
                minus[which] = x.copy()
                minus[which][idx] -= eps
                num[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
            worst = max(worst, float(np.max(np.abs(num - grad))))
    return worst, 1e-7


def pin_torch_autograd(f):
    """torch's fp64 CPU autograd through scaled_dot_product_attention (its
    is_causal is the top-left j <= i mask, the one used here)."""
    import torch
    worst = 0.0
    for causal, (sq, sk) in ((False, (9, 13)), (True, (13, 13)), (True, (6, 11))):
        q, k, v, g = _rand(23 + sq + sk, 2, 3, sq, sk, 8)
        scale = 0.35
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        if causal:
            mask = torch.ones(sq, sk, dtype=torch.bool).tril()
            out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        else:
            out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        out.backward(torch.from_numpy(g))
        dq, dk, dv = f(q, k, v, g, scale, causal)
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            worst = max(worst, _rel(mine, ref.numpy()))
    return worst, 1e-12


def pin_two_key_closed_form(f):
    """d = 1, two keys a, b with values va, vb: the weight of key a is the
    logistic function p = 1 / (1 + exp(-scale q (a - b))), O = p va + (1-p) vb,
    so dO/dq = p(1-p) scale (a-b)(va-vb), dO/da = p(1-p) scale q (va-vb),
    dO/db = -dO/da, dO/dva = p, dO/dvb = 1 - p."""
    worst = 0.0
    for (qv, a, b, va, vb, gv, scale) in ((0.8, 1.5, -0.5, 2.0, -1.0, 1.3, 0.9),
                                          (-1.2, 0.3, 0.7, -0.4, 0.6, -0.7, 1.7)):
        q = np.array(qv).reshape(1, 1, 1, 1)
        k = np.array([a, b]).reshape(1, 1, 2, 1)
        v = np.array([va, vb]).reshape(1, 1, 2, 1)
        g = np.array(gv).reshape(1, 1, 1, 1)
        p = 1.0 / (1.0 + math.exp(-scale * qv * (a - b)))
        w = p * (1 - p) * scale
        exp_dq = gv * w * (a - b) * (va - vb)
        exp_da = gv * w * qv * (va - vb)
        exp_dv = (gv * p, gv * (1 - p))
        dq, dk, dv = f(q, k, v, g, scale, False)
        worst = max(worst, abs(dq.item() - exp_dq), abs(dk[0, 0, 0, 0] - exp_da),
                    abs(dk[0, 0, 1, 0] + exp_da), abs(dv[0, 0, 0, 0] - exp_dv[0]),
                    abs(dv[0, 0, 1, 0] - exp_dv[1]))
    return worst, 1e-14


def pin_key_shift_sum(f):
    """Adding one vector to every key leaves each row's softmax unchanged, so
    the dK rows of a head sum to zero (causal too: the shift is constant over
    the keys a row sees)."""
    worst = 0.0
    for causal in (False, True):
        q, k, v, g = _rand(31 + causal, 2, 2, 17, 17, 5)
        _, dk, _ = f(q, k, v, g, 0.6, causal)
        scale_ref = np.max(np.abs(dk))
        worst = max(worst, float(np.max(np.abs(dk.sum(axis=2)))) / scale_ref)
    return worst, 1e-12


def pin_value_shift_sum(f):
    """Adding c to every value adds c to every output row (rows of P sum to
    one), so sum_j dV_j = sum_i dO_i per head."""
    worst = 0.0
    for causal in (False, True):
        q, k, v, g = _rand(41 + causal, 2, 2, 12, 15, 4)
        _, _, dv = f(q, k, v, g, 1.1, causal)
        worst = max(worst, _rel(dv.sum(axis=2), g.sum(axis=2)))
    return worst, 1e-12


def pin_bilinear_balance(f):
    """Each score is scale * q_i . k_j, so scaling all of Q by t or all of K by
    t has the same effect: sum q.dQ = sum k.dK per head."""
    worst = 0.0
    for causal in (False, True):
        q, k, v, g = _rand(51 + causal, 1, 3, 10, 14, 6)
        dq, dk, _ = f(q, k, v, g, 0.45, causal)
        lhs = np.sum(q * dq, axis=(2, 3))
        rhs = np.sum(k * dk, axis=(2, 3))
        worst = max(worst, float(np.max(np.abs(lhs - rhs))) / float(np.max(np.abs(rhs))))
    return worst, 1e-12


def pin_single_key(f):
    """One key: P = 1 whatever the scores, so dQ = dK = 0 and dV = sum_i dO_i."""
    q, k, v, g = _rand(61, 1, 2, 6, 1, 4)
    dq, dk, dv = f(q, k, v, g, 0.8, False)
    return max(float(np.max(np.abs(dq))), float(np.max(np.abs(dk))),
               float(np.max(np.abs(dv - g.sum(axis=2, keepdims=True))))), 1e-13


PINS = {
    "finite_differences": pin_finite_differences,
    "torch_autograd": pin_torch_autograd,
    "two_key_closed_form": pin_two_key_closed_form,
    "key_shift_sum": pin_key_shift_sum,
    "value_shift_sum": pin_value_shift_sum,
    "bilinear_balance": pin_bilinear_balance,
    "single_key": pin_single_key,
}


def _bwd(q, k, v, g, scale, causal):
    return oracle.attn_bwd(q, k, v, g, scale, causal, nthreads=2)


@pytest.mark.parametrize("pin", sorted(PINS))
def test_bwd_pin_holds(pin):
    err, tol = PINS[pin](_bwd)
    assert err <= tol, (pin, err, tol)


@pytest.mark.parametrize("mutant", sorted(oracle.BWD_MUTANTS))
def test_each_bwd_mutant_fails_a_pin(mutant):
    def f(q, k, v, g, scale, causal):
        return oracle.attn_bwd(q, k, v, g, scale, causal, mutant=mutant, nthreads=2)
    failed = []
    for name, pin in PINS.items():
        err, tol = pin(f)
        if not err <= tol:
            failed.append(name)
    assert failed, mutant


def test_bwd_threads_do_not_change_results():
    q, k, v, g = _rand(71, 2, 3, 33, 29, 8)
    a = oracle.attn_bwd(q, k, v, g, 0.3, True, nthreads=1)
    b = oracle.attn_bwd(q, k, v, g, 0.3, True, nthreads=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_rejects_bad_arguments():
    q, k, v, g = _rand(81, 1, 1, 4, 4, 2)
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, k, v, g[:, :, :3], 1.0)
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, k[..., :1], v, g, 1.0)
