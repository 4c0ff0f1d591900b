"""Pins for an attention implementation that computes in fp64 on the CPU.

Each pin takes ``f(q, k, v, scale, causal) -> (O, LSE)`` (numpy fp64 in and
out, [b,h,s,d] layout) and returns the largest violation it finds, in units
where ``<= TOL`` passes.  None of them re-types the attention formula: each
checks a property the pages or the mathematics fix -- a hand-worked example,
a closed form, an invariant, or agreement with a library routine.

The same pins are run against the oracle (all must pass) and against
deliberately broken copies of it (each must fail at least one pin), which is
how the test suite shows the pins would catch a plausible mistake.
"""
from __future__ import annotations

import glob
import json
import math
import os

import numpy as np

TOL = 1e-12
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        return math.inf
    if not (np.all(np.isfinite(a)) and np.all(np.isfinite(b))):
        return math.inf
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def golden_cases():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        with open(path) as fh:
            out.append(json.load(fh))
    return out


# ---------------------------------------------------------------------------
# hand-worked examples (tests/golden/*.json)
# ---------------------------------------------------------------------------

def pin_golden(f) -> float:
    worst = 0.0
    for c in golden_cases():
        q, k, v = (np.array(c[x], np.float64) for x in ("q", "k", "v"))
        o, lse = f(q, k, v, c["scale"], c["causal"])
        worst = max(worst, _err(o, c["o"]), _err(lse, c["lse"]))
    return worst


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_two_key_tanh(f) -> float:
    """One query, keys [0, a], values [1, -1]: O = -tanh(s a / 2) and
    LSE = ln(1 + e^{s a}) (softplus), for a spread of a and scales."""
    worst = 0.0
    rng = np.random.default_rng(11)
    for a, s in [(0.0, 1.0), (1.0, 1.0), (-3.5, 0.25), (20.0, 1.0), (-40.0, 0.5)] + \
            [(float(x), float(y)) for x, y in zip(rng.normal(0, 4, 8), rng.uniform(0.1, 2, 8))]:
        q = np.ones((1, 1, 1, 1))
        k = np.array([0.0, a]).reshape(1, 1, 2, 1)
        v = np.array([1.0, -1.0]).reshape(1, 1, 2, 1)
        o, lse = f(q, k, v, s, False)
        z = s * a
        softplus = max(z, 0.0) + math.log1p(math.exp(-abs(z)))
        worst = max(worst, _err(o.ravel(), [-math.tanh(z / 2)]), _err(lse.ravel(), [softplus]))
    return worst


def pin_one_hot_selection(f) -> float:
    """K_j = alpha e_j, Q_i = e_{pi(i)}: query i scores alpha*scale on key
    pi(i) and 0 elsewhere, so O_i = V_{pi(i)} up to sk e^{-alpha scale} and
    LSE_i = alpha scale + ln(1 + (sk-1) e^{-alpha scale}).  The second case uses
    alpha*scale = 1000, far beyond exp's range, so a softmax that does not
    subtract the row maximum overflows."""
    worst = 0.0
    rng = np.random.default_rng(12)
    for (sq, sk, d, alpha, scale) in [(7, 5, 8, 512.0, 1 / math.sqrt(128)),
                                      (4, 6, 6, 4000.0, 0.25)]:
        perm = rng.integers(0, sk, sq)
        q = np.zeros((1, 1, sq, d))
        q[0, 0, np.arange(sq), perm] = 1.0
        k = np.zeros((1, 1, sk, d))
        k[0, 0, np.arange(sk), np.arange(sk)] = alpha
        v = rng.standard_normal((1, 1, sk, d))
        o, lse = f(q, k, v, scale, False)
        z = alpha * scale
        worst = max(worst, _err(o[0, 0], v[0, 0, perm]))
        worst = max(worst, _err(lse[0, 0], np.full(sq, z + math.log1p((sk - 1) * math.exp(-z)))))
    return worst


def pin_uniform_weights(f) -> float:
    """Q = 0: every allowed score is 0, so O_i is the mean of the allowed V
    rows and LSE_i = ln(number of allowed keys); covers causal prefixes,
    sq != sk and a ragged tail."""
    worst = 0.0
    rng = np.random.default_rng(13)
    for (sq, sk, d, causal) in [(5, 9, 3, False), (9, 9, 4, True), (6, 11, 2, True), (11, 4, 3, True)]:
        q = np.zeros((1, 2, sq, d))
        k = rng.standard_normal((1, 2, sk, d))
        v = rng.standard_normal((1, 2, sk, d))
        o, lse = f(q, k, v, 0.3, causal)
        for i in range(sq):
            n = min(i + 1, sk) if causal else sk
            worst = max(worst, _err(o[:, :, i], v[:, :, :n].mean(axis=2)))
            worst = max(worst, _err(lse[:, :, i], np.full((1, 2), math.log(n))))
    return worst


def pin_causal_row0(f) -> float:
    """Causal row 0 sees only key 0: O_0 = V_0 exactly and LSE_0 = scale q_0.k_0."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((2, 3, 8, 16))
    k = rng.standard_normal((2, 3, 8, 16))
    v = rng.standard_normal((2, 3, 8, 16))
    o, lse = f(q, k, v, 0.25, True)
    ref = 0.25 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1)
    return max(_err(o[:, :, 0], v[:, :, 0]), _err(lse[:, :, 0], ref))


def pin_constant_v(f) -> float:
    """v_j = c for all j: O_i = c whatever the weights are."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, 2, 13, 8)) * 3
    k = rng.standard_normal((1, 2, 17, 8)) * 3
    v = np.full((1, 2, 17, 8), 0.375)
    worst = 0.0
    for causal in (False, True):
        o, _ = f(q, k, v, 0.5, causal)
        worst = max(worst, _err(o, np.full_like(o, 0.375)))
    return worst


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_shift_invariance(f) -> float:
    """K'_j = K_j + u: O unchanged, LSE'_i = LSE_i + scale q_i.u."""
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 2, 9, 6))
    k = rng.standard_normal((1, 2, 12, 6))
    v = rng.standard_normal((1, 2, 12, 6))
    u = rng.standard_normal(6)
    worst = 0.0
    for causal in (False, True):
        o1, l1 = f(q, k, v, 0.7, causal)
        o2, l2 = f(q, k + u, v, 0.7, causal)
        worst = max(worst, _err(o1, o2), _err(l2, l1 + 0.7 * (q @ u)))
    return worst


def pin_permutation(f) -> float:
    """Non-causal: permuting (K, V) rows together changes nothing; permuting
    Q rows permutes O and LSE rows."""
    rng = np.random.default_rng(17)
    q = rng.standard_normal((2, 1, 10, 5))
    k = rng.standard_normal((2, 1, 14, 5))
    v = rng.standard_normal((2, 1, 14, 5))
    o, lse = f(q, k, v, 0.4, False)
    pk = rng.permutation(14)
    o2, l2 = f(q, k[:, :, pk], v[:, :, pk], 0.4, False)
    pq = rng.permutation(10)
    o3, l3 = f(q[:, :, pq], k, v, 0.4, False)
    return max(_err(o, o2), _err(lse, l2), _err(o[:, :, pq], o3), _err(lse[:, :, pq], l3))


def pin_scale_law(f) -> float:
    """Scaling Q by 2^e and the scale by 2^-e is exact and leaves O, LSE unchanged."""
    rng = np.random.default_rng(18)
    q = rng.standard_normal((1, 1, 7, 4))
    k = rng.standard_normal((1, 1, 7, 4))
    v = rng.standard_normal((1, 1, 7, 4))
    o1, l1 = f(q, k, v, 0.5, True)
    o2, l2 = f(q * 8.0, k, v, 0.0625, True)
    return max(_err(o1, o2), _err(l1, l2))


def pin_head_independence(f) -> float:
    """Changing one (b, h) slice of Q, K, V changes only that slice's outputs."""
    rng = np.random.default_rng(19)
    q = rng.standard_normal((2, 3, 5, 4))
    k = rng.standard_normal((2, 3, 6, 4))
    v = rng.standard_normal((2, 3, 6, 4))
    o1, l1 = f(q, k, v, 0.5, False)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[1, 2] += 1.0
    k2[1, 2] *= -1.0
    v2[1, 2] += 2.0
    o2, l2 = f(q2, k2, v2, 0.5, False)
    mask = np.ones((2, 3), bool)
    mask[1, 2] = False
    changed = float(np.max(np.abs(o1[1, 2] - o2[1, 2])))
    return max(_err(o1[mask], o2[mask]), _err(l1[mask], l2[mask]),
               0.0 if changed > 1e-3 else math.inf)


# ---------------------------------------------------------------------------
# library routine
# ---------------------------------------------------------------------------

def pin_torch_sdpa(f) -> float:
    """Agreement with torch's fp64 CPU scaled_dot_product_attention (its
    is_causal is the top-left j <= i mask) and with torch.logsumexp of the
    masked scaled scores, on random shapes with sq != sk and ragged sizes."""
    import torch
    worst = 0.0
    rng = np.random.default_rng(20)
    for (b, h, sq, sk, d, causal, scale) in [(1, 2, 33, 33, 16, False, 0.25),
                                             (2, 1, 17, 40, 8, False, 0.125),
                                             (1, 3, 40, 40, 32, True, 1 / math.sqrt(32)),
                                             (1, 1, 20, 37, 12, True, 0.3),
                                             (1, 1, 65, 130, 64, False, 0.125)]:
        q = rng.standard_normal((b, h, sq, d)) * 2
        k = rng.standard_normal((b, h, sk, d)) * 2
        v = rng.standard_normal((b, h, sk, d))
        o, lse = f(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=scale).numpy()
        scores = (tq @ tk.transpose(-1, -2).contiguous()) * scale
        if causal:
            allowed = torch.ones(sq, sk, dtype=torch.bool).tril()
            scores = scores.masked_fill(~allowed, float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1).numpy()
        worst = max(worst, _err(o, ref), _err(lse, ref_lse))
    return worst


PINS = {
    "golden": pin_golden,
    "two_key_tanh": pin_two_key_tanh,
    "one_hot_selection": pin_one_hot_selection,
    "uniform_weights": pin_uniform_weights,
    "causal_row0": pin_causal_row0,
    "constant_v": pin_constant_v,
    "shift_invariance": pin_shift_invariance,
    "permutation": pin_permutation,
    "scale_law": pin_scale_law,
    "head_independence": pin_head_independence,
    "torch_sdpa": pin_torch_sdpa,
}
