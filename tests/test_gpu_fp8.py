"""GPU parity of the FP8 forward (fa_fwd_fp8) against the fp64 oracle.

Inputs: the usual seeded draws, each tensor multiplied by a power of two that
fills the E4M3 range, rounded to OCP E4M3 and paired with the inverse power
of two as its descale factor (``workloads.make_fp8``).  The oracle computes the
plain definition on the dequantized values (stored E4M3 value x descale,
widened exactly to fp64), with the fp32 scale.

Tolerances, derived from what the kernel rounds:
* LSE: the scores are exact products of E4M3 values summed in fp32 and the
  row sum adds fp32 probabilities, so LSE meets the 16-bit forward's bound,
  1e-3 absolute.
* O, element by element: the probabilities enter the second product rounded
  to E4M3.  A normal E4M3 value carries a relative error of at most 2^-4; a
  subnormal one (below 2^-6) an absolute error of at most 2^-10, while the
  row sum is at least 2^8 (the row max contributes exactly 2^8).  So
  |O - O_ref| <= 2^-4 A + 2^-18 n max|v| + 2^-8 |O_ref|, where
  A = sum_j P_ij |v_j| / l_i is the oracle's attention over |V|, n the number
  of keys the row sees, and the last term the bf16 rounding of O.
"""
import sys

import numpy as np
import pytest

import exact_attention_86_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dequant(t, s):
    return t.to(__import__("torch").float64).numpy() * s


def keys_seen(sq, sk, causal):
    i = np.arange(sq)
    return np.minimum(i + 1, sk) if causal else np.full(sq, sk)


def check_fp8(w, seed=None, scale=None):
    import torch
    q8, k8, v8, (dq, dk, dv) = W.make_fp8(w, seed)
    s = float(np.float32(w.scale if scale is None else scale))
    note(f"[fp8] b{w.b} h{w.h} sq{w.sq} sk{w.sk} causal={w.causal} scale={s}")
    o, lse = fa.attention_fp8(q8.cuda(), k8.cuda(), v8.cuda(), causal=w.causal, scale=s,
                              descale_q=dq, descale_k=dk, descale_v=dv)
    torch.cuda.synchronize()
    q, k, v = dequant(q8, dq), dequant(k8, dk), dequant(v8, dv)
    ro, rl = oracle.attn(q, k, v, s, w.causal)
    ra, _ = oracle.attn(q, k, np.abs(v), s, w.causal)
    go = o.double().cpu().numpy()
    gl = lse.double().cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    n = keys_seen(w.sq, w.sk, w.causal)[None, None, :, None]
    vmax = np.max(np.abs(v), axis=2, keepdims=True)
    tol = 2.0 ** -4 * ra + 2.0 ** -18 * n * vmax + 2.0 ** -8 * np.abs(ro) + 1e-6
    err = np.abs(go - ro)
    el = float(np.max(np.abs(gl - rl)))
    note(f"   O max-abs {float(err.max()):.3e}, worst err/tol {float((err / tol).max()):.3f}; LSE max-abs {el:.2e}")
    assert np.all(err <= tol), f"O error over the bound at {np.unravel_index(np.argmax(err / tol), err.shape)}"
    assert el <= 1e-3


CASES = [
    # b, h, sq, sk, causal, scale (None: 1/sqrt(d))
    (1, 2, 128, 128, False, None),
    (1, 2, 128, 128, True, None),
    (2, 3, 200, 328, False, None),
    (1, 2, 300, 300, True, None),
    (1, 2, 100, 257, True, None),
    (1, 2, 333, 150, True, None),
    (1, 1, 1, 1, False, None),
    (1, 2, 1, 77, False, None),
    (1, 2, 77, 1, True, None),
    (2, 2, 640, 384, False, 0.2),
    (1, 2, 190, 140, False, -0.07),
    (2, 4, 1024, 1024, True, None),
    (1, 2, 150, 150, True, 0.0),     # uniform weights over each causal prefix
    (1, 2, 256, 512, False, 1.0),    # near one-hot rows: the reference max moves often
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%dh%d_sq%d_sk%d_%s_%s" % (
    c[0], c[1], c[2], c[3], "causal" if c[4] else "full", c[5]))
def test_fp8_matches_oracle(case):
    b, h, sq, sk, causal, scale = case
    w = W.shape("fp8", "bf16", b, h, sq, sk, 128, causal, scale=scale, seed=31 * sq + sk)
    check_fp8(w)


# many heads (grids of 256-1024 workgroups), ragged query and key tails,
# sq != sk, causal and not
MANY_HEAD_CASES = [
    (1, 256, 300, 300, True, None),
    (2, 128, 260, 260, False, None),
    (1, 256, 200, 333, True, None),
]


@pytest.mark.parametrize("case", MANY_HEAD_CASES, ids=lambda c: "b%dh%d_sq%d_sk%d_%s" % (
    c[0], c[1], c[2], c[3], "causal" if c[4] else "full"))
def test_fp8_many_heads(case):
    b, h, sq, sk, causal, scale = case
    w = W.shape("fp8heads", "bf16", b, h, sq, sk, 128, causal, scale=scale, seed=7 * sq + sk)
    check_fp8(w)


def test_fp8_headline_shape_sampled_rows():
    """The [4, 32, 4096, 128] causal problem at full size; the oracle computes
    sampled rows (first and last tiles of two heads, tile edges, random)."""
    import torch
    w = W.HEADLINE
    q8, k8, v8, (dq, dk, dv) = W.make_fp8(w)
    s = float(np.float32(w.scale))
    note("[fp8] headline shape")
    o, lse = fa.attention_fp8(q8.cuda(), k8.cuda(), v8.cuda(), causal=True, scale=s,
                              descale_q=dq, descale_k=dk, descale_v=dv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    bh = w.b * w.h
    rows = set()
    for hh in (0, bh - 1):
        for i in list(range(0, 128)) + list(range(w.sq - 128, w.sq)):
            rows.add(hh * w.sq + i)
    for i in rng.integers(0, bh * w.sq, 128):
        rows.add(int(i))
    for hh in (3, 77):
        for i in (63, 64, 127, 128, 129, 2047, 2048):
            rows.add(hh * w.sq + i)
    rows = np.array(sorted(rows), dtype=np.int64)
    q, k, v = dequant(q8, dq), dequant(k8, dk), dequant(v8, dv)
    ro, rl = oracle.attn_rows(q, k, v, rows, s, True)
    ra, _ = oracle.attn_rows(q, k, np.abs(v), rows, s, True)
    go = o.reshape(bh * w.sq, w.d)[torch.from_numpy(rows)].double().cpu().numpy()
    gl = lse.reshape(-1)[torch.from_numpy(rows)].double().cpu().numpy()
    i = rows % w.sq
    n = np.minimum(i + 1, w.sk)[:, None]
    vmax = np.max(np.abs(v.reshape(bh, w.sk, w.d)), axis=1)[rows // w.sq]
    tol = 2.0 ** -4 * ra + 2.0 ** -18 * n * vmax + 2.0 ** -8 * np.abs(ro) + 1e-6
    err = np.abs(go - ro)
    note(f"   {len(rows)} rows: O worst err/tol {float((err / tol).max()):.3f}; LSE max-abs {float(np.max(np.abs(gl - rl))):.2e}")
    assert np.all(err <= tol)
    assert float(np.max(np.abs(gl - rl))) <= 1e-3


def test_fp8_first_row_selects_first_value():
    """Causal row 0 sees key 0 only: its probability is exactly 2^8 (E4M3
    exact), so O_0 = descale_v v_0 up to the bf16 rounding of O."""
    import torch
    w = W.shape("fp8row0", "bf16", 2, 3, 70, 90, 128, True, seed=3)
    q8, k8, v8, (dq, dk, dv) = W.make_fp8(w)
    o, _ = fa.attention_fp8(q8.cuda(), k8.cuda(), v8.cuda(), causal=True,
                            descale_q=dq, descale_k=dk, descale_v=dv)
    torch.cuda.synchronize()
    ref = dequant(v8, dv)[:, :, 0, :]
    got = o[:, :, 0, :].double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-12)
