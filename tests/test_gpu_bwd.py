"""GPU parity of the backward (fa_bwd) against the fp64 oracle's gradient.

The forward runs on the GPU (fa_fwd), its O and LSE feed fa_bwd, and the
three gradients are compared with oracle.attn_bwd evaluated on the same
seeded inputs (widened exactly to fp64, fp32 scale).  The oracle never sees a
GPU value.

Tolerance: max |GPU - oracle| <= 4u * max(max|oracle|, 0.05) per tensor, u the
unit roundoff of the dtype (2^-8 bf16, 2^-11 fp16).  The GPU rounds each
gradient to the dtype once (u * max), and rounds P and dS to the dtype before
the matrix cores and O before D = dO.O is formed (each a relative error u on
one factor of an fp32-accumulated sum whose terms are bounded by the result's
scale); 4u covers the four.  The floor 0.05 covers gradients that vanish in
exact arithmetic (one key: dQ = dK = 0), where what remains is the fp32
cancellation of O(1) terms summed in another order than the oracle's
(dP_i - D_i with D_i from the stored O).

* small and medium shapes with ragged tiles in both sequence dimensions,
  causal with sq < sk and sq > sk, one row, one key, a negative scale: every
  element compared;
* the headline shape [4, 32, 4096, 128] bf16 causal at full size, compared on
  whole heads (heads are independent, so the oracle runs on a slice);
* bitwise determinism (no atomics).
"""
import sys

import numpy as np
import pytest

import exact_attention_86_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_bwd(q, k, v, g, causal, scale):
    import torch
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(name, got, ref, dtype):
    got = got.double().cpu().numpy()
    assert np.all(np.isfinite(got)), name
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    tol = 4 * UNIT[dtype] * max(m, 0.05)
    note(f"   {name}: max-abs {err:.3e} (max|ref| {m:.3e}, tol {tol:.3e})")
    assert err <= tol, f"{name}: max-abs {err} > {tol}"


CASES = [
    # dtype, b, h, sq, sk, causal, scale (None: 1/sqrt(d))
    ("bf16", 1, 2, 128, 128, False, None),
    ("bf16", 1, 2, 128, 128, True, None),
    ("f16", 2, 3, 200, 328, False, None),
    ("bf16", 1, 2, 300, 300, True, None),
    ("bf16", 1, 2, 100, 257, True, None),
    ("bf16", 1, 2, 333, 150, True, None),
    ("f16", 1, 1, 1, 1, True, None),
    ("f16", 1, 2, 1, 77, False, None),
    ("f16", 1, 2, 77, 1, True, None),
    ("f16", 1, 2, 512, 512, True, None),
    ("bf16", 1, 2, 190, 140, False, -0.07),
    ("f16", 2, 2, 640, 384, False, 0.2),
]


# the same backward kernels with d = 64 (128-byte rows, half the d tiles)
CASES_D64 = [
    ("bf16", 1, 2, 128, 128, True, None, 64),
    ("f16", 2, 3, 200, 328, False, None, 64),
    ("bf16", 1, 3, 333, 150, True, None, 64),
    ("f16", 1, 2, 77, 1, True, None, 64),
    ("bf16", 1, 2, 190, 140, False, -0.07, 64),
    ("f16", 1, 2, 512, 512, True, 0.0, 64),
]


# d = 256: dK and dV accumulated in two halves of d, one wave per SIMD
CASES_D256 = [
    ("bf16", 1, 2, 128, 128, True, None, 256),
    ("f16", 1, 2, 200, 328, False, None, 256),
    ("bf16", 2, 2, 333, 150, True, None, 256),
    ("f16", 1, 1, 1, 77, False, None, 256),
    ("bf16", 1, 2, 190, 140, False, -0.07, 256),
]


@pytest.mark.parametrize("case", CASES + CASES_D64 + CASES_D256, ids=lambda c: "%s_b%dh%d_sq%d_sk%d_%s_%s_d%d" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", c[6], c[7] if len(c) > 7 else 128))
def test_bwd_matches_oracle(case):
    dtype, b, h, sq, sk, causal, scale = case[:7]
    d = case[7] if len(case) > 7 else 128
    w = W.shape("bwd", dtype, b, h, sq, sk, d, causal, scale=scale, seed=17 * sq + sk + d)
    q, k, v = W.make(w)
    g = W.make_dout(w)
    s = float(np.float32(w.scale))
    note(f"[bwd] {dtype} b{b} h{h} sq{sq} sk{sk} d{d} causal={causal} scale={s}")
    dq, dk, dv = gpu_bwd(q, k, v, g, causal, s)
    rq, rk, rv = oracle.attn_bwd(q, k, v, g, s, causal)
    check("dq", dq, rq, dtype)
    check("dk", dk, rk, dtype)
    check("dv", dv, rv, dtype)


def test_bwd_headline_shape_on_whole_heads():
    """Full [4, 32, 4096, 128] bf16 causal problem on the GPU; the oracle
    computes two whole heads (first and last) from sliced inputs."""
    w = W.HEADLINE
    q, k, v = W.make(w)
    g = W.make_dout(w)
    s = float(np.float32(w.scale))
    note(f"[bwd] headline {w.name}")
    dq, dk, dv = gpu_bwd(q, k, v, g, w.causal, s)
    for (bi, hi) in ((0, 0), (w.b - 1, w.h - 1)):
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        rq, rk, rv = oracle.attn_bwd(q[sl], k[sl], v[sl], g[sl], s, w.causal)
        note(f"  head b{bi} h{hi}")
        check("dq", dq[sl], rq, w.dtype)
        check("dk", dk[sl], rk, w.dtype)
        check("dv", dv[sl], rv, w.dtype)


def test_bwd_is_deterministic():
    import torch
    w = W.shape("det", "bf16", 2, 4, 700, 900, 128, True, seed=5)
    q, k, v = (t.cuda() for t in W.make(w))
    g = W.make_dout(w).cuda()
    o, lse = fa.attention(q, k, v, causal=True)
    a = fa.attention_bwd(q, k, v, o, lse, g, causal=True)
    b = fa.attention_bwd(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_workspace_contents_do_not_matter():
    import torch
    w = W.shape("ws", "f16", 1, 3, 257, 300, 128, False, seed=9)
    q, k, v = (t.cuda() for t in W.make(w))
    g = W.make_dout(w).cuda()
    o, lse = fa.attention(q, k, v)
    n = fa.fa_bwd_workspace_bytes(1, 3, 257)
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device="cuda")  # garbage (3.4e38 as fp32)
    a = fa.attention_bwd(q, k, v, o, lse, g, workspace=ws)
    ws.fill_(0)
    b = fa.attention_bwd(q, k, v, o, lse, g, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
