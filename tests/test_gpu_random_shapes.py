"""Seeded random shapes, every element against the fp64 oracle (GPU).

The hand-picked parity cases fix the shapes the kernels were written around;
these draw the problem at random from a fixed seed so that ragged tails in
both sequence dimensions, small and uneven head counts, every head size and
both mask kinds meet every kernel (the 4-wave and 8-wave forwards, fp32, the
backward).  Each case prints its parameters before it runs.  Tolerances are
the ones the other parity tests use: O and LSE as test_gpu_parity, the
gradients as test_gpu_bwd.
"""
import math
import sys

import numpy as np
import pytest

import exact_attention_86_amd as fa
import oracle
import workloads as W
from tests.test_gpu_bwd import check
from tests.test_gpu_parity import TOL_LSE, TOL_O, scale32

pytestmark = pytest.mark.gpu


def draw_cases(seed, n, with_f32):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = rng.choice(["f16", "bf16", "f32"] if with_f32 else ["f16", "bf16"])
        d = int(rng.choice([64, 128] if dt == "f32" else [64, 128, 256]))
        b = int(rng.integers(1, 3))
        h = int(rng.integers(1, 5))
        sq = int(rng.integers(1, 700))
        sk = int(rng.integers(1, 700))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.choice([1.0 / math.sqrt(d), 0.3, -0.05]))
        cases.append((str(dt), b, h, sq, sk, d, causal, scale, 7000 + i))
    return cases


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw_many_heads(seed, n):
    """Shapes with enough work items for the 8-wave ping-pong kernel (per-item
    or persistent grid): d = 128, 16-bit, 256-320 heads."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = str(rng.choice(["f16", "bf16"]))
        sq = int(rng.integers(200, 700))
        sk = int(rng.integers(1, 700))
        cases.append((dt, 1, int(rng.integers(256, 321)), sq, sk, 128, bool(rng.integers(0, 2)),
                      float(rng.choice([1.0 / math.sqrt(128), 0.3, -0.05])), 7500 + i))
    return cases


FWD = draw_cases(11, 16, True) + draw_many_heads(13, 6)
BWD = draw_cases(12, 10, False)
ids = lambda c: "%s-b%dh%d-sq%d-sk%d-d%d-%s" % (c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full")


@pytest.mark.parametrize("case", FWD, ids=ids)
def test_random_forward(case):
    import torch
    dt, b, h, sq, sk, d, causal, scale, seed = case
    note(f"[random-fwd] {case}")
    w = W.shape("rnd", dt, b, h, sq, sk, d, causal, scale=scale, seed=seed)
    q, k, v = W.make(w)
    s = scale32(w.scale)
    if dt != "f32":
        note(f"   kernel waves {fa.fa_query_config(W.DTYPE_CODE[dt], d, int(causal), b, h, sq, sk)['waves']}")
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=s)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(q, k, v, s, causal)
    eo = float(np.max(np.abs(o.double().cpu().numpy() - ro)))
    el = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    note(f"   O max-abs {eo:.3e}, LSE max-abs {el:.3e}")
    assert eo <= TOL_O[dt] and el <= TOL_LSE


@pytest.mark.parametrize("case", BWD, ids=ids)
def test_random_backward(case):
    import torch
    dt, b, h, sq, sk, d, causal, scale, seed = case
    note(f"[random-bwd] {case}")
    w = W.shape("rndb", dt, b, h, sq, sk, d, causal, scale=scale, seed=seed)
    q, k, v = W.make(w)
    g = W.make_dout(w)
    s = float(np.float32(w.scale))
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=s)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, gd, causal=causal, scale=s)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, g, s, causal)
    check("dq", dq, rq, dt)
    check("dk", dk, rk, dt)
    check("dv", dv, rv, dt)
