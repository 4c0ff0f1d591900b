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


def draw_packed(seed, n):
    """Packed batches that take the ping-pong kernel's variable-length form:
    d = 128, h a multiple of 8, 2-64 sequences averaging at least 1024 query
    rows, enough 256-row tiles for a work item per CU.  Query and key lengths
    are drawn apart (sq < sk and sq > sk, equal lengths, so equal costs,
    single rows, and sequences without queries or keys)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dt = str(rng.choice(["f16", "bf16"]))
        h = int(rng.choice([8, 16, 32]))
        nb = int(rng.integers(2, 65))
        causal = bool(rng.integers(0, 2))
        base = int(rng.integers(1024, 2600))
        ql = [int(x) for x in rng.integers(1, 2 * base, nb)]
        kl = [int(x) if rng.random() < 0.6 else ql[i] for i, x in enumerate(rng.integers(1, 2 * base, nb))]
        if nb > 3:
            ql[1] = ql[2]  # a tie in the cost ranking
            kl[1] = kl[2]
            ql[3], kl[0] = 0, 0  # no queries; no keys
        tq = sum(ql)
        work = sum(h * a * b * 128 * 4 for a, b in zip(ql, kl))
        if tq < 1024 * nb or h * (tq // 256) // (2 if causal else 1) < 256 or work > 4e11:
            continue
        cases.append((dt, h, causal, ql, kl, 8100 + len(cases)))
    return cases


FWD = draw_cases(11, 16, True) + draw_many_heads(13, 6)
PACKED = draw_packed(14, 6)
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


@pytest.mark.parametrize("case", PACKED, ids=lambda c: "%s-h%d-%s-%dseqs" % (c[0], c[1], "causal" if c[2] else "full", len(c[3])))
def test_random_packed_forward(case):
    """Every sequence of a random packed batch against the oracle on that
    sequence alone (the rows of a sequence without keys are not written)."""
    import torch
    dt, h, causal, ql, kl, seed = case
    note(f"[random-packed] {dt} h{h} causal={causal} q={ql} k={kl}")
    qs, ks, vs = [], [], []
    for i, (a, b) in enumerate(zip(ql, kl)):
        w = W.shape("rndp%d" % i, dt, 1, h, max(a, 1), max(b, 1), 128, causal, seed=seed * 100 + i)
        q, k, v = W.make(w)
        qs.append(q[0, :, :a])
        ks.append(k[0, :, :b])
        vs.append(v[0, :, :b])
    cat = lambda xs: torch.cat(xs, dim=1).contiguous()
    qp, kp, vp = cat(qs), cat(ks), cat(vs)
    cq = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(kl)]).astype(np.int32)
    s = scale32(1.0 / math.sqrt(128))
    o, lse = fa.attention_varlen(qp.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(cq).cuda(),
                                 torch.from_numpy(ck).cuda(), max(ql), causal=causal, scale=s)
    torch.cuda.synchronize()
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    worst_o = worst_l = 0.0
    for i in range(len(ql)):
        if ql[i] == 0 or kl[i] == 0:
            continue
        q0, q1, k0, k1 = cq[i], cq[i + 1], ck[i], ck[i + 1]
        ro, rl = oracle.attn(qp[None, :, q0:q1], kp[None, :, k0:k1], vp[None, :, k0:k1], s, causal)
        worst_o = max(worst_o, float(np.max(np.abs(go[:, q0:q1] - ro[0]))))
        worst_l = max(worst_l, float(np.max(np.abs(gl[:, q0:q1] - rl[0]))))
    note(f"   O max-abs {worst_o:.3e}, LSE max-abs {worst_l:.3e}")
    assert worst_o <= TOL_O[dt] and worst_l <= TOL_LSE
