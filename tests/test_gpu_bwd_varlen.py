"""GPU parity of the variable-length backward (fa_bwd_varlen) against the fp64
oracle's gradient, sequence by sequence.

Each sequence is drawn on its own from the seeded generator, the sequences
are packed along the row axis of every head, the forward runs on the GPU
(fa_fwd_varlen) and its O and LSE feed fa_bwd_varlen.  For every sequence
with queries and keys the three gradient slices are compared with
oracle.attn_bwd on that sequence alone (tolerance as in test_gpu_bwd: 4u of
the largest oracle magnitude, floor 0.05), and with fa_bwd run on that
sequence alone from the same O and LSE slices, which must give the same bits
(the same kernels on the same rows, only the offsets differ).  A sequence
without queries must leave dk = dv = 0 on its keys, one without keys dq = 0
on its rows.  The shapes put sequence boundaries inside 128-row tiles, mix
sq > sk and sq < sk under the causal mask, and include single rows and keys.
"""
import math

import numpy as np
import pytest

import exact_attention_86_amd as fa
import oracle
import workloads as W
from tests.test_gpu_bwd import check, note

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, h, d, causal, query lengths, key lengths)
    ("bf16", 2, 128, True, [130, 257, 64], [130, 300, 64]),
    ("bf16", 2, 128, False, [100, 1, 300], [100, 50, 300]),
    ("f16", 3, 64, True, [5, 0, 200], [7, 9, 150]),
    ("f16", 2, 128, True, [77, 200, 1], [1, 333, 129]),
    ("bf16", 1, 64, False, [129, 128, 127, 300], [129, 128, 127, 40]),
    ("bf16", 2, 128, False, [50, 40], [60, 0]),
    ("f16", 2, 256, True, [200, 3, 129], [250, 3, 300]),
]


def packed(case):
    """Packed q, k, v, dout [h, total, d] (CPU) and the offset arrays."""
    import torch
    dt, h, d, causal, qlens, klens = case
    qs, ks, vs, gs = [], [], [], []
    for i, (sq_i, sk_i) in enumerate(zip(qlens, klens)):
        w = W.shape("bwdvl%d" % i, dt, 1, h, max(sq_i, 1), max(sk_i, 1), d, causal,
                    seed=1000 + 100 * i + sq_i + 7 * sk_i)
        q, k, v = W.make(w)
        g = W.make_dout(w)
        qs.append(q[0, :, :sq_i])
        gs.append(g[0, :, :sq_i])
        ks.append(k[0, :, :sk_i])
        vs.append(v[0, :, :sk_i])
    cat = lambda xs: torch.cat(xs, dim=1).contiguous()
    cq = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(klens)]), dtype=torch.int32)
    return cat(qs), cat(ks), cat(vs), cat(gs), cq, ck


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-h%d-d%d-%s-%s-%s" % (
    c[0], c[1], c[2], "causal" if c[3] else "full", "_".join(map(str, c[4])), "_".join(map(str, c[5]))))
def test_bwd_varlen_per_sequence(case):
    import torch
    dt, h, d, causal, qlens, klens = case
    note(f"[bwd-varlen] {case}")
    q, k, v, g, cq, ck = packed(case)
    s = float(np.float32(1.0 / math.sqrt(d)))
    qd, kd, vd, gd, cqd, ckd = (t.cuda() for t in (q, k, v, g, cq, ck))
    o, lse = fa.attention_varlen(qd, kd, vd, cqd, ckd, max(qlens), causal=causal, scale=s)
    for i in range(len(qlens)):
        if klens[i] == 0:  # the forward leaves these rows unwritten
            o[:, int(cq[i]):int(cq[i + 1])] = 0
            lse[:, int(cq[i]):int(cq[i + 1])] = 0
    dq, dk, dv = fa.attention_bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, max(qlens), max(klens),
                                         causal=causal, scale=s)
    torch.cuda.synchronize()
    for i in range(len(qlens)):
        q0, q1, k0, k1 = int(cq[i]), int(cq[i + 1]), int(ck[i]), int(ck[i + 1])
        note(f"  seq {i}: sq={q1 - q0} sk={k1 - k0}")
        if q1 == q0:
            assert not bool(dk[:, k0:k1].any()) and not bool(dv[:, k0:k1].any())
            continue
        if k1 == k0:
            assert not bool(dq[:, q0:q1].any())
            continue
        rq, rk, rv = oracle.attn_bwd(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1],
                                     g[None, :, q0:q1], s, causal)
        check("dq", dq[:, q0:q1], rq[0], dt)
        check("dk", dk[:, k0:k1], rk[0], dt)
        check("dv", dv[:, k0:k1], rv[0], dt)
        # the dense entry point on this sequence alone, from the same O and LSE
        sl_q, sl_k = slice(q0, q1), slice(k0, k1)
        one = lambda t, sl: t[:, sl][None].contiguous()
        eq, ek, ev = fa.attention_bwd(one(qd, sl_q), one(kd, sl_k), one(vd, sl_k), one(o, sl_q),
                                      one(lse, sl_q), one(gd, sl_q), causal=causal, scale=s)
        torch.cuda.synchronize()
        assert torch.equal(eq[0], dq[:, sl_q]) and torch.equal(ek[0], dk[:, sl_k]) and torch.equal(ev[0], dv[:, sl_k])


def test_bwd_varlen_is_deterministic():
    import torch
    case = ("bf16", 4, 128, True, [700, 1, 513, 900], [700, 300, 600, 900])
    q, k, v, g, cq, ck = (t.cuda() for t in packed(case))
    o, lse = fa.attention_varlen(q, k, v, cq, ck, 900, causal=True)
    a = fa.attention_bwd_varlen(q, k, v, o, lse, g, cq, ck, 900, 900, causal=True)
    b = fa.attention_bwd_varlen(q, k, v, o, lse, g, cq, ck, 900, 900, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
