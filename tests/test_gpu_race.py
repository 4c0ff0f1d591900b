"""Race guards on the debug build libfa_poison.so (GPU).

In that build every global->LDS copy first sets its destination bytes to NaN.
A wave that read an LDS stage before the copies meant for it had landed, or a
copy that overwrote a stage another wave was still reading, would then put NaN
into O, LSE or the gradients instead of stale but finite numbers that a loose
tolerance might let through.  Each case runs through the poisoned build and is
compared with the fp64 oracle element by element, exactly as in the parity
tests.  The shapes cover every kernel that copies into LDS: the 8-wave
ping-pong forward (per-item and persistent grids, causal, ragged, sq != sk),
the 4-wave forward (d = 64, 128, 256) and its two-key-group form, split-KV, variable-length sequences,
the backward (dense and variable-length) and the FP8 forward.  The number of waves per workgroup is varied
by the shapes themselves (4 and 8 waves run the same tiles), and
test_gpu_parity compares the two bit for bit on shared rows.
"""
import math

import numpy as np
import pytest

import exact_attention_86_amd as fa
import workloads as W
from tests import test_gpu_bwd as B
from tests import test_gpu_bwd_varlen as BV
from tests import test_gpu_fp8 as F8
from tests import test_gpu_parity as P

pytestmark = pytest.mark.gpu

FWD = [
    # dtype, b, h, sq, sk, d, causal, expected waves, persistent
    ("bf16", 1, 256, 512, 512, 128, True, 8, False),
    ("bf16", 1, 256, 300, 520, 128, False, 8, False),
    ("f16", 1, 256, 1000, 333, 128, True, 8, False),
    ("bf16", 1, 320, 512, 512, 128, True, 8, True),
    ("f16", 2, 8, 1024, 1024, 128, False, 8, False),      # 4 waves x 2 key groups
    ("bf16", 1, 3, 333, 700, 64, True, 8, False),         # 4 waves x 2 key groups
    ("bf16", 1, 64, 777, 777, 128, True, 4, False),       # 4 waves
    ("bf16", 2, 2, 250, 250, 256, False, 4, False),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "%s-b%dh%d-sq%d-sk%d-d%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_poisoned_forward(case, gpu):
    dt, b, h, sq, sk, d, causal, waves, persistent = case
    w = W.shape("race", dt, b, h, sq, sk, d, causal, seed=sq + sk + d)
    code = W.DTYPE_CODE[dt]
    assert fa.fa_query_config(code, d, int(causal), b, h, sq, sk)["waves"] == waves
    assert fa.fa_query_launch(code, d, int(causal), b, h, sq, sk)["persistent"] == persistent
    with fa.poisoned():
        P.compare_full(w)


def test_poisoned_split_kv(gpu):
    w = W.shape("race-split", "bf16", 1, 4, 64, 4096, 128, False, seed=11)
    with fa.poisoned():
        P.compare_full(w, nsplit=8)


def test_poisoned_varlen(gpu):
    with fa.poisoned():
        P.test_varlen_per_sequence_compare(("bf16", 2, 128, True, (300, 17, 130), (300, 40, 129)), gpu)
        P.test_varlen_per_sequence_compare(("bf16", 2, 128, True, (700, 1, 1500), (900, 300, 1500)), gpu)
        P.test_varlen_per_sequence_compare(("bf16", 32, 128, True, (700, 1, 1500, 2048, 300, 4000),
                                            (900, 300, 1500, 2048, 300, 3000)), gpu)


def test_poisoned_backward(gpu):
    with fa.poisoned():
        B.test_bwd_matches_oracle(("bf16", 1, 2, 300, 300, True, None))
        B.test_bwd_matches_oracle(("f16", 2, 2, 640, 384, False, 0.2))
        B.test_bwd_matches_oracle(("bf16", 1, 2, 300, 300, True, None, 64))
        B.test_bwd_matches_oracle(("f16", 1, 2, 300, 260, True, None, 256))


def test_poisoned_backward_varlen(gpu):
    with fa.poisoned():
        BV.test_bwd_varlen_per_sequence(("bf16", 2, 128, True, [130, 257, 64], [130, 300, 64]))


def test_poisoned_fp8(gpu):
    with fa.poisoned():
        F8.check_fp8(W.shape("race-fp8", "bf16", 1, 300, 333, 700, 128, True, seed=5))
