"""bench.py's contract checks that need no GPU: the one-GPU rule, option
validation before any device call, the FLOP and byte conventions the
roofline uses, and the gate that drops a stale HBM traffic record."""
import json
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("args", [["--bwd", "--split", "4"], ["--fp8", "--bwd"],
                                  ["--fp8", "--workload", "tiny_fp32_b1h2s128d64"],
                                  ["--shape", "bf16,1,2,3"], ["--shape", "q8,1,1,64,64,128,0"],
                                  ["--shape", "bf16,1,1,64,64,128,2"], ["--varlen", "4", "--bwd"],
                                  ["--varlen", "4", "--fp8"], ["--varlen", "4", "--split", "2"],
                                  ["--varlen", "-1"], ["--varlen", "4", "--workload", "tiny_fp32_b1h2s128d64"]])
def test_exclusive_options_are_refused_before_any_device_call(args):
    r = run_bench(*args)
    assert r.returncode == 2, r.stderr


def test_headline_flop_and_byte_conventions():
    w = W.HEADLINE
    assert (w.b, w.h, w.sq, w.sk, w.d, w.causal, w.dtype) == (4, 32, 4096, 4096, 128, True, "bf16")
    # 4 b h sq sk d, halved for causal
    assert w.flops == 4 * 4 * 32 * 4096 * 4096 * 128 / 2
    # Q, K, V read once, O written once (bf16), LSE written once (fp32)
    assert w.algorithmic_bytes == 2 * 4 * 32 * (2 * 4096 + 2 * 4096) * 128 + 4 * 4 * 32 * 4096


def test_stale_traffic_record_is_dropped(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    w = W.HEADLINE
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % w.name)
    with open(path) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "kernel_sha", lambda: rec["kernel_sha"])
    assert bench.traffic_record(w) == rec["traffic_bytes"]
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 16)
    assert bench.traffic_record(w) is None


def test_source_digest_ignores_comments_and_layout_only():
    sys.path.insert(0, ROOT)
    import bench
    a = 'int f() { // note\n  return 1; /* block\n comment */ }\nconst char* s = "x // y";\n'
    same = 'int f() {\n    return 1;   }\nconst char* s = "x // y";   // trailing\n'
    code = 'int f() { return 2; }\nconst char* s = "x // y";\n'
    literal = 'int f() { return 1; }\nconst char* s = "x // z";\n'
    assert bench.source_digest([a]) == bench.source_digest([same])
    assert bench.source_digest([a]) != bench.source_digest([code])
    assert bench.source_digest([a]) != bench.source_digest([literal])
    assert len(bench.kernel_sha()) == 16


def test_metric_names_the_workload_that_ran():
    sys.path.insert(0, ROOT)
    import argparse
    import bench
    a = argparse.Namespace(bwd=False, fp8=False)
    assert bench.metric_name(W.HEADLINE, a) == bench.METRIC
    assert bench.metric_name(W.HEADLINE, argparse.Namespace(bwd=True, fp8=False)) == bench.METRIC_BWD
    assert bench.metric_name(W.HEADLINE, argparse.Namespace(bwd=False, fp8=True)) == bench.METRIC_FP8
    other = W.BY_NAME["prefill_fp16_b2h8s1024d128"]
    assert other.name in bench.metric_name(other, a)
    v = bench.metric_name(W.HEADLINE, argparse.Namespace(bwd=False, fp8=False, varlen=16))
    assert "variable-length" in v and "16 sequences of 256-4096" in v and v != bench.METRIC


def test_varlen_lengths_are_seeded_and_in_range():
    a = W.varlen_lengths(16, 256, 4096, 3)
    assert a == W.varlen_lengths(16, 256, 4096, 3)
    assert a != W.varlen_lengths(16, 256, 4096, 4)
    assert len(a) == 16 and all(256 <= n <= 4096 for n in a)
    assert W.varlen_lengths(50, 7, 7, 0) == [7] * 50
