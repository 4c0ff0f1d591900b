"""Throughput of the exact-attention prefill forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--split N | --bwd | --fp8 | --varlen N] [--no-cpu-baseline]

One step is one fa_fwd call (the whole hot path: tile schedule, Q/K/V tile
loads, S = QK^T, masking, online softmax, O += PV, epilogue) over the
workload's synthetic inputs, which are resident in HBM before timing starts.
With --split N > 1 a step is one fa_fwd_split call (split-KV forward plus the
merge kernel; the workspace is allocated before timing).  With --bwd a step
is one fa_bwd call (the D = dO.O pass, the dK/dV kernel and the dQ kernel)
on O and LSE that one fa_fwd call produced before timing; its FLOP count is
the usual 2.5x the forward's (five sq x sk x d products where the forward has
two), and the roofline covers the three kernels of the call together.
With --varlen N a step is one fa_fwd_varlen call over N packed sequences of
the workload's head count, head size, dtype and mask, with lengths uniform on
[256, sq] (seeded; queries and keys alike); FLOP and bytes are summed per
sequence with the same conventions.
With --fp8 a step is one fa_fwd_fp8 call on the workload's draws quantized to
OCP E4M3 with per-tensor power-of-two descale factors; its roofline is priced
against the dense FP8 matrix peak and its oracle leg runs on the dequantized
values.
Warm-up runs at least W steps and at least 0.5 s of launches (clocks settle).
Prints ONE JSON line.  ``value`` is TFLOP/s with the usual attention count
4*b*h*sq*sk*d (halved when causal) over the wall-clock of the K timed steps;
``roofline`` prices the kernel's average launch time (HIP events around each
launch, on the stream the kernel runs on) against MI355X's dense bf16/fp16
matrix peak; ``cpu_baseline`` times the fp64 oracle on a bounded sample of
the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

METRIC = "attn fwd TFLOP/s, b4 h32 sq4096 d128 bf16 causal; % of MFMA peak"
METRIC_FP8 = "attn fwd TFLOP/s, b4 h32 sq4096 d128 fp8 e4m3 inputs (bf16 out) causal; % of FP8 MFMA peak"
METRIC_BWD = "attn bwd TFLOP/s (2.5x fwd FLOP count), b4 h32 sq4096 d128 bf16 causal; % of MFMA peak"
# MI355X dense matrix peaks (TFLOP/s): 256 CUs x 2.4 GHz x FLOP/clk/CU
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "fp8_e4m3": 5033.2}
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_86_amd", "csrc", f)
                  for f in ("fa_fwd_kernels.hip", "fa_device.h", "fa_kernels.h", "fa_api.cpp")]


def metric_name(w: W.Workload, args) -> str:
    """The headline metric strings for the headline workload; otherwise the
    same form naming the workload that ran."""
    if getattr(args, "varlen", 0):
        return "attn fwd TFLOP/s, packed variable-length %s h%d d%d %s, %d sequences of %d-%d; %% of MFMA peak" % (
            w.dtype, w.h, w.d, "causal" if w.causal else "non-causal", args.varlen, min(256, w.sq), w.sq)
    if w.name == W.HEADLINE.name:
        return METRIC_BWD if args.bwd else (METRIC_FP8 if args.fp8 else METRIC)
    kind = "bwd" if args.bwd else "fwd"
    extra = " (2.5x fwd FLOP count)" if args.bwd else ""
    inputs = ", fp8 e4m3 inputs" if args.fp8 else ""
    peak = "FP8 MFMA" if args.fp8 else ("fp32 MFMA" if w.dtype == "f32" else "MFMA")
    return "attn %s TFLOP/s%s, %s%s; %% of %s peak" % (kind, extra, w.name, inputs, peak)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def shader_clock(torch_mod, fa_mod, step, stream, n: int = 24, ticks: int = 2000):
    """Shader clock the kernels ran at, in MHz: after the timed region, n more
    steps each followed on the same stream by fa_clock_probe (one wave counts
    shader-clock cycles over `ticks` ticks of the 100 MHz real-time counter).
    The power manager sets the clock on a millisecond scale, so a probe right
    behind a launch sees that launch's clock.  The probe lands on one XCD; the
    rocprofv3 summaries give the all-XCD figure (GRBM_GUI_ACTIVE per XCD over
    the kernel duration)."""
    buf = torch_mod.zeros(2 * n, dtype=torch_mod.int64, device="cuda")
    for i in range(n):
        step()
        rc = fa_mod.lib().fa_clock_probe(buf.data_ptr() + 16 * i, ticks, stream.cuda_stream)
        if rc != fa_mod.FA_OK:
            raise fa_mod.FaError(rc, fa_mod.fa_last_error())
    torch_mod.cuda.synchronize()
    mhz = sorted(c / r * 100.0 for c, r in buf.view(n, 2).cpu().tolist() if r > 0)
    return {"mhz_median": round(mhz[len(mhz) // 2], 1), "mhz_min": round(mhz[0], 1),
            "mhz_max": round(mhz[-1], 1), "samples": len(mhz),
            "source": "fa_clock_probe (s_memtime cycles over s_memrealtime 100 MHz ticks, "
                      "%d us) right behind each of %d launches after the timed region" % (ticks // 100, n)}


# C/C++ string and character literals (kept) or comments (dropped)
_LITERAL_OR_COMMENT = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def source_digest(texts) -> str:
    """sha256[:16] of C/C++ sources with comments removed and whitespace
    collapsed, so that edits to comments or layout do not mark a counter
    record as taken on other code."""
    h = hashlib.sha256()
    for t in texts:
        code = _LITERAL_OR_COMMENT.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), t)
        h.update(" ".join(code.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def kernel_sha() -> str:
    texts = []
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            texts.append(f.read())
    return source_digest(texts)


def traffic_record(w: W.Workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % w.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("traffic_bytes")


def cpu_baseline(w: W.Workload, q, k, v, budget_s: float):
    """Time the fp64 oracle on whole heads of the workload (about budget_s of
    CPU work) and scale to TFLOP/s with the same FLOP convention."""
    import oracle
    nthreads = oracle.default_threads()
    scale = float(np.float32(w.scale))
    q64 = q[0:1, 0:1]
    k64 = k[0:1, 0:1]
    v64 = v[0:1, 0:1]
    head_flops = w.flops / (w.b * w.h)
    t0 = time.perf_counter()
    oracle.attn(q64, k64, v64, scale, w.causal, nthreads=nthreads)
    t1 = time.perf_counter() - t0
    nheads = int(max(1, min(w.b * w.h - 1, budget_s / max(t1, 1e-3))))
    # heads 1..nheads of the flattened [b*h] axis
    qb = q.reshape(1, w.b * w.h, w.sq, w.d)[:, 1:1 + nheads]
    kb = k.reshape(1, w.b * w.h, w.sk, w.d)[:, 1:1 + nheads]
    vb = v.reshape(1, w.b * w.h, w.sk, w.d)[:, 1:1 + nheads]
    t0 = time.perf_counter()
    oracle.attn(qb, kb, vb, scale, w.causal, nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = head_flops * nheads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d of %d heads (full sq=%d x sk=%d each), fp64 C oracle, %.1f s" % (
                nheads, w.b * w.h, w.sq, w.sk, dt)}


def cpu_baseline_varlen(w: W.Workload, lens, q, k, v, budget_s: float):
    """Time the fp64 oracle on whole sequences (all heads) of the packed batch
    q, k, v [1, h, total, d], in order, about budget_s of CPU work, and scale
    to TFLOP/s with the per-sequence FLOP convention."""
    import oracle
    nthreads = oracle.default_threads()
    scale = float(np.float32(w.scale))
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    seq_flops = [4.0 * w.h * n * n * w.d / (2 if w.causal else 1) for n in lens]
    sl = lambda t, i, hs: t[:, hs, offs[i]:offs[i + 1]]
    t0 = time.perf_counter()
    oracle.attn(sl(q, 0, slice(0, 1)), sl(k, 0, slice(0, 1)), sl(v, 0, slice(0, 1)), scale, w.causal,
                nthreads=nthreads)
    rate = seq_flops[0] / w.h / max(time.perf_counter() - t0, 1e-4)
    nseq, planned = 0, 0.0
    while nseq < len(lens) and (nseq == 0 or planned + seq_flops[nseq] <= rate * budget_s):
        planned += seq_flops[nseq]
        nseq += 1
    t0 = time.perf_counter()
    for i in range(nseq):
        oracle.attn(sl(q, i, slice(None)), sl(k, i, slice(None)), sl(v, i, slice(None)), scale, w.causal,
                    nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": planned / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "the first %d of %d sequences (all %d heads, lengths %s), fp64 C oracle, %.1f s" % (
                nseq, len(lens), w.h, ",".join(map(str, lens[:nseq])), dt)}


def cpu_baseline_bwd(w: W.Workload, q, k, v, budget_s: float):
    """Time the oracle's backward on whole heads (about budget_s of CPU work;
    the oracle threads over heads, so at least one head per thread) and scale
    to TFLOP/s with the backward FLOP convention."""
    import oracle
    nthreads = oracle.default_threads()
    scale = float(np.float32(w.scale))
    g = W.make_dout(w)
    head_flops = 2.5 * w.flops / (w.b * w.h)
    t0 = time.perf_counter()
    oracle.attn_bwd(q[0:1, 0:1], k[0:1, 0:1], v[0:1, 0:1], g[0:1, 0:1], scale, w.causal, nthreads=1)
    t1 = time.perf_counter() - t0
    per_round = max(t1, 1e-3)  # one head per thread runs in about t1
    nheads = int(max(1, min(w.b * w.h - 1, nthreads * max(1, int(budget_s / per_round)))))
    sl = lambda t, s: t.reshape(1, w.b * w.h, s, w.d)[:, 1:1 + nheads]
    t0 = time.perf_counter()
    oracle.attn_bwd(sl(q, w.sq), sl(k, w.sk), sl(v, w.sk), sl(g, w.sq), scale, w.causal, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": head_flops * nheads / dt / 1e12, "unit": "TFLOP/s", "cores": min(nthreads, nheads),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "backward of %d of %d heads (full sq=%d x sk=%d each), fp64 C oracle, %.1f s" % (
                nheads, w.b * w.h, w.sq, w.sk, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=W.HEADLINE.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--shape", default=None, metavar="DT,B,H,SQ,SK,D,CAUSAL",
                    help="time an ad-hoc shape instead of a named workload, e.g. bf16,1,36,16384,16384,128,1 "
                         "(N(0,1) inputs, seed 0, scale 1/sqrt(d))")
    ap.add_argument("--split", type=int, default=1, metavar="N",
                    help="split-KV parts per query tile (fa_fwd_split); 1 = fa_fwd")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward (fa_bwd) instead of the forward")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward (fa_fwd_fp8) on E4M3-quantized inputs")
    ap.add_argument("--varlen", type=int, default=0, metavar="N",
                    help="time fa_fwd_varlen on N packed sequences with lengths uniform on [256, sq]")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run a plain device-to-device copy of MIB MiB "
                         "--steps times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the forward pass is sharded over "
              "heads with no exchange, so more GPUs add nothing to measure here; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    w = W.BY_NAME[args.workload]
    if args.shape:
        try:
            dt, b, h, sq, sk, d, causal = args.shape.split(",")
            b, h, sq, sk, d, causal = (int(x) for x in (b, h, sq, sk, d, causal))
            if dt not in W.DTYPES or min(b, h, sq, sk, d) < 1 or causal not in (0, 1):
                raise ValueError(args.shape)
        except ValueError:
            print("--shape wants DT,B,H,SQ,SK,D,CAUSAL with DT in %s" % (W.DTYPES,), file=sys.stderr)
            sys.exit(2)
        w = W.shape("shape_%s_b%dh%ds%dk%dd%d%s" % (dt, b, h, sq, sk, d, "_causal" if causal else ""),
                    dt, b, h, sq, sk, d, bool(causal))
    if args.bwd and args.split > 1:
        print("--bwd and --split are exclusive", file=sys.stderr)
        sys.exit(2)
    if args.fp8 and (args.bwd or args.split > 1 or w.dtype == "f32"):
        print("--fp8 runs the forward of a 16-bit workload only", file=sys.stderr)
        sys.exit(2)
    if args.varlen and (args.bwd or args.fp8 or args.split > 1 or w.dtype == "f32" or args.varlen < 1):
        print("--varlen N (N >= 1) runs the 16-bit forward only", file=sys.stderr)
        sys.exit(2)
    lens = None
    if args.varlen:
        lens = W.varlen_lengths(args.varlen, min(256, w.sq), w.sq, w.seed)
        total = sum(lens)
        packed = W.shape("%s_varlen%d_total%d" % (w.name, args.varlen, total), w.dtype, 1, w.h, total,
                         total, w.d, w.causal, scale=w.scale, seed=w.seed, qk_mult=w.qk_mult, v_dist=w.v_dist)

    import torch
    import exact_attention_86_amd as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}), flush=True)
        return
    log("[bench] generating %s" % (packed.name if lens else w.name))
    q, k, v = W.make(packed if lens else w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    od = torch.empty_like(qd)
    flops = w.flops * (2.5 if args.bwd else 1.0)
    alg_bytes = w.algorithmic_bytes
    if lens:
        # per-sequence conventions: 4 h L^2 d FLOP (halved when causal);
        # Q, K, V, O once and the fp32 LSE
        flops = sum(4.0 * w.h * n * n * w.d for n in lens) / (2 if w.causal else 1)
        alg_bytes = packed.algorithmic_bytes
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    if args.fp8:
        q8, k8, v8, desc = W.make_fp8(w)
        # the oracle leg sees the dequantized values the kernel computes on
        q, k, v = (t.to(torch.float64).numpy() * s for t, s in zip((q8, k8, v8), desc))
        qd, kd, vd = (t.to(dev) for t in (q8, k8, v8))
        od = torch.empty((w.b, w.h, w.sq, w.d), dtype=torch.bfloat16, device=dev)
    lsed = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device=dev)
    scale = float(np.float32(w.scale))
    stream = torch.cuda.current_stream(dev)
    code = W.DTYPE_CODE[w.dtype]
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), od.data_ptr(), lsed.data_ptr())

    if args.bwd:
        rc = fa.fa_fwd(*ptrs, w.b, w.h, w.sq, w.sk, w.d, scale, int(w.causal), code, stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc, fa.fa_last_error())
        gd = W.make_dout(w).to(dev)
        dqd, dkd, dvd = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws_bytes = fa.fa_bwd_workspace_bytes(w.b, w.h, w.sq)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        bptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), od.data_ptr(), gd.data_ptr(),
                 lsed.data_ptr(), dqd.data_ptr(), dkd.data_ptr(), dvd.data_ptr(), ws.data_ptr())

        def step():
            rc = fa.fa_bwd(*bptrs, ws_bytes, w.b, w.h, w.sq, w.sk, w.d, scale, int(w.causal), code,
                           stream.cuda_stream)
            if rc != fa.FA_OK:
                raise fa.FaError(rc, fa.fa_last_error())
    elif args.split > 1:
        ws_bytes = fa.fa_split_workspace_bytes(w.b, w.h, w.sq, w.d, args.split)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def step():
            rc = fa.fa_fwd_split(*ptrs, w.b, w.h, w.sq, w.sk, w.d, scale, int(w.causal), code,
                                 args.split, ws.data_ptr(), ws_bytes, stream.cuda_stream)
            if rc != fa.FA_OK:
                raise fa.FaError(rc, fa.fa_last_error())
    elif lens:
        vptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), od.data_ptr(), lsed.data_ptr(),
                 cu.data_ptr(), cu.data_ptr())

        def step():
            rc = fa.fa_fwd_varlen(*vptrs, len(lens), w.h, total, total, max(lens), w.d, scale,
                                  int(w.causal), code, stream.cuda_stream)
            if rc != fa.FA_OK:
                raise fa.FaError(rc, fa.fa_last_error())
    elif args.fp8:
        def step():
            rc = fa.fa_fwd_fp8(*ptrs, w.b, w.h, w.sq, w.sk, w.d, scale, desc[0], desc[1], desc[2],
                               int(w.causal), stream.cuda_stream)
            if rc != fa.FA_OK:
                raise fa.FaError(rc, fa.fa_last_error())
    else:
        def step():
            rc = fa.fa_fwd(*ptrs, w.b, w.h, w.sq, w.sk, w.d, scale, int(w.causal), code,
                           stream.cuda_stream)
            if rc != fa.FA_OK:
                raise fa.FaError(rc, fa.fa_last_error())

    # untimed warm-up: at least W steps, and at least 0.5 s of launches so the
    # GPU clocks have settled before the timed region
    t_w = time.perf_counter()
    n_w = 0
    while n_w < args.warmup or time.perf_counter() - t_w < 0.5:
        step()
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # per-launch kernel time: HIP events on the launch stream around each call
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = shader_clock(torch, fa, step, stream)
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    avg_ms = sum(per) / len(per)
    med_ms = sorted(per)[len(per) // 2]
    ms_per_step = wall * 1e3 / args.steps

    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    dtype = "fp8_e4m3" if args.fp8 else w.dtype
    peak = PEAK_TFLOPS[dtype]
    log("[bench] shader clock: %s" % sclk)
    log("[bench] %s: wall %.3f ms/step, kernel avg %.3f ms (min %.3f, max %.3f), "
        "%.1f TFLOP/s = %.1f%% of %.1f; %.0f GB/s algorithmic" % (
            packed.name if lens else w.name, ms_per_step, avg_ms, min(per), max(per), achieved,
            100 * achieved / peak, peak, alg_bytes / (avg_ms * 1e-3) / 1e9))

    # the matrix peak scales with the shader clock: % of peak at the clock seen
    frac_sclk = None
    if sclk.get("mhz_median"):
        frac_sclk = round(achieved / (peak * sclk["mhz_median"] / 2400.0), 4)
    kernel = "fa_bwd" if args.bwd else ("fa_fwd_fp8" if args.fp8 else ("fa_fwd_varlen" if lens else
                                         ("fa_fwd" if args.split == 1 else "fa_fwd_split")))
    config = dict(w.describe(), kernel=kernel, nsplit=args.split, parallelism="none (one GPU)")
    if lens:
        config.update(workload=packed.name, b=1, sq=total, sk=total, seq_lens=lens,
                      lens_recipe="uniform integers on [%d, %d], numpy default_rng(%d)" % (
                          min(256, w.sq), w.sq, w.seed))
    out = {
        "metric": metric_name(w, args),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_record(w) if kernel == "fa_fwd" else None},
        "kernel_us": {"mean": round(avg_ms * 1e3, 2), "median": round(med_ms * 1e3, 2),
                      "min": round(min(per) * 1e3, 2), "max": round(max(per) * 1e3, 2),
                      "calls": args.steps, "timed_ms": round(sum(per), 1)},
        "tflops_at_median": round(flops / (med_ms * 1e-3) / 1e12, 3),
        "gbps_algorithmic": round(alg_bytes / (avg_ms * 1e-3) / 1e9, 1),
        "hbm_frac_algorithmic": round(alg_bytes / (avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "sclk": sclk,
        "peak_at_sclk": None if frac_sclk is None else round(peak * sclk["mhz_median"] / 2400.0, 1),
        "frac_at_sclk": frac_sclk,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a sample (~%.0f s)" % args.cpu_budget)
        if args.bwd:
            out["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, args.cpu_budget)
        elif lens:
            out["cpu_baseline"] = cpu_baseline_varlen(w, lens, q, k, v, args.cpu_budget)
        else:
            out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
