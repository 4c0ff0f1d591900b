"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (max-abs over every compared element): O within 1e-5 (fp32),
4e-3 (fp16), 2e-2 (bf16); LSE within 1e-3.  Both sides read the same seeded
inputs (``workloads``), the oracle widening the stored fp32/fp16/bf16 values
exactly to fp64, and both use the fp32 value of the scale.

* the five benchmark workloads run at full size, in the launch configuration
  the benchmark times, and are compared element by element over the whole
  output (every O element and every LSE row of every head);
* small and medium shapes span several tiles in both sequence dimensions
  with ragged tails, compared the same way;
* sampled rows of the large workloads (first and last query tiles, tile
  boundaries, the causal diagonal) as an extra, and invariants that hold at
  any size (constant V, one-hot selection, causal row 0, convex-combination
  bound, bitwise determinism of the 4-wave and the 8-wave kernel, and the
  8-wave kernel bit-for-bit equal to the 4-wave kernel on the same rows).
"""
import math
import sys

import numpy as np
import pytest

import exact_attention_86_amd as fa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "f16": 4e-3, "bf16": 2e-2}
TOL_LSE = 1e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def scale32(scale):
    return float(np.float32(scale))


def run_gpu(q, k, v, causal, scale, nsplit=1):
    import torch
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale, nsplit=nsplit)
    torch.cuda.synchronize()
    return o, lse


def compare_full(w: W.Workload, seed=None, nsplit=1):
    q, k, v = W.make(w, seed)
    s = scale32(w.scale)
    note(f"[parity] {w.name} b{w.b} h{w.h} sq{w.sq} sk{w.sk} d{w.d} {w.dtype} causal={w.causal} nsplit={nsplit}")
    o, lse = run_gpu(q, k, v, w.causal, s, nsplit)
    ro, rl = oracle.attn(q, k, v, s, w.causal)
    go = o.double().cpu().numpy()
    gl = lse.double().cpu().numpy()
    eo = float(np.max(np.abs(go - ro)))
    el = float(np.max(np.abs(gl - rl)))
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert eo <= TOL_O[w.dtype], f"O max-abs {eo} > {TOL_O[w.dtype]}"
    assert el <= TOL_LSE, f"LSE max-abs {el}"
    return eo, el


def sample_rows(w: W.Workload, block_m: int, seed=0, heads=4, random_rows=48):
    """Flat row indices: every row of the first and last query tiles of a few
    heads, tile-boundary rows, and random rows."""
    rng = np.random.default_rng(1000 + seed)
    bh = w.b * w.h
    hs = sorted(set([0, bh - 1] + list(rng.integers(0, bh, max(heads - 2, 0)))))
    rows = set()
    for hh in hs:
        base = hh * w.sq
        first = range(0, min(block_m, w.sq))
        last_start = ((w.sq - 1) // block_m) * block_m
        last = range(last_start, w.sq)
        for i in list(first) + list(last):
            rows.add(base + i)
        for t in range(block_m, w.sq, block_m):
            for i in (t - 1, t, t + 1):
                if 0 <= i < w.sq:
                    rows.add(base + i)
        for i in rng.integers(0, w.sq, random_rows):
            rows.add(base + int(i))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("idx", range(len(W.WORKLOADS)), ids=[w.name for w in W.WORKLOADS])
def test_workload_full_compare(idx, gpu):
    """Every element of O and LSE of each benchmark workload at full size."""
    w = W.WORKLOADS[idx]
    cfg = fa.fa_query_config(W.DTYPE_CODE[w.dtype], w.d, int(w.causal), w.b, w.h, w.sq, w.sk)
    note(f"  kernel tiling {cfg}")
    eo, el = compare_full(w)
    note(f"  O max-abs={eo:.3e} LSE max-abs={el:.3e}")


@pytest.mark.slow
@pytest.mark.parametrize("idx", [2, 3, 4])
def test_workload_full_size_sampled_rows(idx, gpu):
    import torch
    w = W.WORKLOADS[idx]
    note(f"[parity-sampled] {w.name}")
    q, k, v = W.make(w)
    s = scale32(w.scale)
    o, lse = run_gpu(q, k, v, w.causal, s)
    cfg = fa.fa_query_config(W.DTYPE_CODE[w.dtype], w.d, int(w.causal), w.b, w.h, w.sq, w.sk)
    rows = sample_rows(w, cfg["block_m"], seed=idx)
    ro, rl = oracle.attn_rows(q, k, v, rows, s, w.causal)
    go = o.reshape(-1, w.d)[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    gl = lse.reshape(-1)[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    eo = float(np.max(np.abs(go - ro)))
    el = float(np.max(np.abs(gl - rl)))
    note(f"  rows={rows.size} O max-abs={eo:.3e} LSE max-abs={el:.3e}")
    assert eo <= TOL_O[w.dtype] and el <= TOL_LSE
    # properties over the whole output: finite, and each O row a convex
    # combination of V rows (bounded by max |V| up to output rounding)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    vmax = float(v.abs().max())
    assert float(o.abs().max()) <= vmax * (1 + 2 ** -7)
    if w.causal:
        # row 0 of every head attends to key 0 alone: O = V[0] exactly
        assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


SMALL = [
    # (dtype, b, h, sq, sk, d, causal)
    ("bf16", 1, 2, 200, 200, 128, False),
    ("bf16", 1, 2, 200, 200, 128, True),
    ("f16", 2, 1, 129, 257, 128, False),
    ("f16", 1, 3, 257, 129, 128, True),
    ("bf16", 1, 1, 1, 1, 128, False),
    ("bf16", 1, 1, 1, 300, 128, True),
    ("bf16", 1, 1, 300, 1, 128, True),
    ("bf16", 2, 2, 65, 63, 64, False),
    ("f16", 1, 2, 130, 190, 64, True),
    ("bf16", 1, 2, 150, 97, 256, False),
    ("f16", 1, 1, 33, 300, 256, True),
    ("f32", 1, 2, 100, 77, 64, False),
    ("f32", 1, 2, 129, 129, 64, True),
    ("f32", 1, 1, 70, 200, 128, True),
    ("f32", 2, 1, 33, 65, 128, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s-b%dh%d-sq%d-sk%d-d%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_small_shapes_full_compare(case, gpu):
    dt, b, h, sq, sk, d, causal = case
    compare_full(W.shape("small", dt, b, h, sq, sk, d, causal, seed=sq * 7 + sk))


# many heads with short sequences: enough work items for the 8-wave ping-pong
# kernel (d = 128), compared over the whole output, ragged and causal
PINGPONG = [
    ("bf16", 1, 256, 300, 300, 128, True),
    ("f16", 2, 128, 260, 260, 128, False),
    ("bf16", 1, 256, 200, 333, 128, True),
    ("bf16", 1, 256, 333, 200, 128, True),   # causal sq > sk: rows past sk see every key
    ("f16", 1, 512, 520, 130, 128, True),
]


@pytest.mark.parametrize("case", PINGPONG, ids=lambda c: "%s-b%dh%d-sq%d-sk%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[6] else "full"))
def test_pingpong_shapes_full_compare(case, gpu):
    dt, b, h, sq, sk, d, causal = case
    cfg = fa.fa_query_config(W.DTYPE_CODE[dt], d, int(causal), b, h, sq, sk)
    assert cfg["waves"] == 8
    compare_full(W.shape("pp", dt, b, h, sq, sk, d, causal, seed=sq + sk))


# causal problems whose pairs of query tiles would leave the last round of
# workgroups mostly empty run the 8-wave kernel on the persistent grid
PERSISTENT = [
    ("bf16", 1, 300, 1000, 1000, True),     # 600 pairs on 256 CUs
    ("f16", 1, 260, 700, 650, True),        # causal sq > sk, ragged
    ("bf16", 2, 150, 1300, 1300, True),     # ragged last tile
]


@pytest.mark.parametrize("case", PERSISTENT, ids=lambda c: "%s-b%dh%d-sq%d-sk%d" % c[:5])
def test_persistent_schedule_full_compare(case, gpu):
    dt, b, h, sq, sk, causal = case
    launch = fa.fa_query_launch(W.DTYPE_CODE[dt], 128, int(causal), b, h, sq, sk)
    note(f"  launch {launch}")
    assert launch["persistent"] and launch["grid"] % 8 == 0
    compare_full(W.shape("persist", dt, b, h, sq, sk, 128, causal, seed=sq + 2 * sk))


def test_benchmark_shapes_use_the_per_item_grid(gpu):
    """The rule keeps the head-major per-item grid where pairs fill whole
    rounds (the headline and the 16k workloads)."""
    for w in (W.WORKLOADS[2], W.WORKLOADS[3]):
        launch = fa.fa_query_launch(W.DTYPE_CODE[w.dtype], w.d, int(w.causal), w.b, w.h, w.sq, w.sk)
        assert not launch["persistent"], (w.name, launch)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5])
def test_unusual_scales(scale, gpu):
    compare_full(W.shape("scale", "bf16", 1, 2, 100, 130, 128, True, scale=scale, seed=3))
    compare_full(W.shape("scale32", "f32", 1, 1, 50, 70, 64, False, scale=scale, seed=4))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_constant_v_and_one_hot(dt, gpu):
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    d, sk, sq = 64, 64, 96
    rng = np.random.default_rng(5)
    # constant V: O = c exactly representable
    q = torch.from_numpy(rng.standard_normal((1, 2, sq, d)).astype(np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((1, 2, sk, d)).astype(np.float32)).to(tdt)
    v = torch.full((1, 2, sk, d), 0.375, dtype=tdt)
    o, _ = run_gpu(q, k, v, True, 0.125)
    assert float((o.float().cpu() - 0.375).abs().max()) <= TOL_O[dt]
    # one-hot: K_j = 32 e_j, Q_i = e_{pi(i)}, scale 2 -> scores 64 vs 0
    perm = rng.integers(0, sk, sq)
    qn = np.zeros((1, 1, sq, d), np.float32)
    qn[0, 0, np.arange(sq), perm] = 1.0
    kn = np.zeros((1, 1, sk, d), np.float32)
    kn[0, 0, np.arange(sk), np.arange(sk)] = 32.0
    vn = rng.standard_normal((1, 1, sk, d)).astype(np.float32)
    q, k, v = (torch.from_numpy(x).to(tdt) for x in (qn, kn, vn))
    o, lse = run_gpu(q, k, v, False, 2.0)
    ref = v[0, 0, perm].float()
    assert float((o[0, 0].float().cpu() - ref).abs().max()) <= TOL_O[dt]
    assert float((lse.cpu() - 64.0).abs().max()) <= TOL_LSE


@pytest.mark.parametrize("dt,d,sk", [("f16", 64, 64), ("f16", 128, 200), ("f16", 256, 100), ("bf16", 128, 300)])
def test_one_hot_wide_score_range(dt, d, sk, gpu):
    """Scores 64 (selected keys) vs 0 (others), scale 2: the row max lives in
    one of the two lane halves that share a query, so a max exchange that
    drops one half pushes fp16 probabilities past the fp16 range.  With
    sk > d several keys share a column and O is the mean of their V rows."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    sq = 130
    rng = np.random.default_rng(6)
    col = rng.integers(0, min(sk, d), sq)
    qn = np.zeros((1, 1, sq, d), np.float32)
    qn[0, 0, np.arange(sq), col] = 1.0
    kn = np.zeros((1, 1, sk, d), np.float32)
    kn[0, 0, np.arange(sk), np.arange(sk) % d] = 32.0
    vn = rng.standard_normal((1, 1, sk, d)).astype(np.float32)
    q, k, v = (torch.from_numpy(x).to(tdt) for x in (qn, kn, vn))
    o, lse = run_gpu(q, k, v, False, 2.0)
    vr = v[0, 0].double().numpy()
    ref = np.stack([vr[(np.arange(sk) % d) == col[i]].mean(0) for i in range(sq)])
    cnt = np.array([np.sum((np.arange(sk) % d) == col[i]) for i in range(sq)])
    assert float(np.abs(o[0, 0].double().cpu().numpy() - ref).max()) <= TOL_O[dt]
    assert float(np.abs(lse[0, 0].double().cpu().numpy() - (64.0 + np.log(cnt))).max()) <= TOL_LSE


@pytest.mark.parametrize("b,h,sq,waves,block_m", [(1, 64, 777, 4, 128), (2, 4, 777, 8, 128), (1, 256, 4096, 8, 256),
                                                 (1, 300, 1000, 8, 256)])
def test_deterministic(b, h, sq, waves, block_m, gpu):
    """Two runs give the same bits, for the 4-wave kernel, for it with two key
    groups (merged in a fixed order), and for the 8-wave ping-pong kernel
    (which has no barrier between the two slots of a key window, so a race on
    an LDS stage would show up as run-to-run noise), on its per-item and on its
    persistent grid."""
    import torch
    cfg = fa.fa_query_config(W.DTYPE_CODE["bf16"], 128, 1, b, h, sq, sq)
    assert (cfg["waves"], cfg["block_m"]) == (waves, block_m)
    w = W.shape("det", "bf16", b, h, sq, sq, 128, True, seed=9)
    q, k, v = (t.cuda() for t in W.make(w))
    o1, l1 = fa.attention(q, k, v, causal=True)
    o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def four_wave_head_chunk(h, sq, sk, causal):
    """Heads per fa_fwd_varlen call (a divisor of h) for which a one-sequence
    call keeps the plain 4-wave kernel: fewer than 1024 rows, a head count
    that is not a multiple of 8, or fewer than 256 ping-pong items (h * floor(sq / 256), halved when causal) and, unless
    the keys span fewer than 4 tiles of 64, at least 256 row tiles
    (h * (ceil(sq / 128) + 1)), so that neither the ping-pong kernel nor two
    key groups are chosen."""
    def plain(c):
        pp = sq >= 1024 and c % 8 == 0 and c * (sq // 256) // (2 if causal else 1) >= 256
        kg = c * (-(-sq // 128) + 1) < 256 and sk >= 4 * 64
        return not pp and not kg
    return max(c for c in range(1, h + 1) if h % c == 0 and plain(c))


@pytest.mark.parametrize("dt,h,sq,sk,causal", [("bf16", 256, 4096, 4096, True), ("f16", 256, 333, 200, True),
                                              ("bf16", 300, 260, 390, False), ("bf16", 300, 1000, 1000, True)])
def test_eight_waves_equal_four_waves(dt, h, sq, sk, causal, gpu):
    """The same problem through the 8-wave ping-pong kernel (fa_fwd on many
    heads) and through the 4-wave kernel (fa_fwd_varlen with one sequence, on
    head chunks small enough to keep that kernel) gives the same bits: both
    run each 32-row query block through the same instruction sequence per
    64-key tile, in ascending key order, so any difference means a stage was
    read before its copy landed or after it was overwritten.  On the per-item
    causal grid the ping-pong kernel walks the light tile of each pair (query
    tiles below nQ/2, 256 rows each) in descending key order: those rows are
    the same sums in another order and are held to the oracle's tolerance
    instead."""
    import torch
    cfg = fa.fa_query_config(W.DTYPE_CODE[dt], 128, int(causal), 1, h, sq, sk)
    assert (cfg["waves"], cfg["block_m"]) == (8, 256)
    launch = fa.fa_query_launch(W.DTYPE_CODE[dt], 128, int(causal), 1, h, sq, sk)
    w = W.shape("waves", dt, 1, h, sq, sk, 128, causal, seed=sq + sk)
    q, k, v = (t.cuda() for t in W.make(w))
    s = scale32(w.scale)
    o8, l8 = fa.attention(q, k, v, causal=causal, scale=s)
    cu_q = torch.tensor([0, sq], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, sk], dtype=torch.int32, device="cuda")
    hc = four_wave_head_chunk(h, sq, sk, causal)
    note(f"[eight-vs-four] {dt} h{h} sq{sq} sk{sk} causal={causal}: 4-wave on chunks of {hc} heads")
    parts = [fa.attention_varlen(q[0, i:i + hc].contiguous(), k[0, i:i + hc].contiguous(),
                                 v[0, i:i + hc].contiguous(), cu_q, cu_k, sq, causal=causal, scale=s)
             for i in range(0, h, hc)]
    o4 = torch.cat([x[0] for x in parts])
    l4 = torch.cat([x[1] for x in parts])
    torch.cuda.synchronize()
    n_mt = -(-sq // cfg["block_m"])
    desc = min(sq, (n_mt // 2) * cfg["block_m"]) if causal and not launch["persistent"] else 0
    assert torch.equal(o8[0][:, desc:], o4[:, desc:]) and torch.equal(l8[0][:, desc:], l4[:, desc:])
    if desc:
        do = float((o8[0][:, :desc].float() - o4[:, :desc].float()).abs().max())
        dl = float((l8[0][:, :desc] - l4[:, :desc]).abs().max())
        assert do <= TOL_O[dt] and dl <= TOL_LSE, (do, dl)


def test_stream_argument(gpu):
    import torch
    w = W.shape("stream", "f16", 1, 2, 256, 256, 128, False, seed=10)
    q, k, v = (t.cuda() for t in W.make(w))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, stream=s)
    s.synchronize()
    o2, l2 = fa.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


# ---- split-KV forward (fa_fwd_split): same result as the definition ----
SPLIT = [
    # (dtype, b, h, sq, sk, d, causal, nsplit)
    ("f16", 2, 8, 1024, 1024, 128, False, 4),    # the fp16 prefill workload's shape
    ("bf16", 1, 2, 300, 300, 128, True, 3),
    ("bf16", 2, 4, 16, 4000, 128, False, 8),     # decode-shaped: sq << sk
    ("f16", 1, 2, 5, 2049, 64, True, 16),        # causal sq < sk: most parts see no key
    ("bf16", 1, 2, 130, 100, 256, False, 8),     # more parts than key tiles
    ("f16", 1, 3, 257, 129, 64, True, 2),
    ("bf16", 1, 1, 1, 1, 128, False, 2),
    ("f16", 1, 2, 200, 3000, 256, False, 64),
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: "%s-b%dh%d-sq%d-sk%d-d%d-%s-split%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full", c[7]))
def test_split_kv_full_compare(case, gpu):
    dt, b, h, sq, sk, d, causal, nsplit = case
    compare_full(W.shape("split", dt, b, h, sq, sk, d, causal, seed=sq + 3 * sk), nsplit=nsplit)


@pytest.mark.parametrize("nsplit", [1, 64])
def test_million_keys(nsplit, gpu):
    """16 queries against 2^20 keys: the row sum and O accumulate in fp32
    over 16384 key tiles (one workgroup per head without splitting)."""
    compare_full(W.shape("longkeys", "bf16", 1, 2, 16, 1 << 20, 128, False, seed=11), nsplit=nsplit)


def test_split_one_part_is_fa_fwd(gpu):
    import torch
    w = W.shape("split1", "bf16", 1, 2, 200, 333, 128, True, seed=11)
    q, k, v = (t.cuda() for t in W.make(w))
    o1, l1 = fa.attention(q, k, v, causal=True, scale=scale32(w.scale))
    o2, l2 = fa.attention(q, k, v, causal=True, scale=scale32(w.scale), nsplit=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_workspace_contents_do_not_matter(gpu):
    import torch
    w = W.shape("splitws", "f16", 1, 2, 100, 700, 128, False, seed=12)
    q, k, v = (t.cuda() for t in W.make(w))
    need = fa.fa_split_workspace_bytes(1, 2, 100, 128, 5)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for fill in (0xFF, 0x00):  # 0xFF bytes read as fp32 NaN
        ws.fill_(fill)
        outs.append(fa.attention(q, k, v, scale=scale32(w.scale), nsplit=5, workspace=ws))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert bool(torch.isfinite(outs[0][0]).all())


# ---- variable-length packed sequences (fa_fwd_varlen) ----
VARLEN = [
    # (dtype, h, d, causal, query lengths, key lengths)
    ("bf16", 2, 128, False, [100, 1, 300], [100, 50, 300]),
    ("bf16", 2, 128, True, [130, 257, 64], [130, 300, 64]),
    ("f16", 3, 64, True, [5, 0, 200], [7, 9, 150]),
    ("f16", 1, 256, False, [33, 129], [300, 1]),
    # long keys, few tiles: two key groups per tile (8 waves)
    ("bf16", 2, 128, True, [700, 1, 1500], [900, 300, 1500]),
    ("f16", 2, 64, False, [333, 1000], [1200, 2000]),
    # d = 128, h a multiple of 8, sequences of 1024 rows or more on average and
    # a ping-pong work item per CU: the 8-wave ping-pong kernel, one item per (head, sequence,
    # causal pair); sq > sk and sq < sk, a single row, a sequence shorter than
    # one 256-row tile
    ("bf16", 32, 128, True, [700, 1, 1500, 2048, 300, 4000], [900, 300, 1500, 2048, 300, 3000]),
    ("f16", 16, 128, False, [1000, 2500, 1500, 129, 1, 1500], [1000, 2600, 1500, 1, 77, 1500]),
    # 64 sequences: the ping-pong kernel's limit (one lane per sequence when it
    # ranks them by cost); 65: the 4-wave kernel
    ("bf16", 8, 128, False, [1000 + 13 * i for i in range(64)], [1000 + 13 * i for i in range(64)]),
    ("f16", 8, 128, True, [1000 + 9 * i for i in range(65)], [1000 + 9 * i for i in range(65)]),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "%s-h%d-d%d-%s-%s" % (
    c[0], c[1], c[2], "causal" if c[3] else "full",
    "_".join(map(str, c[4])) if len(c[4]) <= 8 else "%dseqs" % len(c[4])))
def test_varlen_per_sequence_compare(case, gpu):
    import torch
    dt, h, d, causal, qlens, klens = case
    note(f"[parity-varlen] {case}")
    qs, ks, vs = [], [], []
    for i, (sq_i, sk_i) in enumerate(zip(qlens, klens)):
        w = W.shape("varlen%d" % i, dt, 1, h, max(sq_i, 1), sk_i, d, causal, seed=100 * i + sq_i + sk_i)
        q, k, v = W.make(w)
        qs.append(q[:, :, :sq_i])
        ks.append(k)
        vs.append(v)
    qp = torch.cat(qs, dim=2)[0].contiguous()
    kp = torch.cat(ks, dim=2)[0].contiguous()
    vp = torch.cat(vs, dim=2)[0].contiguous()
    cq = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(klens)]), dtype=torch.int32)
    s = scale32(1.0 / math.sqrt(d))
    o, lse = fa.attention_varlen(qp.cuda(), kp.cuda(), vp.cuda(), cq.cuda(), ck.cuda(), max(qlens),
                                 causal=causal, scale=s)
    torch.cuda.synchronize()
    go = o.double().cpu().numpy()
    gl = lse.double().cpu().numpy()
    for i in range(len(qlens)):
        if qlens[i] == 0:
            continue
        q0, q1, k0, k1 = int(cq[i]), int(cq[i + 1]), int(ck[i]), int(ck[i + 1])
        ro, rl = oracle.attn(qp[None, :, q0:q1], kp[None, :, k0:k1], vp[None, :, k0:k1], s, causal)
        eo = float(np.max(np.abs(go[:, q0:q1] - ro[0])))
        el = float(np.max(np.abs(gl[:, q0:q1] - rl[0])))
        note(f"  seq {i}: sq={q1 - q0} sk={k1 - k0} O max-abs={eo:.3e} LSE max-abs={el:.3e}")
        assert eo <= TOL_O[dt] and el <= TOL_LSE


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_pingpong_equals_dense(causal, gpu):
    """Equal-length sequences packed through fa_fwd_varlen run the ping-pong
    kernel on the same rows, in the same order, as fa_fwd on [b, h, s, d]
    (per-pair grid, not the persistent one): the results are bitwise equal."""
    import torch
    note(f"[parity-varlen-pp] b2 h64 s2048 d128 bf16 causal={causal}")
    cfg = fa.fa_query_config(2, 128, int(causal), 2, 64, 2048, 2048)
    assert (cfg["waves"], cfg["block_m"]) == (8, 256)
    assert not fa.fa_query_launch(2, 128, int(causal), 2, 64, 2048, 2048)["persistent"]
    w = W.shape("vlpp", "bf16", 2, 64, 2048, 2048, 128, causal, seed=77)
    q, k, v = (t.cuda() for t in W.make(w))
    o, lse = fa.attention(q, k, v, causal=causal)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(64, 2 * 2048, 128).contiguous()
    cu = torch.tensor([0, 2048, 4096], dtype=torch.int32, device="cuda")
    ov, lv = fa.attention_varlen(pack(q), pack(k), pack(v), cu, cu, 2048, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(ov, pack(o))
    assert torch.equal(lv, lse.permute(1, 0, 2).reshape(64, 4096))
