"""Seeded synthetic inputs for exact attention (shared by tests and bench).

This module draws inputs only: it holds none of the attention arithmetic, so
both the GPU path's tests and the fp64 oracle can take their inputs from it.

Recipe (one per workload, all i.i.d.):
  * generator ``numpy.random.default_rng(seed)`` (PCG64);
  * draws in fp64, in the order Q, K, V, each one C-order array [b, h, s, d];
  * optional exact power-of-two multiplier (x2 for the large-head workload);
  * fp64 -> fp32 -> the workload dtype with round-to-nearest-even (torch).

The five workloads are the prefill shapes of page "flash-attn 实现 prefill
阶段" (section 问题分析: [b, h, sq, d], d = 128 first) in fp32, fp16 and bf16,
causal and non-causal, a long causal sequence, and a head size of 256 with a
sequence length that is not a multiple of any tile.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    b: int
    h: int
    sq: int
    sk: int
    d: int
    causal: bool
    scale: float
    seed: int
    qk_mult: float = 1.0          # exact power-of-two multiplier on Q and K
    v_dist: str = "normal"        # "normal" or "uniform" (U(-1, 1))

    @property
    def flops(self) -> float:
        """4*b*h*sq*sk*d, halved when causal (the usual attention convention)."""
        f = 4.0 * self.b * self.h * self.sq * self.sk * self.d
        return f / 2 if self.causal else f

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once, LSE (fp32) written once."""
        e = self.elt_bytes
        return (e * self.b * self.h * (2 * self.sq + 2 * self.sk) * self.d
                + 4 * self.b * self.h * self.sq)

    def describe(self) -> dict:
        return {"workload": self.name, "dtype": self.dtype, "b": self.b, "h": self.h,
                "sq": self.sq, "sk": self.sk, "d": self.d, "causal": self.causal,
                "scale": self.scale, "seed": self.seed}


WORKLOADS = [
    Workload("tiny_fp32_b1h2s128d64", "f32", 1, 2, 128, 128, 64, False, 1 / 8, 1),
    Workload("prefill_fp16_b2h8s1024d128", "f16", 2, 8, 1024, 1024, 128, False,
             1 / math.sqrt(128), 2),
    Workload("causal_bf16_b4h32s4096d128", "bf16", 4, 32, 4096, 4096, 128, True,
             1 / math.sqrt(128), 3),
    Workload("long_causal_bf16_b1h32s16384d128", "bf16", 1, 32, 16384, 16384, 128, True,
             1 / math.sqrt(128), 4),
    Workload("ragged_bf16_b8h16s2000d256", "bf16", 8, 16, 2000, 2000, 256, False,
             1 / 16, 5, qk_mult=2.0, v_dist="uniform"),
]
BY_NAME = {w.name: w for w in WORKLOADS}
# the workload the headline throughput figure is quoted on
HEADLINE = WORKLOADS[2]


def shape(name: str = "custom", dtype: str = "bf16", b: int = 1, h: int = 1,
          sq: int = 64, sk: int | None = None, d: int = 128, causal: bool = False,
          scale: float | None = None, seed: int = 0, qk_mult: float = 1.0,
          v_dist: str = "normal") -> Workload:
    """An ad-hoc workload (scale defaults to 1/sqrt(d))."""
    sk = sq if sk is None else sk
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return Workload(name, dtype, b, h, sq, sk, d, causal, scale, seed, qk_mult, v_dist)


def varlen_lengths(n: int, lo: int, hi: int, seed: int):
    """Lengths of n packed sequences for a variable-length batch: i.i.d.
    integers uniform on [lo, hi] from numpy.random.default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, n)]


def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def draw_f32(w: Workload, seed: int | None = None):
    """Return (q, k, v) as fp32 numpy arrays (before rounding to the dtype)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    qs = (w.b, w.h, w.sq, w.d)
    ks = (w.b, w.h, w.sk, w.d)
    q = rng.standard_normal(qs, dtype=np.float64)
    if w.qk_mult != 1.0:
        q *= w.qk_mult
    q = q.astype(np.float32)
    k = rng.standard_normal(ks, dtype=np.float64)
    if w.qk_mult != 1.0:
        k *= w.qk_mult
    k = k.astype(np.float32)
    if w.v_dist == "uniform":
        v = rng.uniform(-1.0, 1.0, ks).astype(np.float32)
    else:
        v = rng.standard_normal(ks, dtype=np.float64).astype(np.float32)
    return q, k, v


def make(w: Workload, seed: int | None = None):
    """Return (q, k, v) as CPU torch tensors in the workload dtype."""
    import torch
    dt = _torch_dtype(w.dtype)
    return tuple(torch.from_numpy(a).to(dt) for a in draw_f32(w, seed))


def with_(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


def make_dout(w: Workload, seed: int | None = None):
    """The output gradient dO for a backward pass: i.i.d. standard normal
    [b, h, sq, d] from its own generator (seed + 7919), fp64 -> fp32 -> the
    workload dtype, as a CPU torch tensor."""
    import torch
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    g = rng.standard_normal((w.b, w.h, w.sq, w.d), dtype=np.float64).astype(np.float32)
    return torch.from_numpy(g).to(_torch_dtype(w.dtype))


FP8_MAX = 448.0  # largest finite OCP E4M3 value


def make_fp8(w: Workload, seed: int | None = None):
    """FP8 inputs for the same draws as ``make``: each of Q, K, V (fp32) is
    multiplied by a power of two that brings its largest magnitude into
    (FP8_MAX/2, FP8_MAX], rounded to OCP E4M3 (torch, round to nearest even),
    and paired with the inverse power of two as its descale factor.  Returns
    (q8, k8, v8, (descale_q, descale_k, descale_v)) with CPU tensors of dtype
    torch.float8_e4m3fn; dequantized value = stored E4M3 value * descale."""
    import torch
    out, desc = [], []
    for a in draw_f32(w, seed):
        amax = float(np.max(np.abs(a))) if a.size else 1.0
        e = math.floor(math.log2(FP8_MAX / amax)) if amax > 0 else 0
        out.append(torch.from_numpy(a * np.float32(2.0 ** e)).to(torch.float8_e4m3fn))
        desc.append(2.0 ** -e)
    return out[0], out[1], out[2], tuple(desc)

