"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import, link or call it, and it shares no code with them.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, pthreads over query
rows).  This module only builds that file with gcc and marshals numpy arrays
into it.  It computes the attention formula of page "flash-attn 实现 prefill
阶段" (section 问题分析): O = softmax(scale * Q K^T) V over [b, h, s, d], with
the max-subtracted exponent and scale placement of page "flash.cu"
(forward_kernel), plus the row log-sum-exp LSE_i = m_i + ln l_i.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, invariants, hand-worked examples under ``tests/golden/`` and a library
routine (torch's fp64 CPU scaled-dot-product attention).  The two online
forms are pinned to the naive form by brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
# deliberately broken copies for the pin tests, kept apart from the definition
_SRC_MUTANTS = os.path.join(_HERE, "attn_mutants.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# mutant codes understood by oracle_attn_mutant (0 = correct definition)
MUTANTS = {
    "no_scale": 1,
    "causal_strict": 2,
    "k_transposed": 3,
    "lse_no_max": 4,
    "no_normalise": 5,
    "drop_last_key": 6,
    "exp_sign": 7,
    "v_row_off": 8,
    "max_last": 9,
}

# deliberate mistakes of the backward (pin tests only)
BWD_MUTANTS = {
    "no_d": 1,
    "dk_no_scale": 2,
    "dv_uses_dp": 3,
    "dq_uses_v": 4,
}


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so with gcc; returns the path."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_MUTANTS)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-std=c11", "-march=x86-64-v2", "-fPIC", "-shared",
           "-pthread", _SRC, _SRC_MUTANTS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lp = ctypes.POINTER(ctypes.c_int64)
        dims = [i64, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int]
        lib.oracle_attn.argtypes = [dp, dp, dp, dp, dp] + dims + [ctypes.c_int]
        lib.oracle_attn_mutant.argtypes = [dp, dp, dp, dp, dp] + dims + [ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_rows.argtypes = [dp, dp, dp, lp, i64, dp, dp] + dims + [ctypes.c_int]
        lib.oracle_attn_probs.argtypes = [dp, dp, dp, dp, dp, dp] + dims
        lib.oracle_attn_online_kv_outer.argtypes = [dp, dp, dp, dp, dp] + dims + [i64, i64]
        lib.oracle_attn_online_q_outer.argtypes = [dp, dp, dp, dp, dp] + dims + [i64, i64]
        lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp] + dims + [ctypes.c_int]
        lib.oracle_attn_bwd_mutant.argtypes = [dp, dp, dp, dp, dp, dp, dp] + dims + [ctypes.c_int]
        for f in ("oracle_attn", "oracle_attn_mutant", "oracle_attn_rows",
                  "oracle_attn_probs", "oracle_attn_online_kv_outer",
                  "oracle_attn_online_q_outer", "oracle_attn_bwd", "oracle_attn_bwd_mutant"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
        return lib


def default_threads() -> int:
    """Host threads the oracle uses by default (all cores this process may use)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _as_f64(a) -> np.ndarray:
    """Widen to a C-contiguous fp64 array (exact for fp32/fp16/bf16 values)."""
    if hasattr(a, "detach"):  # torch tensor: widen in torch (bf16 is exact there)
        import torch
        a = a.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [b, h, s, d]")
    b, h, sq, d = q.shape
    if k.shape[:2] != (b, h) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("shape mismatch among q, k, v")
    return b, h, sq, k.shape[2], d


def _scale_f64(scale) -> float:
    """The scale exactly as given.  Callers comparing with the GPU library pass
    the fp32 value that library receives (``float(numpy.float32(scale))``)."""
    return float(scale)


def attn(q, k, v, scale, causal=False, nthreads=None):
    """Naive definition.  Returns (O [b,h,sq,d] fp64, LSE [b,h,sq] fp64)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, h, sq, sk, d = _shapes(q, k, v)
    o = np.empty((b, h, sq, d), np.float64)
    lse = np.empty((b, h, sq), np.float64)
    rc = _load().oracle_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             b, h, sq, sk, d, _scale_f64(scale), int(bool(causal)),
                             int(nthreads or default_threads()))
    if rc:
        raise ValueError("oracle_attn rejected its arguments")
    return o, lse


def attn_mutant(q, k, v, scale, causal, mutant, nthreads=None):
    """A deliberately broken copy of the definition (see MUTANTS; the copy
    lives in attn_mutants.c, apart from the definition); pin tests only."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, h, sq, sk, d = _shapes(q, k, v)
    o = np.empty((b, h, sq, d), np.float64)
    lse = np.empty((b, h, sq), np.float64)
    code = MUTANTS[mutant] if isinstance(mutant, str) else int(mutant)
    rc = _load().oracle_attn_mutant(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                    b, h, sq, sk, d, _scale_f64(scale),
                                    int(bool(causal)), code,
                                    int(nthreads or default_threads()))
    if rc:
        raise ValueError("oracle_attn_mutant rejected its arguments")
    return o, lse


def attn_rows(q, k, v, rows, scale, causal=False, nthreads=None):
    """The definition for selected rows only.

    ``rows`` holds flat row indices r = (bi*h + hi)*sq + i.  Returns
    (O [len(rows), d], LSE [len(rows)]) in fp64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, h, sq, sk, d = _shapes(q, k, v)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.size
    o = np.empty((max(n, 1), d), np.float64)
    lse = np.empty((max(n, 1),), np.float64)
    rc = _load().oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v),
                                  rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  n, _ptr(o), _ptr(lse), b, h, sq, sk, d,
                                  _scale_f64(scale), int(bool(causal)),
                                  int(nthreads or default_threads()))
    if rc:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return o[:n], lse[:n]


def attn_probs(q, k, v, scale, causal=False):
    """The normalised softmax matrix P [b,h,sq,sk] with O and LSE (tiny inputs)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, h, sq, sk, d = _shapes(q, k, v)
    p = np.empty((b, h, sq, sk), np.float64)
    o = np.empty((b, h, sq, d), np.float64)
    lse = np.empty((b, h, sq), np.float64)
    rc = _load().oracle_attn_probs(_ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(o),
                                   _ptr(lse), b, h, sq, sk, d, _scale_f64(scale),
                                   int(bool(causal)))
    if rc:
        raise ValueError("oracle_attn_probs rejected its arguments")
    return p, o, lse


def _online(fn, q, k, v, scale, causal, br, bc):
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, h, sq, sk, d = _shapes(q, k, v)
    o = np.empty((b, h, sq, d), np.float64)
    lse = np.empty((b, h, sq), np.float64)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, h, sq, sk, d,
            _scale_f64(scale), int(bool(causal)), int(br), int(bc))
    if rc:
        raise ValueError("online oracle rejected its arguments")
    return o, lse


def attn_online_kv_outer(q, k, v, scale, causal=False, br=32, bc=32):
    """Online-softmax recurrence, key tile outer (normalised O per step)."""
    return _online(_load().oracle_attn_online_kv_outer, q, k, v, scale, causal, br, bc)


def attn_online_q_outer(q, k, v, scale, causal=False, br=64, bc=64):
    """Online-softmax recurrence, query tile outer (unnormalised accumulator)."""
    return _online(_load().oracle_attn_online_q_outer, q, k, v, scale, causal, br, bc)


def attn_bwd(q, k, v, dout, scale, causal=False, mutant=0, nthreads=None):
    """Gradient of the definition: (dQ, dK, dV) of sum(O * dout), fp64.

    ``mutant`` != 0 runs a deliberately broken copy instead (BWD_MUTANTS; the
    copy lives in attn_mutants.c); pin tests only."""
    q, k, v, g = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    b, h, sq, sk, d = _shapes(q, k, v)
    if g.shape != q.shape:
        raise ValueError("dout must have q's shape")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    code = BWD_MUTANTS[mutant] if isinstance(mutant, str) else int(mutant)
    if code:
        rc = _load().oracle_attn_bwd_mutant(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dk),
                                            _ptr(dv), b, h, sq, sk, d, _scale_f64(scale),
                                            int(bool(causal)), code)
    else:
        rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dk), _ptr(dv),
                                     b, h, sq, sk, d, _scale_f64(scale), int(bool(causal)),
                                     int(nthreads or default_threads()))
    if rc:
        raise ValueError("oracle_attn_bwd rejected its arguments")
    return dq, dk, dv
