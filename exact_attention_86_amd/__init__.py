"""Exact attention prefill forward for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/fa.h`` (``libfa.so`` built
in-tree by ``exact_attention_86_amd.build``).  The functions here only marshal
arguments; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing or fails to load, calls
raise.

    fa_fwd(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, stream)
        the C entry point with raw device addresses (ints) and sizes
    fa_fwd_split(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, nsplit,
                 workspace, workspace_bytes, stream)
        split-KV forward; fa_split_workspace_bytes(b, h, sq, d, nsplit) sizes
        its workspace
    fa_fwd_split_noalloc(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype,
                         nsplit, stream)
        the same with the library's own per-GPU scratch (allocates nothing)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, h, total_q,
                  total_k, max_sq, d, scale, causal, dtype, stream)
        packed variable-length sequences
    attention(q, k, v, causal=False, scale=None, out=None, lse=None, nsplit=1)
        convenience wrapper over torch device tensors [b, h, s, d]
    attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_sq, causal=False, ...)
        convenience wrapper over packed torch tensors [h, total, d]
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_MISALIGNED, FA_ERR_TOO_LARGE, FA_ERR_HIP = range(6)
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
                3: "FA_ERR_MISALIGNED", 4: "FA_ERR_TOO_LARGE", 5: "FA_ERR_HIP"}
DTYPE_CODES = {"f32": FA_F32, "f16": FA_F16, "bf16": FA_BF16}

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, code: int, msg: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(code, str(code)), msg))
        self.code = code


def _declare(L):
    """Argument and result types of every exported entry point."""
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                         ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    L.fa_fwd.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    L.fa_query_config.argtypes = [ctypes.c_int, i64, ctypes.c_int, i64, i64, i64, i64, ip, ip, ip, ip]
    L.fa_query_config.restype = ctypes.c_int
    L.fa_query_launch.argtypes = [ctypes.c_int, i64, ctypes.c_int, i64, i64, i64, i64, ip, ip]
    L.fa_query_launch.restype = ctypes.c_int
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = ctypes.c_int
    L.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                               ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               vp, ctypes.c_size_t, vp]
    L.fa_fwd_split.restype = ctypes.c_int
    L.fa_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.fa_fwd_split_noalloc.restype = ctypes.c_int
    L.fa_split_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    L.fa_split_workspace_bytes.restype = ctypes.c_size_t
    L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    L.fa_fwd_varlen.restype = ctypes.c_int
    L.fa_bwd.argtypes = [vp] * 10 + [ctypes.c_size_t, i64, i64, i64, i64, i64,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa_bwd_varlen.argtypes = [vp] * 10 + [ctypes.c_size_t, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                            ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    L.fa_bwd_varlen.restype = ctypes.c_int
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                             ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int, vp]
    L.fa_fwd_fp8.restype = ctypes.c_int
    L.fa_clock_probe.argtypes = [vp, i64, vp]
    L.fa_clock_probe.restype = ctypes.c_int


def lib() -> ctypes.CDLL:
    """Load libfa.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _routed is not None:
            return _routed
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfa.so is not built; run python -m exact_attention_86_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
        return L


POISON_LIB_PATH = os.path.join(PKG, "libfa_poison.so")
_poison_lib = None
_routed = None


def poison_lib():
    """Load the debug build libfa_poison.so: the same entry points, with every
    global->LDS copy preceded by a NaN fill of its destination.  For race
    tests only; raises if it has not been built."""
    global _poison_lib
    with _lock:
        if _poison_lib is None:
            if not os.path.exists(POISON_LIB_PATH):
                raise RuntimeError("libfa_poison.so is not built; run python -m exact_attention_86_amd.build")
            L = ctypes.CDLL(POISON_LIB_PATH)
            _declare(L)
            _poison_lib = L
        return _poison_lib


@contextlib.contextmanager
def poisoned():
    """Route every call of this module to the debug build libfa_poison.so
    while the block runs (race tests; not thread-safe)."""
    global _routed
    L = poison_lib()
    _routed = L
    try:
        yield L
    finally:
        _routed = None


def fa_last_error() -> str:
    return lib().fa_last_error().decode()


def fa_version() -> int:
    return lib().fa_version()


def fa_query_config(dtype: int, d: int, causal: int = 0, b: int = 1, h: int = 1, sq: int = 1,
                    sk: int = 1) -> dict:
    """Tiling of fa_fwd for a problem (the kernel choice may depend on sizes)."""
    vals = [ctypes.c_int(0) for _ in range(4)]
    rc = lib().fa_query_config(int(dtype), int(d), int(causal), int(b), int(h), int(sq), int(sk),
                               *[ctypes.byref(x) for x in vals])
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return dict(zip(("block_m", "block_n", "waves", "lds"), (x.value for x in vals)))


def fa_query_launch(dtype: int, d: int, causal: int = 0, b: int = 1, h: int = 1, sq: int = 1,
                    sk: int = 1) -> dict:
    """The grid fa_fwd launches on the current device, and whether it is the
    persistent schedule."""
    vals = [ctypes.c_int(0) for _ in range(2)]
    rc = lib().fa_query_launch(int(dtype), int(d), int(causal), int(b), int(h), int(sq), int(sk),
                               *[ctypes.byref(x) for x in vals])
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return {"grid": vals[0].value, "persistent": bool(vals[1].value)}


def fa_fwd(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, stream) -> int:
    """The C entry point: device addresses as ints, returns the status code."""
    return lib().fa_fwd(q, k, v, o, lse, int(b), int(h), int(sq), int(sk), int(d),
                        float(scale), int(causal), int(dtype), stream)


def fa_fwd_split(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, nsplit, workspace,
                 workspace_bytes, stream) -> int:
    """The split-KV C entry point: device addresses as ints, returns the status code."""
    return lib().fa_fwd_split(q, k, v, o, lse, int(b), int(h), int(sq), int(sk), int(d),
                              float(scale), int(causal), int(dtype), int(nsplit), workspace,
                              int(workspace_bytes), stream)


def fa_fwd_split_noalloc(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, nsplit,
                         stream) -> int:
    """The split-KV C entry point that allocates nothing (library-owned
    scratch of FA_NOALLOC_SCRATCH_BYTES per GPU): device addresses as ints,
    returns the status code."""
    return lib().fa_fwd_split_noalloc(q, k, v, o, lse, int(b), int(h), int(sq), int(sk), int(d),
                                      float(scale), int(causal), int(dtype), int(nsplit), stream)


FA_NOALLOC_SCRATCH_BYTES = 64 << 20


def fa_split_workspace_bytes(b, h, sq, d, nsplit) -> int:
    """Workspace bytes fa_fwd_split needs (0 for nsplit = 1 or invalid sizes)."""
    return int(lib().fa_split_workspace_bytes(int(b), int(h), int(sq), int(d), int(nsplit)))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, h, total_q, total_k,
                  max_sq, d, scale, causal, dtype, stream) -> int:
    """The variable-length C entry point: device addresses as ints, returns the status code."""
    return lib().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, int(batch), int(h),
                               int(total_q), int(total_k), int(max_sq), int(d), float(scale),
                               int(causal), int(dtype), stream)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, b, h, sq, sk, d,
           scale, causal, dtype, stream) -> int:
    """The backward C entry point: device addresses as ints, returns the status code."""
    return lib().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, int(workspace_bytes),
                        int(b), int(h), int(sq), int(sk), int(d), float(scale), int(causal),
                        int(dtype), stream)


def fa_fwd_fp8(q, k, v, o, lse, b, h, sq, sk, d, scale, descale_q, descale_k, descale_v, causal,
               stream) -> int:
    """The FP8 forward C entry point: device addresses as ints, returns the status code."""
    return lib().fa_fwd_fp8(q, k, v, o, lse, int(b), int(h), int(sq), int(sk), int(d), float(scale),
                            float(descale_q), float(descale_k), float(descale_v), int(causal), stream)


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, cu_seqlens_q,
                  cu_seqlens_k, batch, h, total_q, total_k, max_sq, max_sk, d, scale, causal, dtype,
                  stream) -> int:
    """The variable-length backward C entry point: device addresses as ints,
    returns the status code."""
    return lib().fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, int(workspace_bytes),
                               cu_seqlens_q, cu_seqlens_k, int(batch), int(h), int(total_q),
                               int(total_k), int(max_sq), int(max_sk), int(d), float(scale),
                               int(causal), int(dtype), stream)


def fa_bwd_workspace_bytes(b, h, sq) -> int:
    """Workspace bytes fa_bwd needs (0 for invalid sizes)."""
    return int(lib().fa_bwd_workspace_bytes(int(b), int(h), int(sq)))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise FaError(FA_ERR_UNSUPPORTED, "dtype %s not served" % t.dtype)
    return codes[t.dtype]


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output or workspace must be a contiguous tensor of
    the given shape and dtype on the given device: the kernels write exactly
    the elements the input sizes imply, so a smaller or wrongly typed buffer
    would be written past its end or filled with the wrong encoding."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise FaError(FA_ERR_INVALID_ARG, "%s must be a torch tensor" % name)
    if t.device != device:
        raise FaError(FA_ERR_INVALID_ARG, "%s must be on %s (got %s)" % (name, device, t.device))
    if dtype is not None and t.dtype != dtype:
        raise FaError(FA_ERR_INVALID_ARG, "%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise FaError(FA_ERR_INVALID_ARG, "%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise FaError(FA_ERR_INVALID_ARG, "%s must be contiguous" % name)


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None,
              lse=None, stream=None, nsplit: int = 1, workspace=None):
    """O, LSE for torch device tensors q [b,h,sq,d], k/v [b,h,sk,d].

    Outputs are allocated with torch when not given.  Runs on ``stream`` (a
    torch stream) or torch's current stream; returns (O, LSE) without
    synchronising.  ``nsplit`` > 1 runs the split-KV forward; its workspace
    (a torch uint8 device tensor) is allocated when not given.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be 4-d [b, h, s, d]")
    b, h, sq, d = q.shape
    sk = k.shape[2]
    if tuple(k.shape) != (b, h, sk, d) or tuple(v.shape) != (b, h, sk, d):
        raise FaError(FA_ERR_INVALID_ARG, "k and v must be [b, h, sk, d] matching q")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must share a dtype")
    if out is not None:
        _check_buffer("out", out, (b, h, sq, d), q.dtype, q.device)
    if lse is not None:
        _check_buffer("lse", lse, (b, h, sq), torch.float32, q.device)
    if workspace is not None:
        _check_buffer("workspace", workspace, None, None, q.device)
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be device tensors")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((b, h, sq), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    if nsplit == 1:
        rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    b, h, sq, sk, d, scale, int(bool(causal)), _dtype_code(q), s.cuda_stream)
    else:
        need = fa_split_workspace_bytes(b, h, sq, d, nsplit)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        nbytes = workspace.numel() * workspace.element_size()
        rc = fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          b, h, sq, sk, d, scale, int(bool(causal)), _dtype_code(q), nsplit,
                          workspace.data_ptr(), nbytes, s.cuda_stream)
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return out, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_sq: int, causal: bool = False,
                     scale: float | None = None, out=None, lse=None, stream=None):
    """O [h, total_q, d], LSE [h, total_q] for packed sequences: q [h, total_q, d],
    k/v [h, total_k, d] device tensors, cu_seqlens_* int32 device tensors of
    batch + 1 offsets.  Returns without synchronising."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be 3-d [h, total, d]")
    h, total_q, d = q.shape
    total_k = k.shape[1]
    if tuple(k.shape) != (h, total_k, d) or tuple(v.shape) != (h, total_k, d):
        raise FaError(FA_ERR_INVALID_ARG, "k and v must be [h, total_k, d] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must share a dtype")
    if out is not None:
        _check_buffer("out", out, (h, total_q, d), q.dtype, q.device)
    if lse is not None:
        _check_buffer("lse", lse, (h, total_q), torch.float32, q.device)
    for t in (q, k, v, cu_seqlens_q, cu_seqlens_k):
        if not (t.is_cuda and t.is_contiguous()):
            raise FaError(FA_ERR_INVALID_ARG, "all tensors must be contiguous device tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise FaError(FA_ERR_INVALID_ARG, "cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise FaError(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k need batch + 1 entries each")
    batch = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((h, total_q), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch, h, total_q, total_k,
                       max_sq, d, scale, int(bool(causal)), _dtype_code(q), s.cuda_stream)
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return out, lse


def attention_bwd(q, k, v, out, lse, dout, causal: bool = False, scale: float | None = None,
                  dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV for torch device tensors: q, out, dout [b,h,sq,d], k/v
    [b,h,sk,d], lse [b,h,sq] fp32 as attention() returned them for the same
    causal and scale.  Outputs and the workspace are allocated with torch when
    not given.  Returns (dQ, dK, dV) without synchronising."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be 4-d [b, h, s, d]")
    b, h, sq, d = q.shape
    sk = k.shape[2]
    if tuple(k.shape) != (b, h, sk, d) or tuple(v.shape) != (b, h, sk, d):
        raise FaError(FA_ERR_INVALID_ARG, "k and v must be [b, h, sk, d] matching q")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise FaError(FA_ERR_INVALID_ARG, "out and dout must have q's shape")
    if tuple(lse.shape) != (b, h, sq) or lse.dtype != torch.float32:
        raise FaError(FA_ERR_INVALID_ARG, "lse must be fp32 [b, h, sq]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v, out, dout must share a dtype")
    for name, t, shp in (("dq", dq, (b, h, sq, d)), ("dk", dk, (b, h, sk, d)), ("dv", dv, (b, h, sk, d))):
        if t is not None:
            _check_buffer(name, t, shp, q.dtype, q.device)
    if workspace is not None:
        _check_buffer("workspace", workspace, None, None, q.device)
    for t in (q, k, v, out, lse, dout):
        if not (t.is_cuda and t.is_contiguous()):
            raise FaError(FA_ERR_INVALID_ARG, "all tensors must be contiguous device tensors")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fa_bwd_workspace_bytes(b, h, sq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                nbytes, b, h, sq, sk, d, scale, int(bool(causal)), _dtype_code(q), s.cuda_stream)
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return dq, dk, dv


def attention_bwd_varlen(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_sq: int, max_sk: int,
                         causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
                         workspace=None, stream=None):
    """dQ, dK, dV for packed sequences: q, out, dout [h, total_q, d], k/v
    [h, total_k, d], lse [h, total_q] fp32 as attention_varlen() returned
    them for the same offsets, causal and scale; cu_seqlens_* int32 device
    tensors of batch + 1 offsets.  Returns (dQ, dK, dV) without
    synchronising."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be 3-d [h, total, d]")
    h, total_q, d = q.shape
    total_k = k.shape[1]
    if tuple(k.shape) != (h, total_k, d) or tuple(v.shape) != (h, total_k, d):
        raise FaError(FA_ERR_INVALID_ARG, "k and v must be [h, total_k, d] matching q")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise FaError(FA_ERR_INVALID_ARG, "out and dout must have q's shape")
    if tuple(lse.shape) != (h, total_q) or lse.dtype != torch.float32:
        raise FaError(FA_ERR_INVALID_ARG, "lse must be fp32 [h, total_q]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v, out, dout must share a dtype")
    for name, t, shp in (("dq", dq, (h, total_q, d)), ("dk", dk, (h, total_k, d)), ("dv", dv, (h, total_k, d))):
        if t is not None:
            _check_buffer(name, t, shp, q.dtype, q.device)
    if workspace is not None:
        _check_buffer("workspace", workspace, None, None, q.device)
    for t in (q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k):
        if not (t.is_cuda and t.is_contiguous()):
            raise FaError(FA_ERR_INVALID_ARG, "all tensors must be contiguous device tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise FaError(FA_ERR_INVALID_ARG, "cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise FaError(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k need batch + 1 entries each")
    batch = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fa_bwd_workspace_bytes(1, h, total_q)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                       nbytes, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch, h, total_q,
                       total_k, max_sq, max_sk, d, scale, int(bool(causal)), _dtype_code(q), s.cuda_stream)
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return dq, dk, dv


def attention_fp8(q, k, v, causal: bool = False, scale: float | None = None, descale_q: float = 1.0,
                  descale_k: float = 1.0, descale_v: float = 1.0, out=None, lse=None, stream=None):
    """O (bf16), LSE for E4M3 device tensors q [b,h,sq,d], k/v [b,h,sk,d]
    (torch.float8_e4m3fn or their uint8 bytes) with per-tensor descale
    factors.  Returns (O, LSE) without synchronising."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be 4-d [b, h, s, d]")
    b, h, sq, d = q.shape
    sk = k.shape[2]
    if tuple(k.shape) != (b, h, sk, d) or tuple(v.shape) != (b, h, sk, d):
        raise FaError(FA_ERR_INVALID_ARG, "k and v must be [b, h, sk, d] matching q")
    for t in (q, k, v):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise FaError(FA_ERR_UNSUPPORTED, "q, k, v must be float8_e4m3fn (or its uint8 bytes)")
    if out is not None:
        _check_buffer("out", out, (b, h, sq, d), torch.bfloat16, q.device)
    if lse is not None:
        _check_buffer("lse", lse, (b, h, sq), torch.float32, q.device)
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous()):
            raise FaError(FA_ERR_INVALID_ARG, "q, k, v must be contiguous device tensors")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, h, sq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, h, sq), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    b, h, sq, sk, d, scale, descale_q, descale_k, descale_v, int(bool(causal)),
                    s.cuda_stream)
    if rc != FA_OK:
        raise FaError(rc, fa_last_error())
    return out, lse

