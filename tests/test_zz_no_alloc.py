"""fa_fwd_split_noalloc: the split-KV forward on the library's own per-GPU
scratch (for callers that cannot allocate) gives the same bits as
fa_fwd_split on a caller workspace -- the same kernels run -- over two calls
in a row, the second smaller than the first, so the second call works on
scratch the first one left behind."""
import numpy as np
import pytest

import exact_attention_86_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

CALLS = [
    # (dtype, b, h, sq, sk, d, causal, nsplit): the first nearly fills the
    # 64 MiB scratch (8 * 16 * 1000 * 129 * 4 = 66.0 MB), the second is smaller
    ("bf16", 1, 16, 1000, 3000, 128, True, 8),
    ("f16", 1, 2, 50, 700, 64, False, 4),
]


def _pair(dt, b, h, sq, sk, d, causal, nsplit):
    import torch
    print(f"[noalloc] {dt} b{b} h{h} sq{sq} sk{sk} d{d} causal={causal} nsplit={nsplit}", flush=True)
    w = W.shape("noalloc", dt, b, h, sq, sk, d, causal, seed=sq + sk + nsplit)
    q, k, v = (t.cuda() for t in W.make(w))
    s = float(np.float32(w.scale))
    code = W.DTYPE_CODE[dt]
    need = fa.fa_split_workspace_bytes(b, h, sq, d, nsplit)
    assert 0 < need <= fa.FA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1, o2 = torch.empty_like(q), torch.full_like(q, float("nan"))
    l1 = torch.empty((b, h, sq), dtype=torch.float32, device="cuda")
    l2 = torch.full_like(l1, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr())
    rc = fa.fa_fwd_split(*ptrs, o1.data_ptr(), l1.data_ptr(), b, h, sq, sk, d, s, int(causal), code,
                         nsplit, ws.data_ptr(), need, stream)
    assert rc == fa.FA_OK, fa.fa_last_error()
    rc = fa.fa_fwd_split_noalloc(*ptrs, o2.data_ptr(), l2.data_ptr(), b, h, sq, sk, d, s, int(causal),
                                 code, nsplit, stream)
    assert rc == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert bool(torch.isfinite(o2).all()) and bool(torch.isfinite(l2).all())


def test_noalloc_matches_workspace_entry_point_two_calls(gpu):
    for case in CALLS:
        _pair(*case)

