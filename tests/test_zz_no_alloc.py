"""kv_attend_decode_noalloc (decode with the library's fixed scratch instead
of a caller's workspace) against kv_attend_decode, through the C ABI: the
same kernels run, so out and lse must match bit for bit.  Two calls in a
row, the second on a smaller cache, so that the second reuses scratch the
first left behind."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_compress_amd as kvc
from compressed_kv_cache_compress_amd import gen, runtime
from helpers import SCALE, say

pytestmark = pytest.mark.gpu


def _case(B, N, S):
    say(f"[noalloc] B={B} N={N} S={S}")
    w = gen.make_workload("batched128k", B=B, N=N, device="cuda")
    r = runtime.compress(w["K"], w["V"], w["Qw"], seg_tokens=S, strategies=gen.table9(S),
                         budget_bytes=gen.budget_bytes(25, S), scale=float(SCALE))
    q = w["q"]
    ref, ref_lse = runtime.decode(q, r.packed, r.desc, n_kv_heads=w["Hkv"],
                                  max_desc_per_stream=r.n_seg, scale=float(SCALE))
    p = runtime.decode_params(batch=B, n_q_heads=w["Hq"], n_kv_heads=w["Hkv"],
                              max_desc_per_stream=r.n_seg, scale=float(SCALE))
    _, L = kvc.kv_layout_query(p)
    assert 0 < L.decode_ws_bytes <= kvc.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    kvc.kv_attend_decode_noalloc(p, q, r.packed, r.desc, None, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    return L.decode_ws_bytes


def test_noalloc_decode_matches_workspace_decode():
    big = _case(4, 8192, 128)
    small = _case(1, 2048, 128)
    assert small < big


def test_noalloc_decode_rejects_oversized_scratch():
    """A shape whose split partials exceed the fixed scratch is refused on
    the host, before anything is enqueued."""
    p = kvc.KvParams(batch=64, n_q_heads=32, n_kv_heads=8, max_desc_per_stream=4096,
                     decode_splits=512)
    _, L = kvc.kv_layout_query(p)
    assert L.decode_ws_bytes > kvc.NOALLOC_SCRATCH_BYTES
    x = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kv_attend_decode_noalloc(p, x, x, x, None, x, None)
    assert e.value.status == -4
    assert np.isfinite(float(L.decode_ws_bytes))
