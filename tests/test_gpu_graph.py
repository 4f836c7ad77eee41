"""HIP graph capture of a whole step (kv_compress + kv_attend_decode): the
library enqueues kernels only (no allocation, no memset, no synchronisation),
so a step captures into one graph.  The graph is replayed several times with
eager work and synchronisations between replays, and every replay must
reproduce the eager step bit for bit (packed bytes, descriptors, output)."""
import pytest
import torch

import compressed_kv_cache_compress_amd as kvc
from compressed_kv_cache_compress_amd import gen
from helpers import SCALE, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("store_logits", [0, 1])
def test_graph_replays_match_eager_step(store_logits):
    say(f"[graph] store_logits={store_logits}")
    w = gen.make_workload("batched128k", B=2, N=4096, device="cuda")
    c = gen.CONFIGS["batched128k"]
    S = c["S"]
    p = kvc.KvParams(batch=2, n_q_heads=c["Hq"], n_kv_heads=c["Hkv"], n_ctx=4096, seg_tokens=S,
                     n_win=c["W"], strategies=gen.table9(S),
                     budget_bytes=gen.budget_bytes(c["budget_pct"], S), scale=float(SCALE),
                     store_logits=store_logits)
    _, L = kvc.kv_layout_query(p)
    dev = torch.device("cuda")
    streams = 2 * c["Hkv"]
    packed = torch.zeros(L.packed_bytes_max, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * L.n_seg * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    cws = torch.empty(L.compress_ws_bytes, dtype=torch.uint8, device=dev)
    dws = torch.empty(L.decode_ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((2, c["Hq"], 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, c["Hq"]), dtype=torch.float32, device=dev)

    def step():
        kvc.kv_compress(p, w["K"], w["V"], w["Qw"], None, packed, desc, used, None, None, cws)
        kvc.kv_attend_decode(p, w["q"], packed, desc, None, out, lse, dws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (packed, desc, used, out, lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (packed, desc, out, lse):
            t.zero_()  # eager work between replays; the replay must rewrite everything
        used.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("packed", "desc", "used", "out", "lse"), (packed, desc, used, out, lse), ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int64 else a,
                               b.view(torch.uint8) if b.dtype != torch.int64 else b), (rep, name)
