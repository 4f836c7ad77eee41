"""GPU parity of query-aware segment selection (kv_summarize,
kv_select_segments) against the CPU oracle: summaries, scores and kept
descriptor lists bit-exact; decode over the kept descriptors within the
attention tolerance of the oracle's decode over its own kept descriptors.
Caches are packed by the oracle, so this does not depend on the compress
kernels (the full-size case uses the library's own compress)."""
import numpy as np
import pytest
import torch

from compressed_kv_cache_compress_amd import DESC_DTYPE, gen, kara, runtime
from helpers import (SCALE, assemble_cache, check_attention, desc_to_dev, oracle_compress_all,
                     say, to_dev_u8)
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _check(q, buf_dev, desc_dev, descs_host, buf_host, keeps, *, n_kv_heads, n_desc=None,
           streams_to_check=None, label=""):
    """Runs summarize + select (+ decode over the selection) for each keep and
    compares the sampled streams with the oracle."""
    B, Hq = q.shape[0], q.shape[1]
    streams, maxd = descs_host.shape
    G = Hq // n_kv_heads
    nd_dev = None if n_desc is None else torch.tensor(np.asarray(n_desc, np.int32)).cuda()
    say(f"[select] {label}: streams={streams} maxd={maxd} keeps={keeps}")
    sm = runtime.summarize(buf_dev, desc_dev, batch=B, n_q_heads=Hq, n_kv_heads=n_kv_heads,
                           max_desc_per_stream=maxd, n_desc=nd_dev)
    torch.cuda.synchronize()
    smh = sm.cpu().numpy().view(np.uint16)
    qn = gen.u16(q)
    check = range(streams) if streams_to_check is None else streams_to_check
    for s in check:
        nd = maxd if n_desc is None else int(n_desc[s])
        ref = O.summarize_stream(buf_host, descs_host[s, :nd])
        assert np.array_equal(smh[s, :nd], ref), f"{label}: summary s={s}"
        assert not smh[s, nd:].any()
    for keep in keeps:
        od, on, score = runtime.select(q, sm, desc_dev, keep, n_kv_heads=n_kv_heads,
                                       max_desc_per_stream=maxd, n_desc=nd_dev)
        kk = min(keep, maxd)
        out, lse = runtime.decode(q, buf_dev, od, n_kv_heads=n_kv_heads, max_desc_per_stream=kk,
                                  n_desc=on, scale=float(SCALE))
        torch.cuda.synchronize()
        odh = od.cpu().numpy().view(DESC_DTYPE).reshape(streams, kk)
        onh = on.cpu().numpy()
        sch = score.cpu().numpy()
        for s in check:
            b, h = divmod(s, n_kv_heads)
            nd = maxd if n_desc is None else int(n_desc[s])
            qs = qn[b, h * G:(h + 1) * G]
            sel, rs = O.select_stream(qs, smh[s, :nd], descs_host[s, :nd], keep)
            assert np.array_equal(sch[s, :nd].view(np.uint32), rs.view(np.uint32)), \
                f"{label}: scores s={s} keep={keep}"
            assert np.all(np.isneginf(sch[s, nd:]))
            assert onh[s] == len(sel), (label, s, keep, onh[s], len(sel))
            assert np.array_equal(odh[s, :len(sel)].view(np.uint8),
                                  descs_host[s, sel].view(np.uint8)), f"{label}: kept s={s}"
            ro, rl = O.decode_stream(qs, buf_host, descs_host[s, sel], SCALE)
            check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                            f"{label} s={s} keep={keep}")


def test_select_mixed_strategies_gqa():
    w = gen.make_workload("batched128k", B=2, N=4096)
    S = 128
    strat = gen.table9(S)
    res = oracle_compress_all(w, S=S, strategies=strat, budget=gen.budget_bytes(25, S),
                              capacity=(4096 // S) * 16 * 1024)
    cap = (4096 // S) * 16 * 1024
    buf, descs = assemble_cache(res, cap)
    _check(w["q"].cuda(), to_dev_u8(buf), desc_to_dev(descs), descs, buf, [1, 4, 7, 32, 40],
           n_kv_heads=w["Hkv"], label="batched shape")


def test_select_empty_segments_ragged_lists_and_ties():
    """Zero-retention segments are never kept, per-stream descriptor counts
    differ (one stream has none), keep exceeds the non-empty count, and
    uniform keys make every score tie (kept by index)."""
    w = gen.make_workload("llama8b", B=1, N=2048)
    S = 128
    streams = w["B"] * w["Hkv"]
    nseg = 2048 // S
    g = torch.Generator().manual_seed(9)
    w["K"][:, :2] = torch.randint(-2, 3, w["K"][:, :2].shape, generator=g).to(torch.bfloat16)
    w["K"][:, 2, :] = 1.0  # every key equal: all scores of stream 2 tie
    forced = np.array([[(s + j) % 3 for j in range(nseg)] for s in range(streams)], np.uint8)
    strat = [(S, 128), (0, 0), (37, 56)]
    cap = nseg * 4 * S * 128
    res = oracle_compress_all(w, S=S, strategies=strat, budget=4 * S * 128, forced=forced,
                              capacity=cap)
    buf, descs = assemble_cache(res, cap)
    n_desc = np.array([nseg - (s % 5) for s in range(streams)], np.uint32)
    n_desc[3] = 0
    _check(w["q"].cuda(), to_dev_u8(buf), desc_to_dev(descs), descs, buf, [1, 3, 16],
           n_kv_heads=w["Hkv"], n_desc=n_desc, label="ragged")


@pytest.mark.parametrize("G", [1, 16])
def test_select_group_sizes(G):
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=2 * G, Hkv=2, N=1024, S=64, W=4)
    w = gen.make_workload(c)
    S = 64
    cap = (1024 // S) * 4 * S * 128
    res = oracle_compress_all(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(33, S),
                              capacity=cap)
    buf, descs = assemble_cache(res, cap)
    _check(w["q"].cuda(), to_dev_u8(buf), desc_to_dev(descs), descs, buf, [2, 5],
           n_kv_heads=2, label=f"G={G}")


def test_select_kara_cache():
    """Mixed cache: dense 256-token prompt segments, 13-token event segments,
    dense tail; selection keeps 1/8 of the descriptors."""
    k = gen.KARA
    w = gen.make_kara(device="cuda", B=2, prompt=2048, gen=1024)
    cache = kara.build_cache(w["K"], w["V"], w["Qall"], prompt=w["prompt"], gen=w["gen"],
                             window=k["window"], delta=k["delta"], protect=k["protect"], seg=64,
                             retention_pct=k["retention_pct"], alpha=k["alpha"], gamma=k["gamma"],
                             scale=float(SCALE))
    torch.cuda.synchronize()
    streams = w["B"] * w["Hkv"]
    descs = cache.desc.cpu().numpy().view(DESC_DTYPE).reshape(streams, cache.max_desc)
    buf = cache.packed.cpu().numpy()
    keep = max(1, cache.max_desc // 8)
    _check(w["q"], cache.packed, cache.desc, descs, buf, [keep], n_kv_heads=w["Hkv"],
           streams_to_check=[0, 5, streams - 1], label="kara")


def test_select_fullsize_batched128k():
    """batched128k at full size, the library's own compress, 12.5 % of the
    segments kept; sampled streams against the oracle."""
    c = gen.CONFIGS["batched128k"]
    S = c["S"]
    w = gen.make_workload("batched128k", device="cuda")
    r = runtime.compress(w["K"], w["V"], w["Qw"], seg_tokens=S, strategies=gen.table9(S),
                         budget_bytes=gen.budget_bytes(c["budget_pct"], S), scale=float(SCALE))
    torch.cuda.synchronize()
    del w["K"], w["V"], w["Qw"]
    torch.cuda.empty_cache()
    descs = r.desc_host()
    maxd = r.n_seg
    streams = descs.shape[0]
    keep = maxd // 8
    check = [0, 77]
    # the sampled streams' bytes only (the whole buffer is 1.2 GB)
    buf = np.zeros(int(max(int(descs[s]["offset"].max()) for s in check)) + 64 * 1024, np.uint8)
    for s in check:
        a = s * r.layout.stream_capacity
        n = int(r.used[s].item())
        buf[a:a + n] = r.packed[a:a + n].cpu().numpy()
    _check(w["q"], r.packed, r.desc, descs, buf, [keep], n_kv_heads=c["Hkv"],
           streams_to_check=check, label="batched128k full size")


@pytest.mark.parametrize("n_seg,S", [(2048, 16), (5000, 16)])
def test_select_long_descriptor_lists(n_seg, S):
    """More than 1024 and more than 4096 descriptors per stream (the wider
    register layouts of the top-k)."""
    c = dict(gen.CONFIGS["tiny"])
    N = ((n_seg * S + 63) // 64) * 64
    c.update(Hq=2, Hkv=1, N=N, S=S, W=2)
    w = gen.make_workload(c)
    cap = n_seg * 4 * S * 128
    res = oracle_compress_all(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(33, S),
                              region_len=n_seg * S, capacity=cap)
    buf, descs = assemble_cache(res, cap)
    _check(w["q"].cuda(), to_dev_u8(buf), desc_to_dev(descs), descs, buf, [1, n_seg // 16, n_seg],
           n_kv_heads=1, label=f"{n_seg} segments")
