"""GPU parity of kv_compress against the CPU oracle: bit-exact on every
selection and indexing output (scores, objective, descriptors incl. chosen
strategy and offsets, channel masks, kept values, token index lists -- i.e.
the whole packed byte range of every stream)."""
import numpy as np
import pytest
import torch

from compressed_kv_cache_compress_amd import DESC_DTYPE, gen, runtime
from helpers import SCALE, oracle_compress_all, say

pytestmark = pytest.mark.gpu


def _compare(w, *, S, strategies, budget, region_begin=0, region_len=None, t2c_alpha=0,
             t2c_gamma=0, forced=None, streams=None, label="", budget_scope=0,
             compress_max_waves=0, store_logits=False):
    say(f"[compress] {label} B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} N={w['N']} S={S} "
        f"W={w['W']} region=({region_begin},{region_len})")
    K, V, Qw = w["K"].cuda(), w["V"].cuda(), w["Qw"].cuda()
    fdev = None if forced is None else torch.from_numpy(np.ascontiguousarray(forced)).cuda()
    r = runtime.compress(K, V, Qw, seg_tokens=S, strategies=strategies, budget_bytes=budget,
                         region_begin=region_begin, region_len=region_len, t2c_alpha=t2c_alpha,
                         t2c_gamma=t2c_gamma, scale=float(SCALE), forced=fdev, want_scores=True,
                         want_objective=True, budget_scope=budget_scope,
                         compress_max_waves=compress_max_waves, store_logits=store_logits)
    torch.cuda.synchronize()
    cap = r.layout.stream_capacity
    ref = oracle_compress_all(w, S=S, strategies=strategies, budget=budget,
                              region_begin=region_begin, region_len=region_len,
                              t2c_alpha=t2c_alpha, t2c_gamma=t2c_gamma, forced=forced,
                              streams=streams, capacity=cap, budget_scope=budget_scope)
    packed = r.packed.cpu().numpy()
    desc = r.desc_host()
    used = r.used.cpu().numpy()
    scores = r.scores.cpu().numpy()
    obj = r.objective.cpu().numpy()
    for s, o in ref.items():
        assert np.array_equal(scores[s].view(np.uint32), o["scores"].view(np.uint32)), f"scores s={s}"
        assert np.array_equal(obj[s].view(np.uint32), o["objective"].view(np.uint32)), f"objective s={s}"
        assert np.array_equal(desc[s].view(np.uint8), o["desc"].view(np.uint8)), \
            f"desc s={s}: gpu {desc[s][:4]} oracle {o['desc'][:4]}"
        assert used[s] == o["used"]
        got = packed[s * cap:s * cap + o["used"]]
        if not np.array_equal(got, o["packed"]):
            bad = np.nonzero(got != o["packed"])[0]
            raise AssertionError(f"packed s={s}: {bad.size} bytes differ, first at {bad[0]}")
    hist = np.bincount(desc["strategy"].ravel(), minlength=len(strategies))
    say(f"  strategies {hist.tolist()}")
    return r, ref


def test_compress_tiny_full_size():
    w = gen.make_workload("tiny")
    S = 64
    _compare(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(33, S), label="tiny")


def test_compress_llama_shape():
    w = gen.make_workload("llama8b", N=2048)
    S = 128
    _compare(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(33, S), label="llama8b")


def test_compress_batched_shape_budget25():
    w = gen.make_workload("batched128k", B=2, N=2048)
    S = 128
    _compare(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(25, S), label="batched")


def test_compress_million_shape_s256():
    w = gen.make_workload("million", N=8192)
    S = 256
    _compare(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(20, S), label="million",
             streams=[0, 3, 7])


@pytest.mark.parametrize("S", [16, 32])
def test_compress_small_segments_ragged_region(S):
    """Domain of 17 blocks of 64 (not a multiple of the region), region not at 0."""
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=4, Hkv=2, N=1088, S=S, W=8)
    w = gen.make_workload(c)
    _compare(w, S=S, strategies=gen.table9(S), budget=gen.budget_bytes(33, S), region_begin=64,
             region_len=960, label=f"S{S}")


def test_compress_ties_uniform_keys():
    """K = small integers (many equal magnitudes: channel ties) and window
    queries = 0 (all scores equal: token ties broken by position)."""
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=2, Hkv=1, N=512, S=64, W=4)
    w = gen.make_workload(c)
    g = torch.Generator().manual_seed(5)
    w["K"] = torch.randint(-3, 4, w["K"].shape, generator=g).to(torch.bfloat16)
    w["V"] = torch.randint(-2, 3, w["V"].shape, generator=g).to(torch.bfloat16)
    w["Qw"] = torch.zeros_like(w["Qw"])
    _compare(w, S=64, strategies=gen.table9(64), budget=gen.budget_bytes(33, 64), label="ties")


def test_compress_forced_and_rejected():
    w = gen.make_workload("tiny", N=1024)
    S = 64
    strat = gen.table9(S)
    nseg = 1024 // S
    forced = np.full((1, nseg), 0xFF, np.uint8)
    forced[0, :6] = [8, 5, 0, 40, 2, 7]  # 0: over budget, 40: out of range -> rejected
    r, _ = _compare(w, S=S, strategies=strat, budget=gen.budget_bytes(33, S), forced=forced,
                    label="forced")
    d = r.desc_host()[0]
    assert list(d["strategy"][[0, 1, 4, 5]]) == [8, 5, 2, 7]
    assert d["flags"][2] & 0x80 and d["flags"][3] & 0x80 and not d["flags"][6] & 0x80


def test_compress_many_channel_counts():
    """Six distinct channel counts below 128 (six interleaved threshold
    searches per vector), odd token counts, choice under a mid budget and a
    forced pattern."""
    w = gen.make_workload("llama8b", B=1, N=2048)
    S = 128
    strat = [(37, 8), (100, 56), (17, 96), (128, 104), (45, 112), (99, 120), (77, 128), (128, 128)]
    _compare(w, S=S, strategies=strat, budget=gen.budget_bytes(40, S), label="six c, choice")
    nseg = 2048 // S
    streams = w["B"] * w["Hkv"]
    forced = np.array([[(s + 3 * j) % len(strat) for j in range(nseg)] for s in range(streams)],
                      np.uint8)
    _compare(w, S=S, strategies=strat, budget=4 * S * 128, forced=forced, label="six c, forced")


@pytest.mark.parametrize("hq,hkv,W", [(1, 1, 150), (4, 1, 37), (2, 2, 71)])
def test_compress_window_query_split(hq, hkv, W):
    """Window-query counts that do not divide into the per-wave split (a
    wave takes at most 64 queries, four at a time, then single ones):
    G*W = 150, 148 and 71 queries per stream."""
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=hq, Hkv=hkv, N=2048, S=64, W=W)
    w = gen.make_workload(c, seed=3)
    _compare(w, S=64, strategies=gen.table9(64), budget=gen.budget_bytes(33, 64),
             region_begin=256, region_len=1472, label=f"G*W={hq // hkv * W}")


def _tie_workload(seed):
    """Small integer K and V (many equal magnitudes in every vector)."""
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=2, Hkv=1, N=512, S=64, W=4)
    w = gen.make_workload(c)
    g = torch.Generator().manual_seed(seed)
    w["K"] = torch.randint(-3, 4, w["K"].shape, generator=g).to(torch.bfloat16)
    w["V"] = torch.randint(-2, 3, w["V"].shape, generator=g).to(torch.bfloat16)
    return w


def test_compress_one_channel_count():
    """A single distinct channel count below 128: the per-vector threshold is
    found by the bit search instead of the sort (random and tied keys)."""
    w = gen.make_workload("llama8b", B=1, N=2048)
    strat = [(128, 128), (64, 48), (32, 48), (96, 128)]
    _compare(w, S=128, strategies=strat, budget=gen.budget_bytes(30, 128), label="one c")
    _compare(_tie_workload(11), S=64, strategies=[(64, 128), (32, 40), (16, 40)],
             budget=gen.budget_bytes(30, 64), label="one c, ties")


def test_compress_eight_channel_counts_ties():
    """The most distinct channel counts a table may hold (8), on vectors full
    of equal magnitudes: one sort serves all eight thresholds and ties go to
    the lower channels."""
    strat = [(64, 8), (48, 16), (40, 32), (32, 48), (24, 64), (16, 80), (12, 96), (8, 120),
             (64, 128)]
    _compare(_tie_workload(12), S=64, strategies=strat, budget=gen.budget_bytes(35, 64),
             label="eight c, ties")


@pytest.mark.parametrize("cfg,pct", [("tiny", 25), ("llama8b", 33), ("batched128k", 25)])
def test_compress_stream_budget(cfg, pct):
    """Per-stream budget (Lagrangian choice over all strategies): descriptors,
    packed bytes and objectives bit-exact; the stream stays within
    n_seg * budget and some segment exceeds the per-segment cap."""
    c = gen.CONFIGS[cfg]
    w = gen.make_workload(cfg, N=2048 if cfg != "tiny" else None, B=min(c["B"], 2))
    S = c["S"]
    budget = gen.budget_bytes(pct, S)
    r, ref = _compare(w, S=S, strategies=gen.table9(S), budget=budget, budget_scope=1,
                      label=f"{cfg} stream budget")
    n_seg = w["N"] // S
    used = r.used.cpu().numpy()
    assert np.all(used <= n_seg * budget)
    sb = [r.layout.seg_bytes[i] for i in range(9)]
    d = r.desc_host()
    assert max(sb[i] for i in d["strategy"].ravel()) > budget


def test_compress_kara_event_strided_window():
    """One Kara event: window = last 512 positions of a longer buffer (strided
    views), region [384, 448), T = 13 of 64, Token2Chunk alpha 3, gamma 16."""
    kw = gen.make_kara(B=2, prompt=512, gen=512)
    L = kw["L"]
    Hkv, G = kw["Hkv"], kw["G"]
    w0 = L - 512
    Kd, Vd, Qd = kw["K"].cuda(), kw["V"].cuda(), kw["Qall"].cuda()
    say(f"[compress] kara event B=2 L={L}")
    r = runtime.compress(Kd[:, :, w0:], Vd[:, :, w0:], Qd[:, :, w0:], seg_tokens=64,
                         strategies=[(13, 128)], budget_bytes=4 * 64 * 128, region_begin=384,
                         region_len=64, t2c_alpha=3, t2c_gamma=16, scale=float(SCALE),
                         n_ctx=512, kv_stream_stride=L * 128, qw_head_stride=L * 128,
                         want_scores=True)
    torch.cuda.synchronize()
    cap = r.layout.stream_capacity
    w = dict(B=2, Hkv=Hkv, G=G, K=kw["K"][:, :, w0:], V=kw["V"][:, :, w0:], Qw=kw["Qall"][:, :, w0:])
    ref = oracle_compress_all(w, S=64, strategies=[(13, 128)], budget=4 * 64 * 128,
                              region_begin=384, region_len=64, t2c_alpha=3, t2c_gamma=16,
                              capacity=cap)
    packed = r.packed.cpu().numpy()
    desc = r.desc_host()
    scores = r.scores.cpu().numpy()
    for s, o in ref.items():
        assert np.array_equal(scores[s].view(np.uint32), o["scores"].view(np.uint32))
        assert np.array_equal(desc[s].view(np.uint8), o["desc"].view(np.uint8))
        assert np.array_equal(packed[s * cap:s * cap + o["used"]], o["packed"])


def test_compress_deterministic():
    w = gen.make_workload("batched128k", B=1, N=1024)
    K, V, Qw = w["K"].cuda(), w["V"].cuda(), w["Qw"].cuda()
    outs = []
    for _ in range(2):
        r = runtime.compress(K, V, Qw, seg_tokens=128, strategies=gen.table9(128),
                             budget_bytes=gen.budget_bytes(25, 128), scale=float(SCALE),
                             want_scores=True)
        torch.cuda.synchronize()
        cap = r.layout.stream_capacity
        used = r.used.cpu().numpy()
        pk = r.packed.cpu().numpy()
        outs.append(([pk[s * cap:s * cap + used[s]] for s in range(len(used))],
                     r.desc.cpu().numpy(), r.scores.cpu().numpy()))
    assert all(np.array_equal(a, b) for a, b in zip(outs[0][0], outs[1][0]))
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][2].view(np.uint32), outs[1][2].view(np.uint32))


@pytest.mark.parametrize("waves", [1, 7, 64])
def test_compress_wave_cap(waves):
    """A cap on the waves in flight (each workgroup then walks several work
    units) changes nothing: still bit-exact against the oracle, on a shape
    that takes the shared token-score kernel and the query split of the
    partials, and one with several channel counts."""
    w = gen.make_workload("batched128k", B=1, N=1024)
    _compare(w, S=128, strategies=gen.table9(128), budget=gen.budget_bytes(25, 128),
             label=f"cap {waves} waves", compress_max_waves=waves)
    t = gen.make_workload("tiny", N=2048)
    _compare(t, S=64, strategies=gen.table9(64), budget=gen.budget_bytes(33, 64),
             label=f"tiny cap {waves} waves", compress_max_waves=waves)


def test_compress_stored_logits():
    """store_logits: the first scoring pass keeps the logits of the region
    and the second pass reads them back instead of recomputing them.  Every
    output stays bit-exact: whole domain, a region that starts mid-domain
    with a ragged query count, several channel counts, and a wave cap."""
    w = gen.make_workload("batched128k", B=2, N=2048)
    _compare(w, S=128, strategies=gen.table9(128), budget=gen.budget_bytes(25, 128),
             label="stored logits", store_logits=True)
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=4, Hkv=2, N=1088, S=32, W=9)
    t = gen.make_workload(c)
    _compare(t, S=32, strategies=gen.table9(32), budget=gen.budget_bytes(33, 32), region_begin=64,
             region_len=960, label="stored logits, region", store_logits=True)
    _compare(t, S=32, strategies=gen.table9(32), budget=gen.budget_bytes(33, 32), region_begin=64,
             region_len=960, label="stored logits, capped", store_logits=True,
             compress_max_waves=5)
