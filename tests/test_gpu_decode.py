"""GPU parity of kv_attend_decode against the fp64 oracle (inputs packed by
the oracle, so decode parity does not depend on the compress kernels)."""
import numpy as np
import pytest
import torch

from compressed_kv_cache_compress_amd import DESC_DTYPE, gen, runtime
from helpers import (SCALE, assemble_cache, check_attention, desc_to_dev, oracle_compress_all,
                     oracle_decode_all, say, to_dev_u8)
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _run(w, S, strategies, budget, splits=0, forced=None, n_desc=None, region_len=None):
    say(f"[decode] B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} N={w['N']} S={S} splits={splits}")
    streams = w["B"] * w["Hkv"]
    cap = ((w["N"] // S) * max(O.seg_bytes(t, c, S) for t, c in strategies) + 255) // 256 * 256
    res = oracle_compress_all(w, S=S, strategies=strategies, budget=budget, forced=forced,
                              capacity=cap, region_len=region_len)
    buf, descs = assemble_cache(res, cap)
    q = w["q"].cuda()
    nd_dev = None if n_desc is None else torch.tensor(n_desc, dtype=torch.int32).cuda()
    out, lse = runtime.decode(q, to_dev_u8(buf), desc_to_dev(descs), n_kv_heads=w["Hkv"],
                              max_desc_per_stream=descs.shape[1], n_desc=nd_dev,
                              decode_splits=splits, scale=float(SCALE))
    torch.cuda.synchronize()
    ref, rlse = oracle_decode_all(w["q"], buf, descs, n_desc)
    return check_attention(out, lse, ref, rlse, label=f"S={S} splits={splits}"), out, lse


def test_decode_tiny_mixed_strategies():
    w = gen.make_workload("tiny")
    S = 64
    worst, _, _ = _run(w, S, gen.table9(S), gen.budget_bytes(33, S))
    say(f"  worst rel err {worst:.2e}")


def test_decode_gqa_budget25_and_split_invariance():
    w = gen.make_workload("batched128k", B=2, N=2048)
    S = 128
    _, o1, l1 = _run(w, S, gen.table9(S), gen.budget_bytes(25, S), splits=1)
    _, o2, l2 = _run(w, S, gen.table9(S), gen.budget_bytes(25, S), splits=7)
    d = (o1.float() - o2.float()).abs().max().item()
    say(f"  split 1 vs 7 max diff {d:.2e}")
    # the merge of the splits has three shapes: up to 8 splits one group of
    # 128 threads (splits 1 and 7 above), up to 32 eight groups, beyond that
    # 32 groups x 32 channels per workgroup
    w = gen.make_workload("batched128k", B=1, N=8192)
    for sp in (20, 33, 64):
        _run(w, S, gen.table9(S), gen.budget_bytes(25, S), splits=sp)


def test_decode_keep_all_equals_dense_attention():
    w = gen.make_workload("llama8b", B=1, N=1024)
    S = 128
    _, out, lse = _run(w, S, [(S, 128)], 4 * S * 128)
    # independent reference: torch fp64 dense attention on the CPU
    K = w["K"].double()
    V = w["V"].double()
    q = w["q"].double()
    G = w["G"]
    Kr = K.repeat_interleave(G, dim=1)
    Vr = V.repeat_interleave(G, dim=1)
    L = torch.einsum("bhd,bhnd->bhn", q, Kr) * float(SCALE)
    P = torch.softmax(L, dim=-1)
    ref = torch.einsum("bhn,bhnd->bhd", P, Vr)
    rl = torch.logsumexp(L, dim=-1)
    check_attention(out, lse, ref.numpy().reshape(-1, 128), rl.numpy().reshape(-1), "keep-all")


def test_decode_zero_retention_and_nan_poison():
    """Segments forced to keep nothing own no bytes; every byte outside the
    segments is 0xFF (NaN as bf16) and must never be read."""
    w = gen.make_workload("llama8b", B=1, N=1024)
    S = 128
    streams = w["B"] * w["Hkv"]
    forced = np.tile(np.array([0, 1, 1, 0, 1, 0, 0, 1], np.uint8), (streams, 1))
    worst, out, _ = _run(w, S, [(S, 128), (0, 0)], 4 * S * 128, forced=forced)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("G", [1, 8, 16])
def test_decode_group_sizes(G):
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=2 * G, Hkv=2, N=1024, S=64, W=4)
    w = gen.make_workload(c)
    _run(w, 64, gen.table9(64), gen.budget_bytes(33, 64))


@pytest.mark.parametrize("G", [2, 3])
def test_decode_workgroup_merge_and_numbering(G):
    """Groups of 2 and 3 q heads (some waves of a workgroup merge no head)
    at split counts that are multiples of 4 (the four splits of a workgroup
    merged in the split kernel: 4, 12, 16) and that are not (6), with
    workgroup counts that are multiples of 8 (renumbered across the XCDs: 16
    splits x 2 streams = 8 workgroups) and that are not (4 and 12 splits)."""
    c = dict(gen.CONFIGS["tiny"])
    c.update(Hq=2 * G, Hkv=2, N=1024, S=64, W=4)
    w = gen.make_workload(c)
    for splits in (4, 6, 12, 16):
        _run(w, 64, gen.table9(64), gen.budget_bytes(33, 64), splits=splits)


def test_decode_ragged_descriptor_lists_and_empty_streams():
    """Per-stream descriptor counts differ (one stream has none), segments hold
    13 tokens (a ragged 16-token chunk) or all 256 (dense)."""
    w = gen.make_workload("llama8b", B=1, N=2048)
    streams = w["B"] * w["Hkv"]
    Sd, Sc = 256, 64
    capd = 4 * Sd * 128
    parts = []
    res_d = oracle_compress_all(w, S=Sd, strategies=[(Sd, 128)], budget=capd, region_len=1024,
                                capacity=None)
    res_c = oracle_compress_all(w, S=Sc, strategies=[(13, 128), (13, 64)], budget=4 * Sc * 128,
                                region_begin=1024, region_len=1024, t2c_alpha=3, t2c_gamma=16)
    cap = 4 * 1024 * 128 + 16 * (13 * 512 + 32) + 256
    buf = np.full(streams * cap, 0xFF, np.uint8)
    maxd = 4 + 16
    descs = np.zeros((streams, maxd), DESC_DTYPE)
    n_desc = np.zeros(streams, np.uint32)
    for s in range(streams):
        base = s * cap
        dd, dc = res_d[s], res_c[s]
        buf[base:base + dd["used"]] = dd["packed"]
        buf[base + dd["used"]:base + dd["used"] + dc["used"]] = dc["packed"]
        d1 = dd["desc"].copy()
        d1["offset"] += base
        d2 = dc["desc"].copy()
        d2["offset"] += base + dd["used"]
        k = s % 4  # ragged: drop some descriptors per stream
        lst = np.concatenate([d1[:4 - (k % 2)], d2[:16 - 3 * k]])
        if s == 5:
            lst = lst[:0]
        descs[s, :len(lst)] = lst
        n_desc[s] = len(lst)
    q = w["q"].cuda()
    ref, rlse = oracle_decode_all(w["q"], buf, descs, n_desc)
    G = w["G"]
    # default splits (at least one descriptor each), then 2 and 5 splits: more
    # descriptors than splits, so each split takes an equal share of chunks
    # (a dense 256-token segment is 22 chunks, a 13-token one 1)
    for splits in (0, 2, 5):
        out, lse = runtime.decode(q, to_dev_u8(buf), desc_to_dev(descs), n_kv_heads=w["Hkv"],
                                  max_desc_per_stream=maxd,
                                  n_desc=torch.tensor(n_desc.astype(np.int32)).cuda(),
                                  decode_splits=splits, scale=float(SCALE))
        torch.cuda.synchronize()
        check_attention(out, lse, ref, rlse, f"ragged, splits={splits}")
        assert np.all(np.isneginf(lse.cpu().numpy().reshape(-1)[5 * G:6 * G]))


def test_decode_wide_rows_and_chunk_tails():
    """Masked rows up to 88 channels take 16 tokens per chunk (88 fills the
    prefetch slots exactly), wider masked rows 8 (one transposed V block) and
    dense rows 12: every channel-count class (8, 16, 24, 32, 56, 88, 96, 104,
    112, 120, dense) with token counts that leave ragged chunk tails and
    partial V blocks (tails of 5, 14, 1 and 16 tokens among them), forced per
    segment, at several split counts."""
    w = gen.make_workload("llama8b", B=1, N=2048)
    S = 128
    strategies = [(37, 8), (100, 56), (17, 96), (128, 104), (45, 112), (99, 120), (77, 128),
                  (128, 128), (1, 120), (29, 104), (53, 88), (21, 32), (30, 24), (16, 16),
                  (49, 32)]
    streams = w["B"] * w["Hkv"]
    n_seg = w["N"] // S
    forced = np.array([[(s + 3 * j) % len(strategies) for j in range(n_seg)] for s in range(streams)],
                      np.uint8)
    for splits in (0, 3):
        worst, _, _ = _run(w, S, strategies, 4 * S * 128, splits=splits, forced=forced)
        say(f"  splits={splits} worst rel err {worst:.2e}")


def test_decode_long_ragged_lists():
    """Lists of up to 512 descriptors (capacity 512: the path that loads each
    descriptor's token and channel counts for the chunk shares, then fetches
    the descriptors) with per-stream lengths 0, 1, 257, 300, 384, 450, 511
    and 512, at the library's split count and at 7 and 24 splits; a split's
    share may start and end inside a segment."""
    c = dict(gen.CONFIGS["llama8b"])
    c.update(B=1, N=8192)
    w = gen.make_workload(c)
    S = 16
    n_desc = [512, 300, 257, 511, 0, 384, 1, 450]
    for splits in (0, 7, 24):
        worst, _, lse = _run(w, S, gen.table9(S), gen.budget_bytes(33, S), splits=splits,
                             n_desc=n_desc)
        G = w["G"]
        assert np.all(np.isneginf(lse.cpu().numpy().reshape(-1)[4 * G:5 * G]))
        say(f"  splits={splits} worst rel err {worst:.2e}")
