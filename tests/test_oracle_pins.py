"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties one oracle function to a closed form, a brute-force search, a
textbook routine or a hand-worked example, chosen so that a plausible slip (a
dropped term, a wrong sign or index, a transposed operand, per-segment instead
of global normalisation) fails.  Passages cited are from the two review pages:
MosaicKV (arXiv 2607.00760) and KARA (arXiv 2607.01237).
"""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from compressed_kv_cache_compress_amd import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = np.float32(1.0 / math.sqrt(128.0))


def bf16_bits(x):
    return gen.u16(torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16))


def bits_to_f(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def nearest_f32(fr):
    """Exactly rounded fp32 of a Fraction (ties to even)."""
    f = np.float32(float(fr))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0] or (d == best[0] and (c.view(np.uint32) & 1) == 0):
            best = (d, c)
    return best[1]


# --------------------------------------------------------------------- exp2
def test_exp2_coefficients_are_exactly_rounded(O):
    getcontext().prec = 60
    ln2 = Fraction(Decimal(2).ln())
    c, l2e = O.exp2_coeffs()
    for k in range(8):
        want = nearest_f32(ln2 ** k / math.factorial(k))
        assert c[k] == want, (k, c[k], want)
    assert l2e == nearest_f32(Fraction(Decimal(1).exp().ln() / Decimal(2).ln()))


def test_exp2_within_two_ulp(O):
    rng = np.random.default_rng(1)
    y = np.concatenate([-rng.random(1_000_000, dtype=np.float32) * np.float32(125.0),
                        np.array([0.0, -0.5, -1.0, -124.5, -125.0], np.float32)])
    r = O.exp2(y).astype(np.float64)
    exact = np.exp2(y.astype(np.float64))
    ulp = np.spacing(exact.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(r - exact) / ulp) <= 2.0


def test_exp2_special_values(O):
    ints = -np.arange(0, 126, dtype=np.float32)
    assert np.array_equal(O.exp2(ints), np.ldexp(np.float32(1.0), ints.astype(np.int32)).astype(np.float32))
    assert np.all(O.exp2(np.array([-125.01, -126, -1000, -np.inf], np.float32)) == 0.0)


# ------------------------------------------------------------------ scoring
def _stream(seed, N, G, W, uniform_k=False):
    rng = np.random.default_rng(seed)
    K = bf16_bits(np.zeros((N, 128)) if uniform_k else rng.standard_normal((N, 128)) * 1.5)
    Qw = bf16_bits(rng.standard_normal((G * W, 128)))
    return K, Qw


def test_scores_uniform_keys_exact(O):
    """K = 0: every logit is 0, every exp is 1, Z = N, so each token gets
    exactly G*W/N (power-of-two N)."""
    G, W, N = 2, 8, 512
    K, Qw = _stream(3, N, G, W, uniform_k=True)
    m, iz = O.normalisers(K, Qw, SCALE)
    assert np.all(m == 0.0) and np.all(iz == np.float32(1.0 / N))
    s = O.token_scores(K, Qw, SCALE, m, iz)
    assert np.all(s == np.float32(G * W / N))


def test_scores_sum_to_query_count(O):
    """Each query's softmax sums to 1 over the domain, so the scores of all
    tokens sum to G*W ([K] accumulated attention over the window)."""
    G, W, N = 4, 16, 1024
    K, Qw = _stream(4, N, G, W)
    m, iz = O.normalisers(K, Qw, SCALE)
    s = O.token_scores(K, Qw, SCALE, m, iz)
    assert abs(np.sum(s.astype(np.float64)) - G * W) <= 1e-4 * G * W


def test_scores_match_fp64_softmax(O):
    """Brute force in fp64: per query a textbook softmax over all keys (no
    causal mask, [K] Fig. 3), summed over the queries of the group."""
    G, W, N = 2, 4, 256
    K, Qw = _stream(5, N, G, W)
    m, iz = O.normalisers(K, Qw, SCALE)
    s = O.token_scores(K, Qw, SCALE, m, iz)
    Kf = bits_to_f(K).astype(np.float64)
    Qf = bits_to_f(Qw).astype(np.float64)
    L = (Qf @ Kf.T) * float(SCALE)
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    ref = P.sum(axis=0)
    assert np.max(np.abs(s - ref)) <= 1e-5 * ref.max()
    assert np.max(np.abs(m - L.max(axis=1))) <= 1e-5 * np.abs(L).max()
    # a region sub-range returns the same scores
    s2 = O.token_scores(K, Qw, SCALE, m, iz, t0=64, nt=128)
    assert np.array_equal(s2, s[64:192])


# -------------------------------------------------------- channel selection
def test_channel_topc_vs_stable_sort(O):
    """[M] Fig. 6 caption, Stage-1: top elements of each vector; reading:
    magnitude order, ties to the lower channel."""
    rng = np.random.default_rng(6)
    for trial in range(200):
        x = rng.standard_normal(128) * (10.0 ** rng.integers(-2, 3))
        if trial % 3 == 0:  # many equal magnitudes, both signs, zeros
            x = rng.integers(-3, 4, 128).astype(np.float64)
        row = bf16_bits(x)
        key = (row & 0x7FFF).astype(np.int64)
        order = np.lexsort((np.arange(128), -key))
        for c in (8, 32, 64, 120, 128):
            mask, rho = O.channel_topc(row, c)
            bits = np.unpackbits(mask, bitorder="little")
            want = np.zeros(128, np.uint8)
            want[order[:c]] = 1
            assert np.array_equal(bits, want), (trial, c)
            xf = bits_to_f(row).astype(np.float64)
            e_all = np.sum(xf ** 2)
            ref = 1.0 if e_all == 0 else np.sum(xf[want == 1] ** 2) / e_all
            assert abs(rho - ref) <= 2e-6
            if c == 128:
                assert rho == 1.0


def test_outlier_channels_in_every_topc():
    """Generated keys: each of the 4 outlier channels (x10) is among the 32
    largest of nearly every K vector."""
    w = gen.make_workload("tiny", N=256)
    from oracle import oracle as O
    K = gen.u16(w["K"][0, 0])
    mag = np.abs(bits_to_f(K))
    outl = np.argsort(-mag.mean(axis=0))[:4]
    hits = np.zeros(4)
    n = 0
    for t in range(256):
        if w["heavy"][0, 0, t]:
            continue
        mask, _ = O.channel_topc(K[t], 32)
        hits += np.unpackbits(mask, bitorder="little")[outl]
        n += 1
    assert np.all(hits / n >= 0.8)


# ------------------------------------------------------- token selection
def _brute_top_t(s, T):
    best = None
    for sub in itertools.combinations(range(len(s)), T):
        tot = sum(Fraction(float(s[i])) for i in sub)
        if best is None or tot > best[0]:
            best = (tot, sub)
    return set(best[1])  # combinations are lexicographic: first max wins ties


def test_top_t_brute_force(O):
    rng = np.random.default_rng(7)
    for trial in range(40):
        S = 12
        s = rng.random(S).astype(np.float32)
        if trial % 2:
            s = np.round(s * 4).astype(np.float32) / 4  # ties
        for T in (0, 1, 3, 6, 11, 12):
            keep = O.top_t(s, T)
            assert set(np.nonzero(keep)[0]) == _brute_top_t(s, T), (trial, T)


def test_token2chunk_golden(O):
    cases = json.load(open(os.path.join(GOLDEN, "token2chunk_examples.json")))["cases"]
    for cs in cases:
        keep = O.token2chunk(np.array(cs["scores"], np.float32), cs["T"], cs["alpha"], cs["gamma"])
        assert list(np.nonzero(keep)[0]) == cs["keep"], cs["why"]


def test_token2chunk_properties(O):
    rng = np.random.default_rng(8)
    for trial in range(300):
        S = int(rng.choice([16, 32, 64]))
        T = int(rng.integers(2, S))
        alpha = int(rng.integers(0, T))
        gamma = int(rng.integers(2, 17))
        s = rng.random(S).astype(np.float32) ** 3
        keep = O.token2chunk(s, T, alpha, gamma)
        assert keep.sum() == T
        A = O.top_t(s, T - alpha)
        assert np.all(keep[A == 1] == 1)
        if alpha == 0:
            assert np.array_equal(keep, O.top_t(s, T))
        # kept tokens outside A: whole gaps between neighbouring A tokens with
        # span <= gamma (chunks, at most alpha tokens in all), plus the best
        # remaining tokens (fill)
        a = np.nonzero(A)[0]
        chunk = set()
        for k in range(len(a) - 1):
            gap = list(range(a[k] + 1, a[k + 1]))
            if gap and a[k + 1] - a[k] + 1 <= gamma and all(keep[t] for t in gap):
                chunk.update(gap)
        assert len(chunk) <= alpha
        fill = [t for t in np.nonzero(keep)[0] if not A[t] and t not in chunk]
        rest = [t for t in np.lexsort((np.arange(S), -s)) if not A[t] and t not in chunk]
        assert sorted(fill) == sorted(rest[:len(fill)])


# --------------------------------------------------- layout, pack, choice
S128_PCT = [100.0, 56.25, 31.25, 50.2, 28.3, 15.8, 25.1, 14.2, 7.9]


def test_segment_bytes_table(O):
    S = 128
    for (T, c), pct in zip(gen.table9(S), S128_PCT):
        b = O.seg_bytes(T, c, S)
        assert abs(100.0 * b / (4 * S * 128) - pct) < 0.06, (T, c, b)
    assert O.seg_bytes(0, 0, S) == 0
    assert O.seg_bytes(13, 128, 64) == 13 * 512 + 32


def unpack_segment(buf, d, S):
    """Independent parser of one packed segment -> (idx, Kd, Vd, mk, mv): dense
    rows (zero where dropped) as uint16 bits and boolean masks."""
    T, c, off = int(d["n_tok"]), int(d["n_ch"]), int(d["offset"])
    pos = off

    def masks():
        nonlocal pos
        if c < 128:
            m = np.unpackbits(buf[pos:pos + 16 * T].reshape(T, 16), axis=1, bitorder="little")
            pos += 16 * T
            return m.astype(bool)
        return np.ones((T, 128), bool)

    def vals(m):
        nonlocal pos
        v = buf[pos:pos + 2 * T * c].view(np.uint16).reshape(T, c)
        pos += 2 * T * c
        out = np.zeros((T, 128), np.uint16)
        for t in range(T):
            out[t, m[t]] = v[t]
        return out

    def v_blocks():
        # V of a masked segment: blocks of 8 tokens, each transposed: bit
        # nb*(2l + h) + t of the block's mask bytes is (token t, channel
        # 64h + l); its values follow in (l, h, t) order
        nonlocal pos
        mpos, vpos = pos, pos + 16 * T
        m = np.zeros((T, 128), bool)
        out = np.zeros((T, 128), np.uint16)
        for b in range(0, T, 8):
            nb = min(8, T - b)
            bits = np.unpackbits(buf[mpos + 16 * b:mpos + 16 * (b + nb)], bitorder="little")
            lht = bits.reshape(64, 2, nb).astype(bool)  # [l][h][t]
            cnt = int(lht.sum())
            v = buf[vpos + 2 * c * b:vpos + 2 * c * b + 2 * cnt].view(np.uint16)
            ll, hh, tt = np.nonzero(lht)  # (l, h, t) order
            ch = 64 * hh + ll
            m[b + tt, ch] = True
            out[b + tt, ch] = v
        pos += 16 * T + 2 * T * c
        return m, out

    mk = masks()
    Kd = vals(mk)
    if c < 128:
        mv, Vd = v_blocks()
    else:
        mv = masks()
        Vd = vals(mv)
    if T < S:
        idx = buf[pos:pos + 2 * T].view(np.uint16).astype(np.int64)
        pad_end = off + int(O_seg_bytes(T, c, S))
        assert np.all(buf[pos + 2 * T:pad_end] == 0)
    else:
        idx = np.arange(S)
    return idx, Kd, Vd, mk, mv


def O_seg_bytes(T, c, S):
    from oracle import oracle as O
    return O.seg_bytes(T, c, S)


def _small_stream(seed, N=512, G=2, W=8):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((N, 128))
    K[:, rng.choice(128, 4, replace=False)] *= 10
    heavy = rng.choice(N, N // 32, replace=False)
    K[heavy] = K[heavy] * 0.25 + 8.0 * np.sign(rng.standard_normal(128))
    V = rng.standard_normal((N, 128))
    Qw = rng.standard_normal((G, W, 128))
    Qw += 0.7 * np.sign(K[heavy[0]])
    return bf16_bits(K), bf16_bits(V), bf16_bits(Qw)


def test_pack_round_trip(O):
    K, V, Qw = _small_stream(9)
    S = 64
    r = O.compress_stream(K, V, Qw, S=S, strategies=gen.table9(S),
                          budget_bytes=gen.budget_bytes(33, S), scale=SCALE)
    buf = r["packed"]
    off = 0
    for sg, d in enumerate(r["desc"]):
        assert int(d["offset"]) == off and d["seg_tokens"] == S
        T, c = gen.table9(S)[d["strategy"]]
        assert (d["n_tok"], d["n_ch"]) == (T, c)
        idx, Kd, Vd, mk, mv = unpack_segment(buf, d, S)
        assert len(idx) == T and np.all(np.diff(idx) > 0)
        rows = sg * S + idx
        assert np.all(mk.sum(axis=1) == c) and np.all(mv.sum(axis=1) == c)
        assert np.array_equal(Kd, np.where(mk, K[rows], 0))
        assert np.array_equal(Vd, np.where(mv, V[rows], 0))
        off += O.seg_bytes(T, c, S)
    assert r["used"] == off


def test_pack_v_blocks_partial_and_bit_positions(O):
    """Masked V parts are stored in transposed 8-token blocks (the last one
    partial when T is not a multiple of 8): every kept element round-trips
    through the independent unpacker, and one hand-placed element sits at the
    bit and value position the layout names."""
    K, V, Qw = _small_stream(21, N=256)
    S = 64
    strat = [(13, 40), (20, 64), (5, 8), (64, 120)]
    r = O.compress_stream(K, V, Qw, S=S, strategies=strat, budget_bytes=4 * S * 128,
                          scale=SCALE, forced=np.array([0, 1, 2, 3], np.uint8))
    buf = r["packed"]
    for sg, d in enumerate(r["desc"]):
        T, c = strat[sg]
        assert (int(d["n_tok"]), int(d["n_ch"])) == (T, c)
        idx, Kd, Vd, mk, mv = unpack_segment(buf, d, S)
        rows = sg * S + idx
        assert np.all(mv.sum(axis=1) == c)
        assert np.array_equal(Vd, np.where(mv, V[rows], 0))
    # segment 0 (T 13, c 40): block 1 holds tokens 8..12 (nb 5); its first
    # kept element in (l, h, t) order is the block's first value
    d = r["desc"][0]
    T, c = 13, 40
    idx, _, _, _, mv = unpack_segment(buf, d, S)
    vmask = int(d["offset"]) + 16 * T + 2 * T * c
    vval = vmask + 16 * T
    nb = 5
    lht = [(l, h, t) for l in range(64) for h in range(2) for t in range(nb) if mv[8 + t, 64 * h + l]]
    l, h, t = lht[0]
    bit = nb * (2 * l + h) + t
    assert (buf[vmask + 128 + bit // 8] >> (bit % 8)) & 1
    first = buf[vval + 2 * c * 8:vval + 2 * c * 8 + 2].view(np.uint16)[0]
    assert first == V[idx[8 + t], 64 * h + l]


def test_keep_all_pack_is_the_dense_cache(O):
    K, V, Qw = _small_stream(10, N=256)
    S = 64
    r = O.compress_stream(K, V, Qw, S=S, strategies=[(S, 128)], budget_bytes=4 * S * 128,
                          scale=SCALE)
    buf = r["packed"]
    for sg in range(256 // S):
        seg = buf[sg * 4 * S * 128:(sg + 1) * 4 * S * 128].view(np.uint16)
        assert np.array_equal(seg[:S * 128], K[sg * S:(sg + 1) * S].ravel())
        assert np.array_equal(seg[S * 128:], V[sg * S:(sg + 1) * S].ravel())


def _j_from_segment(buf, d, S, s, K, V, sg):
    """Objective recomputed from the materialised segment in fp64: kept score
    mass weighted by the mean kept energy share of the K and V vectors."""
    idx, Kd, Vd, mk, mv = unpack_segment(buf, d, S)
    tot = 0.0
    for j, t in enumerate(idx):
        kr = bits_to_f(K[sg * S + t]).astype(np.float64)
        vr = bits_to_f(V[sg * S + t]).astype(np.float64)
        ek = np.sum(bits_to_f(Kd[j]).astype(np.float64) ** 2) / max(np.sum(kr ** 2), 1e-300)
        ev = np.sum(bits_to_f(Vd[j]).astype(np.float64) ** 2) / max(np.sum(vr ** 2), 1e-300)
        tot += float(s[sg * S + t]) * 0.5 * (ek + ev)
    return tot


def test_choice_brute_force_enumeration(O):
    """[M] abstract / Fig. 5 caption: one strategy per segment; reading: the
    objective is the kept attention mass times the kept energy share, under a
    per-segment byte budget.  All 9^3 assignments of three segments are
    materialised (forced), the objective recomputed from the packed bytes, and
    the best feasible assignment (lowest on ties) must be the free choice."""
    S = 32
    strat = gen.table9(S)
    for seed in (11, 12):
        K, V, Qw = _small_stream(seed, N=96, G=2, W=4)
        budget = gen.budget_bytes(33, S)
        free = O.compress_stream(K, V, Qw, S=S, strategies=strat, budget_bytes=budget, scale=SCALE)
        s = free["scores"]
        feas = [i for i, (T, c) in enumerate(strat) if O.seg_bytes(T, c, S) <= budget]
        # J of every (segment, strategy), each from its own materialised segment
        Jm = {}
        for i in feas:
            f = O.compress_stream(K, V, Qw, S=S, strategies=strat, budget_bytes=budget,
                                  scale=SCALE, forced=np.full(3, i, np.uint8))
            for sg in range(3):
                Jm[(sg, i)] = _j_from_segment(f["packed"], f["desc"][sg], S, s, K, V, sg)
                assert abs(Jm[(sg, i)] - f["objective"][sg, i]) <= 1e-5 * max(1.0, Jm[(sg, i)])
        best = None
        for a in itertools.product(feas, repeat=3):  # lexicographic: first max wins ties
            tot = sum(Fraction(Jm[(sg, a[sg])]) for sg in range(3))  # exact: J spans decades
            if best is None or tot > best[0]:
                best = (tot, a)
        assert tuple(int(x) for x in free["desc"]["strategy"]) == best[1]


def test_budget_feasible_sets(O):
    for S, pct, want in ((64, 33, {2, 4, 5, 6, 7, 8}), (128, 33, {2, 4, 5, 6, 7, 8}),
                         (128, 25, {5, 7, 8}), (256, 20, {5, 7, 8})):
        b = gen.budget_bytes(pct, S)
        got = {i for i, (T, c) in enumerate(gen.table9(S)) if O.seg_bytes(T, c, S) <= b}
        assert got == want, (S, pct, got)


# -------------------------------------------------------------- decode
def dense_attention(q, K, V, scale):
    """Textbook softmax attention in fp64 (q [G,128], K/V [n,128] floats)."""
    L = (q @ K.T) * scale
    if L.shape[1] == 0:
        return np.zeros((q.shape[0], 128)), np.full(q.shape[0], -np.inf)
    mx = L.max(axis=1, keepdims=True)
    P = np.exp(L - mx)
    den = P.sum(axis=1, keepdims=True)
    return (P / den) @ V, (mx + np.log(den))[:, 0]


def test_decode_keep_all_equals_dense_attention(O):
    """Keep-all compression must equal dense softmax attention."""
    K, V, Qw = _small_stream(13, N=256)
    S = 64
    r = O.compress_stream(K, V, Qw, S=S, strategies=[(S, 128)], budget_bytes=4 * S * 128,
                          scale=SCALE)
    q = bf16_bits(np.random.default_rng(1).standard_normal((2, 128)))
    out, lse = O.decode_stream(q, r["packed"], r["desc"], SCALE)
    ref, rlse = dense_attention(bits_to_f(q).astype(np.float64), bits_to_f(K).astype(np.float64),
                                bits_to_f(V).astype(np.float64), float(SCALE))
    assert np.max(np.abs(out - ref)) <= 1e-12 and np.max(np.abs(lse - rlse)) <= 1e-12


def test_decode_zero_retention_segments_contribute_nothing(O):
    """Segments forced to keep no token add nothing: they own no bytes, and the
    output equals dense attention over the remaining tokens."""
    K, V, Qw = _small_stream(14, N=256)
    S = 64
    strat = [(S, 128), (0, 0)]
    r2 = O.compress_stream(K, V, Qw, S=S, strategies=strat, budget_bytes=4 * S * 128,
                           scale=SCALE, forced=np.array([0, 1, 0, 1], np.uint8))
    r = r2
    q = bf16_bits(np.random.default_rng(2).standard_normal((2, 128)))
    out, lse = O.decode_stream(q, r2["packed"], r2["desc"], SCALE)
    keep = np.r_[0:64, 128:192]
    ref, rlse = dense_attention(bits_to_f(q).astype(np.float64),
                                bits_to_f(K[keep]).astype(np.float64),
                                bits_to_f(V[keep]).astype(np.float64), float(SCALE))
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - ref)) <= 1e-12 and np.max(np.abs(lse - rlse)) <= 1e-12
    assert list(r["desc"]["n_tok"]) == [64, 0, 64, 0]


def test_decode_sparse_matches_masked_dense_attention(O):
    """Dropped channels count as 0 (reading): attention over the compressed
    stream equals dense attention over kept tokens with dropped channels
    zeroed, computed from an independent unpack."""
    K, V, Qw = _small_stream(15)
    S = 64
    r = O.compress_stream(K, V, Qw, S=S, strategies=gen.table9(S),
                          budget_bytes=gen.budget_bytes(33, S), scale=SCALE)
    Ks, Vs = [], []
    for d in r["desc"]:
        idx, Kd, Vd, _, _ = unpack_segment(r["packed"], d, S)
        Ks.append(Kd)
        Vs.append(Vd)
    Kc = bits_to_f(np.concatenate(Ks)).astype(np.float64)
    Vc = bits_to_f(np.concatenate(Vs)).astype(np.float64)
    q = bf16_bits(np.random.default_rng(3).standard_normal((2, 128)))
    out, lse = O.decode_stream(q, r["packed"], r["desc"], SCALE)
    ref, rlse = dense_attention(bits_to_f(q).astype(np.float64), Kc, Vc, float(SCALE))
    assert np.max(np.abs(out - ref)) <= 1e-12 and np.max(np.abs(lse - rlse)) <= 1e-12


def test_decode_empty_is_zero_minus_inf(O):
    from oracle.oracle import DESC_DTYPE
    q = bf16_bits(np.ones((3, 128)))
    out, lse = O.decode_stream(q, np.zeros(0, np.uint8), np.zeros(0, DESC_DTYPE), SCALE)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- Kara
def test_kara_window_scores(O):
    """Kara event: window of 512 positions scored bidirectionally; scores of
    all window tokens sum to G*512 queries ([K] Fig. 3: all pairs)."""
    w = gen.make_kara(B=1, prompt=512, gen=512)
    G = w["G"]
    K = gen.u16(w["K"][0, 0, 512:1024])
    Qw = gen.u16(w["Qall"][0, :G, 512:1024]).reshape(G * 512, 128)
    m, iz = O.normalisers(K, Qw, SCALE)
    s = O.token_scores(K, Qw, SCALE, m, iz)
    assert abs(np.sum(s.astype(np.float64)) - G * 512) <= 1e-4 * G * 512
    r = O.compress_stream(K, gen.u16(w["V"][0, 0, 512:1024]), Qw.reshape(G, 512, 128), S=64,
                          strategies=[(13, 128)], budget_bytes=4 * 64 * 128, scale=SCALE,
                          region_begin=384, region_len=64, t2c_alpha=3, t2c_gamma=16)
    assert np.array_equal(r["scores"], s[384:448])
    d = r["desc"][0]
    assert (d["n_tok"], d["n_ch"], d["flags"]) == (13, 128, 2)
    assert r["used"] == 13 * 512 + 32


# ---------------------------------------------------------------------------
# Query-aware segment selection (MosaicKV page, Fig. 6 caption: stage 2 runs
# during decode before each attention layer; Sec. 5.3: sequence compression in
# each decode attention layer; Fig. 8: token selection rates 6.25 % / 12.5 %).
# ---------------------------------------------------------------------------

def _selection_stream(O, seed, S=64):
    K, V, Qw = _small_stream(seed)
    r = O.compress_stream(K, V, Qw, S=S, strategies=gen.table9(S),
                          budget_bytes=gen.budget_bytes(33, S), scale=SCALE)
    return K, V, Qw, r


def test_summary_is_the_exact_channel_range(O):
    """kmin <= k <= kmax per channel over the decoded kept keys (dropped = 0),
    and both bounds are attained (independent unpacking of the segment)."""
    S = 64
    K, V, Qw, r = _selection_stream(O, 21, S)
    sm = O.summarize_stream(r["packed"], r["desc"])
    for i, d in enumerate(r["desc"]):
        _, Kd, _, _, _ = unpack_segment(r["packed"], d, S)
        kf = bits_to_f(Kd)
        assert np.array_equal(bits_to_f(sm[i, 0]), kf.max(axis=0))
        assert np.array_equal(bits_to_f(sm[i, 1]), kf.min(axis=0))


def test_select_score_closed_form(O):
    """Two non-zero channels: q = (1, -2), kmax = (3, 1), kmin = (-1, -4) gives
    max(3, -1) + max(-2, 8) = 11 for head 0; head 1 = -q gives
    max(-3, 1) + max(2, -8) = 3; the segment's score is the larger, 11."""
    q = np.zeros((2, 128), np.float32)
    q[0, :2] = [1, -2]
    q[1, :2] = [-1, 2]
    sm = np.zeros((1, 2, 128), np.float32)
    sm[0, 0, :2] = [3, 1]
    sm[0, 1, :2] = [-1, -4]
    desc = np.zeros(1, O.DESC_DTYPE)
    desc["n_tok"] = 1
    sel, score = O.select_stream(bf16_bits(q), bf16_bits(sm), desc, 1)
    assert score[0] == 11.0 and list(sel) == [0]


def test_select_score_bounds_every_kept_logit(O):
    """For every kept token and head, q.k (fp64, dropped channels 0) is at most
    the segment's score, up to the fp32 rounding of the score's sum."""
    S = 64
    K, V, Qw, r = _selection_stream(O, 22, S)
    q = bf16_bits(np.random.default_rng(3).standard_normal((2, 128)))
    sm = O.summarize_stream(r["packed"], r["desc"])
    _, score = O.select_stream(q, sm, r["desc"], 1)
    qf = bits_to_f(q).astype(np.float64)
    smf = bits_to_f(sm).astype(np.float64)
    for i, d in enumerate(r["desc"]):
        if d["n_tok"] == 0:
            assert np.isneginf(score[i])
            continue
        _, Kd, _, _, _ = unpack_segment(r["packed"], d, S)
        logits = bits_to_f(Kd).astype(np.float64) @ qf.T
        terms = np.maximum(qf[:, None, :] * smf[i, 0][None], qf[:, None, :] * smf[i, 1][None])
        slack = 128 * 2.0 ** -23 * np.abs(terms).sum(axis=-1).max()
        assert logits.max() <= float(score[i]) + slack


def test_select_top_k_brute_force(O):
    """On 8 segments with crafted summaries (ties included), the kept set is
    the k-subset of largest total score, ties to the lexicographically
    smallest indices, for every k."""
    rng = np.random.default_rng(4)
    n = 8
    q = np.zeros((1, 128), np.float32)
    q[0, 0] = 1.0
    sm = np.zeros((n, 2, 128), np.float32)
    vals = rng.integers(-3, 4, n).astype(np.float32)
    vals[5] = vals[2]  # a tie
    sm[:, 0, 0] = vals
    sm[:, 1, 0] = vals - 1
    desc = np.zeros(n, O.DESC_DTYPE)
    desc["n_tok"] = 1
    desc["n_tok"][6] = 0  # empty: never kept
    for k in range(0, n + 2):
        sel, score = O.select_stream(bf16_bits(q), bf16_bits(sm), desc, k)
        cand = [i for i in range(n) if desc["n_tok"][i] > 0]
        kk = min(k, len(cand))
        best = None
        for sub in itertools.combinations(cand, kk):
            key = (-sum(vals[list(sub)]), sub)
            if best is None or key < best:
                best = key
        assert tuple(sel) == best[1], (k, sel, best)


def test_select_all_equals_full_decode(O):
    """Keeping every segment reproduces decode over the whole stream; keeping
    the best quarter is decode over exactly those descriptors."""
    S = 64
    K, V, Qw, r = _selection_stream(O, 23, S)
    q = bf16_bits(np.random.default_rng(5).standard_normal((2, 128)))
    sm = O.summarize_stream(r["packed"], r["desc"])
    sel, _ = O.select_stream(q, sm, r["desc"], len(r["desc"]))
    nonempty = [i for i, d in enumerate(r["desc"]) if d["n_tok"] > 0]
    assert list(sel) == nonempty
    o_all, l_all = O.decode_stream(q, r["packed"], r["desc"], SCALE)
    o_sel, l_sel = O.decode_stream(q, r["packed"], r["desc"][sel], SCALE)
    assert np.array_equal(o_all, o_sel) and np.array_equal(l_all, l_sel)


def test_select_keeps_the_heavy_segment(O):
    """A segment whose keys align with q has the largest bound and is kept at
    the smallest k."""
    S = 64
    N = 512
    rng = np.random.default_rng(6)
    K = rng.standard_normal((N, 128)) * 0.5
    u = np.sign(rng.standard_normal(128))
    K[300] = 4.0 * u
    V = rng.standard_normal((N, 128))
    Qw = rng.standard_normal((1, 8, 128))
    K, V, Qw = bf16_bits(K), bf16_bits(V), bf16_bits(Qw)
    r = O.compress_stream(K, V, Qw, S=S, strategies=[(S, 128)], budget_bytes=4 * S * 128,
                          scale=SCALE)
    q = bf16_bits(u[None, :])
    sm = O.summarize_stream(r["packed"], r["desc"])
    sel, score = O.select_stream(q, sm, r["desc"], 1)
    assert list(sel) == [300 // S] and int(np.argmax(score)) == 300 // S


def test_summary_zero_sign_does_not_depend_on_order(O):
    """A channel holding -0 in one token and a dropped (+0) channel in another
    has range [+0, +0] in either token order."""
    S = 16
    K = np.zeros((S, 128), np.float32)
    K[:, 1:] = 1.0
    K[0, 0] = -0.0
    Kb = bf16_bits(K)
    V = bf16_bits(np.ones((S, 128), np.float32))
    Qw = bf16_bits(np.ones((1, 1, 128), np.float32))
    for order in (np.arange(S), np.arange(S)[::-1]):
        r = O.compress_stream(Kb[order], V, Qw, S=S, strategies=[(S, 128)],
                              budget_bytes=4 * S * 128, scale=SCALE)
        sm = O.summarize_stream(r["packed"], r["desc"])
        assert sm[0, 0, 0] == 0 and sm[0, 1, 0] == 0


# ---------------------------------------------------------------------------
# Per-stream byte budget (MosaicKV page, abstract: strategies chosen per KV
# segment under the memory target; Fig. 5 caption: strategy generation):
# multiple-choice knapsack over a stream's segments by Lagrangian relaxation.
# ---------------------------------------------------------------------------

def _table9_bytes(O, S):
    return [O.seg_bytes(t, c, S) for t, c in gen.table9(S)]


def _exact_sum(vals):
    return sum((Fraction(float(v)) for v in vals), Fraction(0))


def test_stream_budget_brute_force_optimality(O):
    """n_seg = 4, nine strategies: the choice fits B and no assignment using at
    most the chosen bytes has a larger objective sum (the defining property
    of a Lagrangian solution), checked over all 9^4 assignments."""
    S = 64
    nb = _table9_bytes(O, S)
    rng = np.random.default_rng(11)
    J = rng.random((4, 9)).astype(np.float32) * np.array([1, .9, .8, .7, .6, .5, .4, .3, .2],
                                                         np.float32)
    allsum = {}
    for a in itertools.product(range(9), repeat=4):
        allsum[a] = (sum(nb[i] for i in a), _exact_sum(J[k, i] for k, i in enumerate(a)))
    for B in (4 * min(nb), 12000, 20000, 30000, 45000, 4 * max(nb)):
        ch, _ = O.stream_choose(J, nb, B)
        used = sum(nb[i] for i in ch)
        assert used <= B
        val = _exact_sum(J[k, i] for k, i in enumerate(ch))
        best = max(v for (b, v) in allsum.values() if b <= used)
        assert val >= best * (1 - Fraction(1, 10**6)), (B, ch)


def test_stream_budget_dp_optimality(O):
    """n_seg = 24: exact dynamic programme over bytes (in 16-byte units) at the
    chosen total agrees with the choice's objective sum."""
    S = 64
    nb = _table9_bytes(O, S)
    units = [b // 16 for b in nb]
    rng = np.random.default_rng(12)
    n = 24
    J = (rng.random((n, 9)) ** 2).astype(np.float32)
    for frac in (0.2, 0.35, 0.6):
        B = int(frac * n * max(nb))
        ch, _ = O.stream_choose(J, nb, B)
        used = sum(nb[i] for i in ch)
        assert used <= B
        cap = used // 16
        dp = np.full(cap + 1, -np.inf)
        dp[0] = 0.0
        for k in range(n):
            nxt = np.full(cap + 1, -np.inf)
            for i in range(9):
                u = units[i]
                if u <= cap:
                    nxt[u:] = np.maximum(nxt[u:], dp[:cap + 1 - u] + float(J[k, i]))
            dp = nxt
        val = float(sum(float(J[k, i]) for k, i in enumerate(ch)))
        assert val >= dp.max() - 1e-6 * abs(dp.max()), (frac, val, dp.max())


def test_stream_budget_limits_and_monotone(O):
    """A budget covering every segment's best strategy keeps the per-segment
    argmax (multiplier 0); the smallest budget forces the smallest strategy;
    the objective sum never decreases as the budget grows."""
    S = 64
    nb = _table9_bytes(O, S)
    rng = np.random.default_rng(13)
    J = rng.random((10, 9)).astype(np.float32)
    best = J.argmax(axis=1)
    ch, u = O.stream_choose(J, nb, sum(nb[i] for i in best))
    assert u == 0 and list(ch) == list(best)
    small = int(np.argmin(nb))
    ch, _ = O.stream_choose(J, nb, 10 * nb[small])
    assert np.all(ch == small)
    prev = -1.0
    for B in range(10 * nb[small], 10 * max(nb) + 1, 4096):
        ch, _ = O.stream_choose(J, nb, B)
        v = float(sum(float(J[k, i]) for k, i in enumerate(ch)))
        assert v >= prev - 1e-6
        prev = v


def test_stream_budget_compress_end_to_end(O):
    """Stream scope in the compress path: bytes within n_seg * budget, the
    strategies are the Lagrangian choice over the reported objectives, and at
    least one segment exceeds the per-segment cap (the point of the mode)."""
    K, V, Qw = _small_stream(14, N=1024)
    S = 64
    budget = gen.budget_bytes(25, S)
    r = O.compress_stream(K, V, Qw, S=S, strategies=gen.table9(S), budget_bytes=budget,
                          scale=SCALE, budget_scope=1)
    nseg = 1024 // S
    assert r["used"] <= nseg * budget
    ch, _ = O.stream_choose(r["objective"], _table9_bytes(O, S), nseg * budget)
    assert list(r["desc"]["strategy"]) == list(ch)
    assert max(_table9_bytes(O, S)[i] for i in ch) > budget


# ---------------------------------------------------------------------------
# Incremental compression pipeline: the schedule written out from the reading

def test_pipeline_schedule_golden():
    """Hand-worked schedules (tests/golden/pipeline_schedule.json): firing
    steps, regions, the switched set of every step (lag, and the switch forced
    when a page is written again) and the tokens kept at full width."""
    from oracle import pipeline as OP
    with open(os.path.join(GOLDEN, "pipeline_schedule.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = OP.schedule(c["steps"], period=c["period"], protect=c["protect"], pages=c["pages"],
                          lag=c["lag"])
        assert [e["g"] for e in got] == c["g"]
        assert [e["fired"] for e in got] == c["fired"]
        assert [e["switched"] for e in got] == c["switched"]
        assert [list(got[-1]["regions"][i]) for i in range(len(c["regions"]))] == c["regions"]
        for i, want in c["tokens_at"].items():
            assert [list(r) for r in OP.state_tokens(got[int(i)])] == want


def test_pipeline_schedule_kara_counts():
    """The Kara configuration (8192 generated tokens, an event every 64, a
    64-token protected tail, 20 % of 64 = 13 tokens kept per event): 127
    events, and once every event is switched only the protected tail stays
    at full width, so a stream holds 16384 + 127 * 13 + 64 = 18099 tokens."""
    from oracle import pipeline as OP
    sched = OP.schedule([1] * 8192, period=64, protect=64, pages=4, lag=0)
    last = sched[-1]
    assert len(last["regions"]) == 127 and last["switched"] == list(range(127))
    assert last["regions"][0] == (0, 64) and last["regions"][126] == (8064, 8128)
    assert OP.state_tokens(last) == [(8128, 8192)]
    T = (20 * 64 + 50) // 100
    assert 16384 + 127 * T + sum(b - a for a, b in OP.state_tokens(last)) == 18099
    # every step sees each appended token exactly once: either in a switched
    # region or at full width
    for e in sched[::97]:
        seen = sum(b - a for a, b in OP.state_tokens(e)) + \
            sum(e["regions"][k][1] - e["regions"][k][0] for k in e["switched"])
        assert seen == e["g"]


def test_paged_descriptor_decode_pins(O):
    """A paged descriptor (parts sized for seg_tokens, first n_tok filled)
    decodes like the dense attention over its first n_tok rows (closed form
    in numpy), whatever the rows past n_tok hold; at n_tok == seg_tokens it
    is the keep-all descriptor of the same bytes."""
    rng = np.random.default_rng(3)
    cap, n = 16, 11
    K = rng.standard_normal((cap, 128)).astype(np.float32)
    V = rng.standard_normal((cap, 128)).astype(np.float32)
    q = rng.standard_normal((2, 128)).astype(np.float32)
    bf = lambda a: (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Kb, Vb, qb = bf(K), bf(V), bf(q)
    buf = np.full(512 * cap + 16, 0xFF, np.uint8)  # NaN past the filled rows
    buf[:256 * n] = Kb[:n].view(np.uint8).reshape(-1)
    buf[256 * cap:256 * cap + 256 * n] = Vb[:n].view(np.uint8).reshape(-1)
    desc = np.array([(0, n, 128, 0, 0x07, cap)], O.DESC_DTYPE)
    out, lse = O.decode_stream(qb, buf, desc, np.float32(0.125))
    up = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    l = up(qb) @ up(Kb[:n]).T * float(np.float32(0.125))
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    ref = (p / p.sum(axis=1, keepdims=True)) @ up(Vb[:n])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, m[:, 0] + np.log(p.sum(axis=1)), rtol=1e-12)
    full = np.zeros(512 * cap + 16, np.uint8)
    full[:256 * cap] = Kb.view(np.uint8).reshape(-1)
    full[256 * cap:512 * cap] = Vb.view(np.uint8).reshape(-1)
    a = O.decode_stream(qb, full, np.array([(0, cap, 128, 0, 0x07, cap)], O.DESC_DTYPE), np.float32(0.125))
    b = O.decode_stream(qb, full, np.array([(0, cap, 128, 0, 0x03, cap)], O.DESC_DTYPE), np.float32(0.125))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    s_paged = O.summarize_stream(buf, desc)
    s_dense = O.summarize_stream(full, np.array([(0, n, 128, 0, 0x03, n)], O.DESC_DTYPE))
    assert np.array_equal(s_paged, s_dense)


# ---------------------------------------------------------------------------
# SVD rotation before channel selection: Gram matrix, Jacobi, rotation

def _bf16(a):
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_gram_exact_on_integer_data(O):
    """Small integers make every product and partial sum exact in fp32, so
    the Gram matrix equals X^T X exactly and is symmetric."""
    rng = np.random.default_rng(11)
    X = rng.integers(-8, 9, size=(64, 128)).astype(np.float32)
    C = O.gram(_bf16(X))
    ref = X.astype(np.float64).T @ X.astype(np.float64)
    assert np.array_equal(C.astype(np.float64), ref)


def test_gram_is_a_chain_in_token_order(O):
    """Each Gram entry is one fma chain over the tokens in ascending order: a
    column (2^12, 1, 1, ..., 1) squares to 2^24 followed by 63 ones, and
    2^24 + 1 rounds back to 2^24 (ties to even), so the diagonal entry is
    exactly 2^24.  Summing the ones first (reversed order, or a pairwise
    tree) would give 2^24 + 64 (16777279 rounded).  The off-diagonal entry
    with a column of ones, 2^12 + 63, is exact in any order."""
    X = np.zeros((64, 128), np.float32)
    X[:, 5] = 1.0
    X[0, 5] = 4096.0
    X[:, 9] = 1.0
    C = O.gram(_bf16(X))
    assert C[5, 5] == np.float32(2.0 ** 24)
    assert C[5, 9] == C[9, 5] == np.float32(4096 + 63)
    assert C[9, 9] == np.float32(64.0)
    Cr = O.gram(_bf16(X[::-1]))
    assert Cr[5, 5] == np.float32(16777280.0)


def test_jacobi_against_numpy_eigh(O):
    """Eigenvalues within 1e-4 of the largest of numpy's fp64 eigh, sorted
    largest first; R orthogonal; R^T C R diagonal to 1e-5 of the largest."""
    rng = np.random.default_rng(12)
    X = rng.standard_normal((512, 128)).astype(np.float32)
    X[:, 3] *= 10.0  # an outlier channel
    C = O.gram(_bf16(X))
    R, ev = O.jacobi(C)
    w = np.linalg.eigvalsh(C.astype(np.float64))[::-1]
    assert np.all(np.diff(ev) <= 0)
    assert np.abs(ev - w).max() <= 1e-4 * w[0]
    Rd = R.astype(np.float64)
    assert np.abs(Rd.T @ Rd - np.eye(128)).max() <= 1e-4
    D = Rd.T @ C.astype(np.float64) @ Rd
    assert np.abs(D - np.diag(np.diag(D))).max() <= 1e-5 * w[0]


def test_jacobi_planted_spectrum(O):
    """C = Q diag(lambda) Q^T with well-separated planted eigenvalues: the
    eigenvalues come back within the error of a backward-stable fp32 method,
    a small multiple of n eps ||C|| = 128 * 2^-24 * 100 = 7.6e-4 (5e-3, i.e.
    5e-5 of the largest, is allowed), and each eigenvector matches its
    planted column up to sign."""
    rng = np.random.default_rng(13)
    Q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    lam = 100.0 * 0.93 ** np.arange(128)
    C = ((Q * lam) @ Q.T).astype(np.float32)
    C = (C + C.T) / 2
    R, ev = O.jacobi(C)
    assert np.abs(ev - lam).max() <= 5e-5 * lam[0]
    dots = np.abs(np.sum(R.astype(np.float64) * Q, axis=0))
    assert dots[:32].min() > 0.999


def test_jacobi_diagonal_input_is_a_sort(O):
    """A diagonal C needs no rotation (every A[p][q] is 0): R is the
    permutation that sorts the diagonal largest first, ties to the lower
    index, exactly."""
    d = np.array([(i * 37) % 11 for i in range(128)], np.float32)
    R, ev = O.jacobi(np.diag(d))
    order = sorted(range(128), key=lambda i: (-d[i], i))
    assert np.array_equal(ev, d[order])
    P = np.zeros((128, 128), np.float32)
    P[order, np.arange(128)] = 1.0
    assert np.array_equal(R, P)


def test_rotate_identity_and_permutation(O):
    rng = np.random.default_rng(14)
    X = _bf16(rng.standard_normal((40, 128)))
    assert np.array_equal(O.rotate(X, np.eye(128, dtype=np.float32)), X)
    perm = rng.permutation(128)
    P = np.zeros((128, 128), np.float32)
    P[perm, np.arange(128)] = 1.0  # column k selects channel perm[k]
    assert np.array_equal(O.rotate(X, P), X[:, perm])


def test_rotation_concentrates_energy(O):
    """[M] Fig. 4: after the rotation a vector's largest elements hold more of
    its energy.  Vectors with rank-8 structure in a random basis plus small
    noise spread their energy over all channels; rotated, it sits in about
    eight, so the share kept at 32 of 128 channels rises from about a half
    to nearly all, for every vector.  (On the synthetic workloads, whose
    outlier channels are already axis-aligned, the gain is small.)"""
    rng = np.random.default_rng(17)
    X = rng.standard_normal((512, 8)) @ rng.standard_normal((8, 128)) + \
        0.05 * rng.standard_normal((512, 128))
    Xb = _bf16(X)
    R, ev = O.jacobi(O.gram(Xb))
    assert ev[:8].sum() > 0.99 * ev.sum()
    Y = O.rotate(Xb, R)
    before = np.array([O.channel_topc(Xb[t], 32)[1] for t in range(0, 512, 4)])
    after = np.array([O.channel_topc(Y[t], 32)[1] for t in range(0, 512, 4)])
    assert before.mean() < 0.8 and after.min() > 0.99


def test_rotated_decode_pins(O):
    """Decode over a rotated cache: identity matrices give the plain decode
    exactly; permutation matrices (rotations without rounding) applied to
    a keep-all cache give dense attention over the original vectors."""
    rng = np.random.default_rng(15)
    S, T = 64, 64
    K = _bf16(rng.standard_normal((T, 128)))
    V = _bf16(rng.standard_normal((T, 128)))
    q = _bf16(rng.standard_normal((4, 128)))
    r = O.compress_stream(K, V, np.zeros((4, 1, 128), np.uint16), S=S, strategies=[(S, 128)],
                          budget_bytes=4 * S * 128, scale=np.float32(0.125))
    I = np.eye(128, dtype=np.float32)
    a = O.decode_stream(q, r["packed"], r["desc"], np.float32(0.125))
    b = O.decode_stream_rot(q, r["packed"], r["desc"], np.float32(0.125), np.stack([I, I]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    pk, pv = rng.permutation(128), rng.permutation(128)
    PK = np.zeros((128, 128), np.float32)
    PK[pk, np.arange(128)] = 1.0
    PV = np.zeros((128, 128), np.float32)
    PV[pv, np.arange(128)] = 1.0
    rp = O.compress_stream(K[:, pk], V[:, pv], np.zeros((4, 1, 128), np.uint16), S=S,
                           strategies=[(S, 128)], budget_bytes=4 * S * 128, scale=np.float32(0.125))
    o, l = O.decode_stream_rot(q, rp["packed"], rp["desc"], np.float32(0.125), np.stack([PK, PV]))
    Kf, Vf, qf = _f32(K).astype(np.float64), _f32(V).astype(np.float64), _f32(q).astype(np.float64)
    lg = qf @ Kf.T * 0.125
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    ref = (p / p.sum(axis=1, keepdims=True)) @ Vf
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(l, m[:, 0] + np.log(p.sum(axis=1)), rtol=1e-12)


def test_compress_with_rotation_stores_rotated_vectors(O):
    """Keep-all compression with rotation stores R^T x of every region vector
    (the rotation of the oracle's own Jacobi of the region's Gram matrix),
    and returns that R; decode over it stays within the bf16 rounding of the
    rotated vectors of dense attention over the original vectors."""
    rng = np.random.default_rng(16)
    S, N = 64, 256
    K = _bf16(rng.standard_normal((N, 128)))
    V = _bf16(rng.standard_normal((N, 128)))
    q = _bf16(rng.standard_normal((2, 128)))
    r = O.compress_stream(K, V, np.zeros((2, 1, 128), np.uint16), S=S, strategies=[(S, 128)],
                          budget_bytes=4 * S * 128, scale=np.float32(0.125), rotate=True)
    RK, _ = O.jacobi(O.gram(K))
    RV, _ = O.jacobi(O.gram(V))
    assert r["rot"].shape == (1, 2, 128, 128)
    assert np.array_equal(r["rot"][0, 0], RK) and np.array_equal(r["rot"][0, 1], RV)
    seg = 2 * S * 256
    YK, YV = O.rotate(K, RK), O.rotate(V, RV)
    for sg in range(N // S):
        blk = r["packed"][sg * seg:(sg + 1) * seg]
        assert np.array_equal(blk[:S * 256].view(np.uint16).reshape(S, 128), YK[sg * S:(sg + 1) * S])
        assert np.array_equal(blk[S * 256:].view(np.uint16).reshape(S, 128), YV[sg * S:(sg + 1) * S])
    o, l = O.decode_stream_rot(q, r["packed"], r["desc"], np.float32(0.125), r["rot"])
    Kf, Vf, qf = _f32(K).astype(np.float64), _f32(V).astype(np.float64), _f32(q).astype(np.float64)
    lg = qf @ Kf.T * 0.125
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ Vf
    assert np.abs(o - ref).max() <= 2e-2 * np.linalg.norm(ref, axis=1).max()


def test_rotation_per_span(O):
    """With rot_span, every span of the region has its own R_K and R_V: R of
    span j is the Jacobi rotation of span j's own Gram matrix, the span's
    vectors are stored rotated by it, and the rotations of different spans
    differ when their vectors do."""
    rng = np.random.default_rng(18)
    S, N, span = 64, 256, 128
    K = _bf16(rng.standard_normal((N, 128)) * np.repeat(rng.uniform(0.5, 4.0, (N // span, 128)), span, 0))
    V = _bf16(rng.standard_normal((N, 128)))
    r = O.compress_stream(K, V, np.zeros((2, 1, 128), np.uint16), S=S, strategies=[(S, 128)],
                          budget_bytes=4 * S * 128, scale=np.float32(0.125), rotate=True,
                          rot_span=span)
    assert r["rot"].shape == (N // span, 2, 128, 128)
    seg = 2 * S * 256
    for j in range(N // span):
        Ks, Vs = K[j * span:(j + 1) * span], V[j * span:(j + 1) * span]
        RK, _ = O.jacobi(O.gram(Ks))
        RV, _ = O.jacobi(O.gram(Vs))
        assert np.array_equal(r["rot"][j, 0], RK) and np.array_equal(r["rot"][j, 1], RV)
        YK, YV = O.rotate(Ks, RK), O.rotate(Vs, RV)
        for sg in range(span // S):
            g = j * (span // S) + sg
            blk = r["packed"][g * seg:(g + 1) * seg]
            assert np.array_equal(blk[:S * 256].view(np.uint16).reshape(S, 128), YK[sg * S:(sg + 1) * S])
            assert np.array_equal(blk[S * 256:].view(np.uint16).reshape(S, 128), YV[sg * S:(sg + 1) * S])
    assert not np.array_equal(r["rot"][0, 0], r["rot"][1, 0])


def test_rotated_decode_per_span_permutations(O):
    """Decode over spans with their own rotations: a keep-all cache whose
    span j holds K and V with its own channel permutation, decoded with
    those permutation matrices, equals dense attention over the original
    vectors (a span taking another span's matrices would not); identity
    matrices in every span give the plain decode exactly."""
    rng = np.random.default_rng(19)
    S, N, dps = 32, 128, 2  # four segments, two spans of two segments
    K = _bf16(rng.standard_normal((N, 128)))
    V = _bf16(rng.standard_normal((N, 128)))
    q = _bf16(rng.standard_normal((3, 128)))
    span = S * dps
    rot = np.zeros((N // span, 2, 128, 128), np.float32)
    Kp, Vp = K.copy(), V.copy()
    for j in range(N // span):
        for side, (X, Xp) in enumerate(((K, Kp), (V, Vp))):
            perm = rng.permutation(128)
            rot[j, side][perm, np.arange(128)] = 1.0
            Xp[j * span:(j + 1) * span] = X[j * span:(j + 1) * span][:, perm]
    r = O.compress_stream(Kp, Vp, np.zeros((3, 1, 128), np.uint16), S=S, strategies=[(S, 128)],
                          budget_bytes=4 * S * 128, scale=np.float32(0.125))
    o, l = O.decode_stream_rot(q, r["packed"], r["desc"], np.float32(0.125), rot, dps)
    Kf, Vf, qf = _f32(K).astype(np.float64), _f32(V).astype(np.float64), _f32(q).astype(np.float64)
    lg = qf @ Kf.T * 0.125
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    ref = (p / p.sum(axis=1, keepdims=True)) @ Vf
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(l, m[:, 0] + np.log(p.sum(axis=1)), rtol=1e-12)
    swapped = O.decode_stream_rot(q, r["packed"], r["desc"], np.float32(0.125), rot[::-1], dps)[0]
    assert not np.allclose(swapped, ref, rtol=1e-6, atol=1e-6)
    I = np.eye(128, dtype=np.float32)
    eye = np.broadcast_to(I, (N // span, 2, 128, 128))
    a = O.decode_stream(q, r["packed"], r["desc"], np.float32(0.125))
    b = O.decode_stream_rot(q, r["packed"], r["desc"], np.float32(0.125), eye, dps)
    assert np.allclose(a[0], b[0], rtol=1e-13, atol=1e-13) and np.array_equal(a[1], b[1])
