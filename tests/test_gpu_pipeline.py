"""GPU parity of the incremental compression pipeline (kv_append, paged
descriptors, kv_pipe_*) against the CPU oracle.

  * kv_append: page bytes and descriptors bit-exact against a host copy;
  * decode and summaries over paged descriptors (bytes past n_tok hold NaN)
    against the oracle over the same buffer;
  * the Kara generation loop through the pipeline: after every step the
    decode list's switched events are read back; in the deterministic modes
    they must equal the schedule the oracle prescribes, in the asynchronous
    mode they must be an admissible state (a prefix of the fired events that
    holds every event whose page was needed again); every step's decode
    output is checked against the oracle's decode over exactly that state;
    every final segment is bit-exact against the oracle's compression of its
    event.
"""
import numpy as np
import pytest
import torch

from compressed_kv_cache_compress_amd import (DESC_DTYPE, PIPE_ASYNC, PIPE_LAG, PIPE_SYNC, KvParams,
                                              gen, kara, kv_append, runtime)
from helpers import (SCALE, PipelineOracle, assemble_cache, check_attention, check_pipeline_finals,
                     check_pipeline_pages, desc_to_dev, oracle_compress_all, run_pipeline, say,
                     switched_from_list, to_dev_u8)
from oracle import oracle as O
from oracle import pipeline as OP

pytestmark = pytest.mark.gpu

D = 128


def _rows(a):
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def test_append_bitexact():
    """Three appends (1, 5 and 10 tokens) into 16-token pages of 6 streams
    (stream stride of the sources larger than the tokens); every byte of the
    buffer and of the descriptor list checked."""
    B, Hkv, cap = 2, 3, 16
    streams = B * Hkv
    src_len = 40
    g = torch.Generator().manual_seed(5)
    K = torch.randn((B, Hkv, src_len, D), generator=g).to(torch.bfloat16).cuda()
    V = torch.randn((B, Hkv, src_len, D), generator=g).to(torch.bfloat16).cuda()
    pstride = 3 * cap * 512 + 48
    page_off = 1040
    packed = torch.full((streams * pstride + page_off + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    dstride = 5
    desc = torch.full((streams * dstride * 16,), 0x5A, dtype=torch.uint8, device="cuda")
    p = KvParams(batch=B, n_q_heads=Hkv, n_kv_heads=Hkv, kv_stream_stride=src_len * D)
    p.p.packed_stream_stride = pstride
    p.p.desc_stream_stride = dstride
    exp_buf = packed.cpu().numpy().copy()
    Kh, Vh = gen.u16(K), gen.u16(V)
    fill, pos = 0, 0
    for n in (1, 5, 10):
        say(f"[append] fill={fill} n_new={n}")
        kv_append(p, K[:, :, pos:], V[:, :, pos:], n, fill, cap, page_off, packed, desc[16:])
        for s in range(streams):
            b, h = divmod(s, Hkv)
            base = page_off + s * pstride
            for t in range(n):
                r = fill + t
                exp_buf[base + r * 256: base + (r + 1) * 256] = _rows(Kh[b, h, pos + t])
                exp_buf[base + cap * 256 + r * 256: base + cap * 256 + (r + 1) * 256] = \
                    _rows(Vh[b, h, pos + t])
        fill += n
        pos += n
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), exp_buf)
    dh = desc.cpu().numpy().reshape(streams, dstride, 16)
    for s in range(streams):
        d = dh[s, 1].view(DESC_DTYPE)[0]
        assert int(d["offset"]) == page_off + s * pstride
        assert (int(d["n_tok"]), int(d["n_ch"]), int(d["strategy"])) == (fill, 128, 0)
        assert int(d["flags"]) == 0x07 and int(d["seg_tokens"]) == cap
        for j in (0, 2, 3, 4):
            assert np.all(dh[s, j] == 0x5A)


def _paged_cache(w, S, caps, fills, seed=1):
    """Oracle-compressed segments of every stream followed by dense paged
    segments (capacities `caps`, first `fills` rows filled, the rest 0xFF
    bytes, i.e. NaN), all in one host buffer."""
    streams = w["B"] * w["Hkv"]
    strat = gen.table9(S)
    seg_cap = (w["N"] // S) * max(O.seg_bytes(t, c, S) for t, c in strat)
    page_total = sum(512 * c for c in caps)
    cap = (seg_cap + page_total + 255) // 256 * 256
    res = oracle_compress_all(w, S=S, strategies=strat, budget=gen.budget_bytes(33, S),
                              capacity=cap)
    buf, descs = assemble_cache(res, cap)
    rng = np.random.default_rng(seed)
    pages = np.zeros((streams, len(caps)), DESC_DTYPE)
    for s in range(streams):
        off = s * cap + seg_cap
        for j, (c, f) in enumerate(zip(caps, fills)):
            rowsK = rng.standard_normal((f, D)).astype(np.float32)
            rowsV = rng.standard_normal((f, D)).astype(np.float32)
            kb = gen.u16(torch.from_numpy(rowsK).to(torch.bfloat16))
            vb = gen.u16(torch.from_numpy(rowsV).to(torch.bfloat16))
            buf[off:off + 512 * c] = 0xFF
            buf[off:off + 256 * f] = _rows(kb)
            buf[off + 256 * c:off + 256 * c + 256 * f] = _rows(vb)
            pages[s, j] = (off, f, 128, 0, 0x07, c)
            off += 512 * c
    return buf, np.concatenate([descs, pages], axis=1)


def test_decode_and_summaries_over_paged_descriptors():
    w = gen.make_workload("batched128k", B=1, N=1024)
    caps = [16, 32, 64, 256, 16]
    fills = [1, 31, 64, 5, 16]
    buf, descs = _paged_cache(w, 64, caps, fills)
    say(f"[paged] streams={descs.shape[0]} maxd={descs.shape[1]}")
    out, lse = runtime.decode(w["q"].cuda(), to_dev_u8(buf), desc_to_dev(descs),
                              n_kv_heads=w["Hkv"], max_desc_per_stream=descs.shape[1],
                              scale=float(SCALE))
    sm = runtime.summarize(to_dev_u8(buf), desc_to_dev(descs), batch=1, n_q_heads=w["Hq"],
                           n_kv_heads=w["Hkv"], max_desc_per_stream=descs.shape[1])
    torch.cuda.synchronize()
    qn = gen.u16(w["q"])
    G = w["G"]
    smh = sm.cpu().numpy().view(np.uint16)
    for s in range(descs.shape[0]):
        ro, rl = O.decode_stream(qn[0, s * G:(s + 1) * G], buf, descs[s], SCALE)
        check_attention(out[0, s * G:(s + 1) * G], lse[0, s * G:(s + 1) * G], ro, rl, f"paged s={s}")
        assert np.array_equal(smh[s], O.summarize_stream(buf, descs[s])), f"summary s={s}"


# ---------------------------------------------------------------- pipeline

SMALL = dict(B=1, prompt=256, gen=512, window=128, delta=32, protect=32, prompt_seg=64,
             retention_pct=20, alpha=1, gamma=8)


def _make(mode, lag=0, pages=None, start=0, steps=None, seed=0, event_max_waves=0, **over):
    c = dict(SMALL)
    c.update(over)
    w = gen.make_kara(seed=seed, device="cuda", B=c["B"], prompt=c["prompt"], gen=c["gen"])
    kp = kara.KaraPipeline(w["K"], w["V"], w["Qall"], prompt=c["prompt"], start=start,
                           window=c["window"], delta=c["delta"], protect=c["protect"],
                           retention_pct=c["retention_pct"], alpha=c["alpha"], gamma=c["gamma"],
                           prompt_seg=c["prompt_seg"], scale=float(SCALE), mode=mode,
                           switch_lag=lag, pages=pages, steps=steps,
                           event_max_waves=event_max_waves)
    return w, kp, c


@pytest.mark.parametrize("mode,lag", [(PIPE_SYNC, 0), (PIPE_LAG, 0), (PIPE_LAG, 1), (PIPE_LAG, 57)])
def test_pipeline_deterministic_modes(mode, lag):
    w, kp, c = _make(mode, lag=lag, pages=4)
    streams = kp.B * kp.Hkv
    n = c["gen"]
    say(f"[pipeline] mode={mode} lag={lag} steps={n} streams={streams}")
    outs, lists = run_pipeline(kp, n)
    kp.pipe.drain()
    torch.cuda.synchronize()
    st = kp.pipe.stats()
    entries = OP.schedule([1] * n, period=c["delta"], protect=c["protect"], pages=4, lag=lag)
    assert st["events_fired"] == len(entries[-1]["regions"]) == n // c["delta"] - 1
    assert st["events_switched"] == st["events_fired"] and st["host_waits"] == 0
    oe = PipelineOracle(w, kp, c)
    check_all = set(range(0, n, 37)) | {n - 1} | \
        {i for i, e in enumerate(entries) if e["fired"] is not None}
    for i, entry in enumerate(entries):
        sw, d = switched_from_list(kp, lists[i], streams)
        assert sw == entry["switched"], (i, sw, entry["switched"])
        check_pipeline_pages(kp, d, entry, sw, streams)
        ss = range(streams) if i in check_all else (0, streams - 1)
        out, lse = outs[i]
        G = kp.Hq // kp.Hkv
        for s in ss:
            b, h = divmod(s, kp.Hkv)
            ro, rl = oe.state_decode(s, entry, sw)
            check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                            f"step {i} s={s}")
    check_pipeline_finals(kp, oe, entries, streams)
    kp.close()


@pytest.mark.parametrize("cap", [0, 64])
def test_pipeline_async_states_are_admissible(cap):
    """The asynchronous mode (event kernels uncapped, or capped at 64 waves in
    flight): each step's list is a prefix of the fired events that includes
    every event whose page was written again; outputs match the oracle over
    that exact state; after drain the finals equal the oracle's."""
    w, kp, c = _make(PIPE_ASYNC, pages=3, event_max_waves=cap)
    streams = kp.B * kp.Hkv
    n = c["gen"]
    say(f"[pipeline] async steps={n} streams={streams}")
    outs, lists = run_pipeline(kp, n)
    kp.pipe.drain()
    torch.cuda.synchronize()
    st = kp.pipe.stats()
    say(f"  stats {st}")
    forced = OP.schedule([1] * n, period=c["delta"], protect=c["protect"], pages=3, lag=10 ** 9)
    oe = PipelineOracle(w, kp, c)
    G = kp.Hq // kp.Hkv
    for i, entry in enumerate(forced):
        sw, d = switched_from_list(kp, lists[i], streams)
        fired = [e for e in entry["regions"]]
        assert sw == fired[:len(sw)], (i, sw)
        assert set(entry["switched"]) <= set(sw), (i, sw, entry["switched"])
        check_pipeline_pages(kp, d, entry, sw, streams)
        if i % 29 == 0 or i == n - 1:
            out, lse = outs[i]
            for s in (0, streams - 1):
                b, h = divmod(s, kp.Hkv)
                ro, rl = oe.state_decode(s, entry, sw)
                check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                                f"async step {i} s={s}")
    assert st["events_switched"] == st["events_fired"] == n // c["delta"] - 1
    check_pipeline_finals(kp, oe, forced, streams)
    kp.close()


def test_pipeline_resume_with_prefill_and_prefix_events():
    """A pipeline started after 128 generated tokens: the events of those
    tokens are compressed up front (prefix), the protected tail is appended
    in one multi-token step without decode, then single-token steps; lag
    mode checked step by step."""
    start = 128
    w, kp, c = _make(PIPE_LAG, lag=3, pages=4, start=start - 32, steps=512 - start + 32)
    streams = kp.B * kp.Hkv
    n = c["gen"] - start
    say(f"[pipeline] resume prefix_events={kp.n_prefix_events} steps={n}")
    outs, lists = run_pipeline(kp, n, prefill=c["protect"])
    kp.pipe.drain()
    torch.cuda.synchronize()
    entries = OP.schedule([c["protect"]] + [1] * n, period=c["delta"], protect=c["protect"],
                          pages=4, lag=3)[1:]
    oe = PipelineOracle(w, kp, c)
    G = kp.Hq // kp.Hkv
    # the prefix: prompt dense + the events of generated tokens [0, start - 32)
    assert kp.n_prefix_events == (start - 32) // c["delta"]
    for i, entry in enumerate(entries):
        sw, d = switched_from_list(kp, lists[i], streams)
        assert sw == entry["switched"], (i, sw, entry["switched"])
        check_pipeline_pages(kp, d, entry, sw, streams)
    # decode at sampled steps, against an oracle state that includes the prefix events
    for i in (0, 40, n - 1):
        entry = entries[i]
        out, lse = outs[i]
        for s_ in (0, streams - 1):
            b, h = divmod(s_, kp.Hkv)
            ro, rl = oe.state_decode(s_, entry, entry["switched"])
            check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                            f"resume step {i} s={s_}")
    check_pipeline_finals(kp, oe, entries, streams)
    kp.close()


def test_pipeline_rejects_before_enqueue():
    """Errors of kv_pipe_step are raised before anything is enqueued and
    leave the pipeline unchanged: a due event without its window, a step
    that would cross a page, event slots used up; the run then continues
    and matches the deterministic schedule."""
    import ctypes
    from compressed_kv_cache_compress_amd import KvcError, lib
    w, kp, c = _make(PIPE_LAG, lag=0, pages=4, steps=96)
    streams = kp.B * kp.Hkv
    D_ = 128
    K, V = w["K"], w["V"]
    # 63 single-token steps: no event yet (the first fires at token 64)
    for _ in range(63):
        kp.step(1, decode=False)
    p0 = kp.length
    with pytest.raises(KvcError) as e:     # event due, no window
        kp.pipe.step(K[:, :, p0:], V[:, :, p0:], 1, kp.L * D_)
    assert e.value.status == -1
    with pytest.raises(KvcError) as e:     # 2 tokens would cross into the next page
        kp.pipe.step(K[:, :, p0:], V[:, :, p0:], 2, kp.L * D_)
    assert e.value.status == -1
    st = kp.pipe.stats()
    assert (st["steps"], st["tokens"], st["events_fired"]) == (63, 63, 0)
    bad = ctypes.c_void_p(1)               # a different stream handle
    assert lib().kv_pipe_step(kp.pipe.h, ctypes.c_void_p(K.data_ptr()),
                              ctypes.c_void_p(V.data_ptr()), 1, kp.L * D_, None, None, None, None,
                              None, None, bad) == -1
    assert lib().kv_pipe_drain(kp.pipe.h, bad) == -1
    kp.step(1, decode=False)               # fires event 0 with its window
    for _ in range(32):
        kp.step(1, decode=False)           # fires event 1 at token 96
    st = kp.pipe.stats()
    assert (st["steps"], st["tokens"], st["events_fired"], st["events_switched"]) == (96, 96, 2, 2)
    torch.cuda.synchronize()
    kp.close()


def test_pipeline_event_slots_used_up():
    """A pipeline sized for 2 events refuses the third before enqueueing."""
    from compressed_kv_cache_compress_amd import KvcError
    w, kp, c = _make(PIPE_LAG, lag=0, pages=4, steps=96)
    assert kp.cfg.max_events == 2
    for _ in range(127):
        kp.step(1, decode=False)
    assert kp.pipe.stats()["events_fired"] == 2
    p0 = kp.length
    wk = w["K"][:, :, p0 + 1 - c["window"]:]
    wv = w["V"][:, :, p0 + 1 - c["window"]:]
    wq = w["Qall"][:, :, p0 + 1 - c["window"]:]
    with pytest.raises(KvcError) as e:     # the third event has no slot
        kp.pipe.step(w["K"][:, :, p0:], w["V"][:, :, p0:], 1, kp.L * 128, wk, wv, wq)
    assert e.value.status == -1
    assert kp.pipe.stats()["tokens"] == 127
    kp.pipe.drain()
    torch.cuda.synchronize()
    kp.close()
