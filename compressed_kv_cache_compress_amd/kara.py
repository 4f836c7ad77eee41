"""Kara-style sliding-window compression events over a paged decode cache.

KARA review page (arXiv 2607.01237): "What carries the argument" -- only the
recent window is scored (bidirectional attention accumulated from all window
queries) and the selected tokens are expanded into chunks (Token2Chunk);
free-parameter ledger -- retention r, window |W|, protected buffer |U|, chunk
budget alpha, max chunk length gamma, compression period delta.

Reading used here (one stream = one batch entry x one kv head):
  * the prompt stays dense; only generated tokens are compressed;
  * every delta generated tokens, at sequence length L, the window is the last
    `window` positions (their original K and queries), the region is the `seg`
    tokens just before the protected tail of `protect` tokens, and T =
    round(r * seg) tokens of it are kept with all 128 channels (Token2Chunk
    with alpha, gamma); events whose region lies in the prompt are skipped;
  * the final cache of a stream is [dense prompt segments][one compressed
    segment per event][dense tail], each a descriptor into one buffer.

Everything below only arranges buffers and calls the C ABI; all arithmetic
runs in libkvc's kernels.
"""
import torch

from . import (PIPE_ASYNC, KvParams, KvPipe, kv_compress, kv_layout_query, kv_pipe_layout,
               pipe_config)

D = 128


def event_schedule(prompt, generated, *, window, delta, protect, seg, retention_pct):
    """Compression events of a Kara run, in firing order (the reading in the
    module docstring).  Event k fires at length L = prompt + delta * k; its
    region [L - protect - seg, L - protect) starts at or after the prompt
    exactly when delta * k >= protect + seg, so the first event is k0 =
    ceil((protect + seg) / delta) and the last k = generated div delta.
    Returns ([(L, window start, region start inside the window)], T) with T =
    round(r * seg) half up."""
    T = (retention_pct * seg + 50) // 100
    k0 = -(-(protect + seg) // delta)
    rb = window - protect - seg
    assert rb >= 0, "the window must hold the region and the protected tail"
    return [(prompt + delta * k, prompt + delta * k - window, rb)
            for k in range(k0, generated // delta + 1)], T


def _seg_bytes_keep_all(tokens):
    return tokens * 4 * D


class KaraCache:
    """Device buffers of an assembled cache: packed bytes, descriptors
    [streams][max_desc] (16 bytes each), and the per-stream layout."""

    def __init__(self, packed, desc, max_desc, stream_bytes, n_events, T, layout):
        self.packed, self.desc, self.max_desc = packed, desc, max_desc
        self.stream_bytes, self.n_events, self.T, self.layout = stream_bytes, n_events, T, layout


def build_cache(K, V, Qall, *, prompt, gen, window=512, delta=64, protect=64, seg=64,
                retention_pct=20, alpha=3, gamma=16, prompt_seg=256, scale=0.0, events=None):
    """K, V: [B, Hkv, L, 128] bf16; Qall: [B, Hq, L, 128] bf16 (queries at every
    position), L = prompt + gen, all on the GPU.  `events` optionally limits
    the events run (a list of indices into the schedule).  Returns KaraCache."""
    B, Hkv, L = K.shape[0], K.shape[1], K.shape[2]
    Hq = Qall.shape[1]
    assert L == prompt + gen and K.is_contiguous() and V.is_contiguous() and Qall.is_contiguous()
    sched, T = event_schedule(prompt, gen, window=window, delta=delta, protect=protect, seg=seg,
                              retention_pct=retention_pct)
    if events is not None:
        sched = [sched[i] for i in events]
    n_ev = len(sched)
    tail0 = L - protect
    n_prompt_desc = prompt // prompt_seg
    max_desc = n_prompt_desc + n_ev + 1
    # per-stream slot: dense prompt, event segments, dense tail
    p_ev = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=window, region_begin=window - protect - seg,
                    region_len=seg, seg_tokens=seg, n_win=window, strategies=[(T, D)],
                    budget_bytes=4 * seg * D, t2c_alpha=alpha, t2c_gamma=gamma, scale=scale,
                    kv_stream_stride=L * D, qw_head_stride=L * D, store_logits=1)
    _, lev = kv_layout_query(p_ev)
    ev_bytes = lev.seg_bytes[0]
    prompt_bytes = _seg_bytes_keep_all(prompt)
    tail_bytes = _seg_bytes_keep_all(protect)
    stream_bytes = (prompt_bytes + n_ev * ev_bytes + tail_bytes + 255) // 256 * 256
    dev = K.device
    streams = B * Hkv
    packed = torch.empty(streams * stream_bytes, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * max_desc * 16, dtype=torch.uint8, device=dev)
    desc_row = max_desc * 16

    def run(params, Kv, Vv, Qv, base_off, desc_first):
        _, lay = kv_layout_query(params)
        ws = torch.empty(max(int(lay.compress_ws_bytes), 16), dtype=torch.uint8, device=dev)
        params.p.packed_stream_stride = stream_bytes
        params.p.packed_base_offset = base_off
        params.p.desc_stream_stride = max_desc
        kv_compress(params, Kv, Vv, Qv, None, packed[base_off:], desc[desc_first * 16:], None, None,
                    None, ws)

    # dense prompt: keep-all segments of prompt_seg tokens (no scoring)
    pp = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=prompt, seg_tokens=prompt_seg,
                  strategies=[(prompt_seg, D)], budget_bytes=4 * prompt_seg * D, scale=scale,
                  kv_stream_stride=L * D)
    run(pp, K, V, None, 0, 0)
    # compression events
    for e, (Le, w0, rb) in enumerate(sched):
        run(p_ev, K[:, :, w0:], V[:, :, w0:], Qall[:, :, w0:], prompt_bytes + e * ev_bytes,
            n_prompt_desc + e)
    # dense protected tail
    pt = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=protect, seg_tokens=protect,
                  strategies=[(protect, D)], budget_bytes=4 * protect * D, scale=scale,
                  kv_stream_stride=L * D)
    run(pt, K[:, :, tail0:], V[:, :, tail0:], None, prompt_bytes + n_ev * ev_bytes,
        n_prompt_desc + n_ev)
    return KaraCache(packed, desc, max_desc, stream_bytes, n_ev, T,
                     dict(prompt_bytes=prompt_bytes, ev_bytes=ev_bytes, tail_bytes=tail_bytes,
                          n_prompt_desc=n_prompt_desc, schedule=sched, desc_row=desc_row))


class KaraPipeline:
    """The Kara generation loop through the compression pipeline (kv_pipe_*):
    the prompt stays dense (keep-all segments of `prompt_seg` tokens), the
    events of the first `start` generated tokens are compressed up front
    (`start` a multiple of delta), and every later generated token is one
    step: appended to a dense page, decoded with its own query, and every
    `delta` tokens the page `protect` tokens back is compressed on the
    pipeline's stream and switched in (when, depends on `mode`).
    event_max_waves caps the waves an event's compression keeps in flight, so
    that a background event leaves most of the GPU to decode.

    K, V: [B, Hkv, L, 128], Qall: [B, Hq, L, 128] on the GPU (L = prompt +
    generated); they are the full-resolution source of new tokens and of the
    scoring windows and must stay unchanged while the pipeline runs.
    """

    def __init__(self, K, V, Qall, *, prompt, start=0, window=512, delta=64, protect=64,
                 retention_pct=20, alpha=3, gamma=16, prompt_seg=256, scale=0.0, mode=PIPE_ASYNC,
                 switch_lag=0, pages=None, steps=None, decode_splits=0, event_max_waves=0):
        B, Hkv, L = K.shape[0], K.shape[1], K.shape[2]
        Hq = Qall.shape[1]
        assert K.is_contiguous() and V.is_contiguous() and Qall.is_contiguous()
        assert start % delta == 0 and protect % delta == 0 and prompt % prompt_seg == 0
        gen = L - prompt
        self.B, self.Hq, self.Hkv, self.L, self.prompt = B, Hq, Hkv, L, prompt
        self.K, self.V, self.Qall = K, V, Qall
        self.window, self.delta, self.protect = window, delta, protect
        # prefix: events whose region ends by generated token `start`
        sched, T = event_schedule(prompt, gen, window=window, delta=delta, protect=protect,
                                  seg=delta, retention_pct=retention_pct)
        pre = [e for e in sched if e[0] - protect <= prompt + start]
        self.T = T
        n_steps = gen - start if steps is None else steps
        self.g0 = start  # generated index of the pipeline's first token
        # events the pipeline fires over its steps (local count g >= protect + delta)
        n_ev = max(0, (n_steps // delta) - protect // delta)
        pages = pages or (protect // delta + 3)
        n_prompt_desc = prompt // prompt_seg
        self.ev_params = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=window,
                                  region_begin=window - protect - delta, region_len=delta,
                                  seg_tokens=delta, n_win=window, strategies=[(T, D)],
                                  budget_bytes=4 * delta * D, t2c_alpha=alpha, t2c_gamma=gamma,
                                  scale=scale, kv_stream_stride=L * D, qw_head_stride=L * D,
                                  decode_splits=decode_splits, compress_max_waves=event_max_waves,
                                  store_logits=1)
        _, lev = kv_layout_query(self.ev_params)
        ev_bytes = (lev.seg_bytes[0] + 15) // 16 * 16
        prompt_bytes = _seg_bytes_keep_all(prompt)
        events_offset = prompt_bytes + len(pre) * ev_bytes
        self.cfg = pipe_config(mode=mode, switch_lag=switch_lag, pages=pages,
                               max_events=max(1, n_ev), prefix_desc=n_prompt_desc + len(pre),
                               protect=protect, events_offset=events_offset,
                               pages_offset=events_offset + max(1, n_ev) * ev_bytes)
        _, pl = kv_pipe_layout(self.ev_params, self.cfg)
        assert pl.event_bytes == ev_bytes
        stream_bytes = (pl.stream_bytes_min + 255) // 256 * 256
        self.ev_params.p.packed_stream_stride = stream_bytes
        self.layout = pl
        dev = K.device
        streams = B * Hkv
        self.max_desc = pl.desc_per_stream
        self.stream_bytes = stream_bytes
        self.packed = torch.empty(streams * stream_bytes, dtype=torch.uint8, device=dev)
        self.desc = torch.zeros(streams * self.max_desc * 16, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(pl.ws_bytes, dtype=torch.uint8, device=dev)

        def run(params, Kv, Vv, Qv, base_off, desc_first):
            _, lay = kv_layout_query(params)
            ws = torch.empty(max(int(lay.compress_ws_bytes), 16), dtype=torch.uint8, device=dev)
            params.p.packed_stream_stride = stream_bytes
            params.p.packed_base_offset = base_off
            params.p.desc_stream_stride = self.max_desc
            kv_compress(params, Kv, Vv, Qv, None, self.packed[base_off:],
                        self.desc[desc_first * 16:], None, None, None, ws)

        pp = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=prompt, seg_tokens=prompt_seg,
                      strategies=[(prompt_seg, D)], budget_bytes=4 * prompt_seg * D, scale=scale,
                      kv_stream_stride=L * D)
        run(pp, K, V, None, 0, 0)
        for e, (Le, w0, rb) in enumerate(pre):
            pe = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=window,
                          region_begin=window - protect - delta, region_len=delta,
                          seg_tokens=delta, n_win=window, strategies=[(T, D)],
                          budget_bytes=4 * delta * D, t2c_alpha=alpha, t2c_gamma=gamma,
                          scale=scale, kv_stream_stride=L * D, qw_head_stride=L * D,
                          store_logits=1)
            run(pe, K[:, :, w0:], V[:, :, w0:], Qall[:, :, w0:], prompt_bytes + e * ev_bytes,
                n_prompt_desc + e)
        self.n_prefix_events = len(pre)
        self.pipe = KvPipe(self.ev_params, self.cfg, self.packed, self.desc, self.ws)
        self.g = 0
        self.out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

    @property
    def length(self):
        """Sequence length after the tokens appended so far."""
        return self.prompt + self.g0 + self.g

    def step(self, n_new=1, decode=True):
        """Append the next n_new generated tokens; decode the last one's
        query over the cache (unless decode is False).  Returns (out, lse)
        views that the next step overwrites, or None."""
        p0 = self.length
        p1 = p0 + n_new
        assert p1 <= self.L
        g1 = self.g + n_new
        fire = g1 % self.delta == 0 and g1 >= self.protect + self.delta
        w0 = p1 - self.window
        wk = self.K[:, :, w0:] if fire else None
        wv = self.V[:, :, w0:] if fire else None
        wq = self.Qall[:, :, w0:] if fire else None
        q = self.Qall[:, :, p1 - 1].contiguous() if decode else None
        self.pipe.step(self.K[:, :, p0:], self.V[:, :, p0:], n_new, self.L * D, wk, wv, wq,
                       q, self.out if decode else None, self.lse if decode else None)
        self.g = g1
        return (self.out, self.lse) if decode else None

    def close(self):
        self.pipe.close()
