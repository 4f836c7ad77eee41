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

from . import KvParams, kv_compress, kv_layout_query
from .gen import kara_schedule

D = 128


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
    sched, T = kara_schedule(prompt, gen, window=window, delta=delta, protect=protect, seg=seg,
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
                    kv_stream_stride=L * D, qw_head_stride=L * D)
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
