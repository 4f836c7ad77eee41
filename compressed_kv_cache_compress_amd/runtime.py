"""Convenience layer over the C ABI: allocates outputs and workspaces with
torch on the current device and calls kv_compress / kv_attend_decode /
kv_summarize / kv_select_segments.

All computation happens in libkvc's HIP kernels; nothing here touches the
data except to allocate it.
"""
import torch

from . import (DESC_DTYPE, KvParams, kv_attend_decode, kv_attend_decode_rotated, kv_compress,
               kv_compress_rotated, kv_layout_query, kv_select_segments, kv_summarize)


def _u8(n, device):
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


def _as_u16(t):
    assert t.dtype == torch.bfloat16 and t.is_cuda, (t.dtype, t.device)
    return t


class Compressed:
    """Result of compress(): packed bytes, descriptors and optional outputs."""

    def __init__(self, params, layout, packed, desc, used, scores, objective, rot=None):
        self.params, self.layout = params, layout
        self.packed, self.desc, self.used = packed, desc, used
        self.scores, self.objective = scores, objective
        self.rot = rot  # [streams, n_span, 2, 128, 128] fp32 when compressed with rotation

    @property
    def n_seg(self):
        return self.layout.n_seg

    def desc_host(self):
        return self.desc.cpu().numpy().view(DESC_DTYPE).reshape(self.params.streams, -1)


def compress_params(*, batch, n_q_heads, n_kv_heads, n_ctx, seg_tokens, n_win, strategies,
                    budget_bytes, **kw):
    return KvParams(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, n_ctx=n_ctx,
                    seg_tokens=seg_tokens, n_win=n_win, strategies=strategies,
                    budget_bytes=budget_bytes, **kw)


def compress(K, V, Qw, *, seg_tokens, strategies, budget_bytes, region_begin=0, region_len=None,
             t2c_alpha=0, t2c_gamma=0, scale=0.0, forced=None, want_scores=False,
             want_objective=False, ws=None, packed=None, desc=None, n_ctx=None,
             kv_stream_stride=0, qw_head_stride=0, packed_stream_stride=0, packed_base_offset=0,
             desc_stream_stride=0, n_q_heads=None, budget_scope=0, compress_max_waves=0,
             rotate=False, store_logits=False, rot_span=0):
    """K, V: [B, Hkv, N, 128] bf16 (or strided views described by the stride
    arguments); Qw: [B, Hq, W, 128] bf16 or None.  budget_scope 1 shares
    n_seg * budget_bytes among a stream's segments.  rotate: one SVD
    rotation per span of rot_span tokens (0: per stream)."""
    B, Hkv = K.shape[0], K.shape[1]
    N = K.shape[2] if n_ctx is None else n_ctx
    Hq = Qw.shape[1] if Qw is not None else (n_q_heads or Hkv)
    W = Qw.shape[2] if Qw is not None else 0
    p = KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=N, region_begin=region_begin,
                 region_len=region_len, seg_tokens=seg_tokens, n_win=W, strategies=strategies,
                 budget_bytes=budget_bytes, t2c_alpha=t2c_alpha, t2c_gamma=t2c_gamma, scale=scale,
                 kv_stream_stride=kv_stream_stride, qw_head_stride=qw_head_stride,
                 packed_stream_stride=packed_stream_stride,
                 packed_base_offset=packed_base_offset, desc_stream_stride=desc_stream_stride,
                 budget_scope=budget_scope, compress_max_waves=compress_max_waves,
                 rotate=rotate, store_logits=store_logits, rot_span=rot_span)
    _, L = kv_layout_query(p)
    dev = K.device
    streams = B * Hkv
    dstride = desc_stream_stride or L.n_seg
    if packed is None:
        packed = _u8(L.packed_bytes_max, dev)
    if desc is None:
        desc = torch.zeros(streams * dstride * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    scores = torch.empty((streams, p.p.region_len), dtype=torch.float32, device=dev) if want_scores else None
    objective = (torch.empty((streams, L.n_seg, len(strategies)), dtype=torch.float32, device=dev)
                 if want_objective else None)
    if ws is None or ws.numel() < L.compress_ws_bytes:
        ws = _u8(L.compress_ws_bytes, dev)
    rot = None
    if rotate:
        n_span = p.p.region_len // (rot_span or p.p.region_len)
        rot = torch.empty((B * Hkv, n_span, 2, 128, 128), dtype=torch.float32, device=dev)
        kv_compress_rotated(p, _as_u16(K), _as_u16(V), Qw, forced, packed, desc, used, scores,
                            objective, rot, ws)
    else:
        kv_compress(p, _as_u16(K), _as_u16(V), Qw, forced, packed, desc, used, scores, objective,
                    ws)
    return Compressed(p, L, packed, desc, used, scores, objective, rot)


def decode_params(*, batch, n_q_heads, n_kv_heads, max_desc_per_stream, decode_splits=0,
                  scale=0.0):
    return KvParams(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                    max_desc_per_stream=max_desc_per_stream, decode_splits=decode_splits,
                    scale=scale)


def decode(q, packed, desc, *, n_kv_heads, max_desc_per_stream, n_desc=None, decode_splits=0,
           scale=0.0, want_lse=True, out=None, lse=None, ws=None, params=None, rot=None,
           seg_tokens=0, rot_span=0):
    """q: [B, Hq, 128] bf16 -> (out [B, Hq, 128] bf16, lse [B, Hq] fp32 or None).
    rot: the rotations of a cache compressed with rotation (per span of
    rot_span tokens of seg_tokens-token segments when rot_span > 0)."""
    B, Hq = q.shape[0], q.shape[1]
    p = params or decode_params(batch=B, n_q_heads=Hq, n_kv_heads=n_kv_heads,
                                max_desc_per_stream=max_desc_per_stream,
                                decode_splits=decode_splits, scale=scale)
    if rot is not None:
        p.p.rotate = 1
        if rot_span:
            p.p.seg_tokens, p.p.rot_span = seg_tokens, rot_span
    if ws is None:
        _, L = kv_layout_query(p)
        ws = _u8(L.decode_ws_bytes, q.device)
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if rot is not None:
        kv_attend_decode_rotated(p, q, packed, desc, n_desc, rot, out, lse, ws)
    else:
        kv_attend_decode(p, q, packed, desc, n_desc, out, lse, ws)
    return out, lse


def summarize(packed, desc, *, batch, n_q_heads, n_kv_heads, max_desc_per_stream, n_desc=None,
              summary=None):
    """Per-descriptor key summaries: uint16 [streams, max_desc, 2, 128] (bf16
    channel maximum, minimum)."""
    streams = batch * n_kv_heads
    p = decode_params(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                      max_desc_per_stream=max_desc_per_stream)
    if summary is None:
        summary = torch.empty((streams, max_desc_per_stream, 2, 128), dtype=torch.int16,
                              device=packed.device)
    kv_summarize(p, packed, desc, n_desc, summary)
    return summary


def select(q, summary, desc, keep, *, n_kv_heads, max_desc_per_stream, n_desc=None,
           out_desc=None, out_n=None, score=None):
    """Query-aware selection: (out_desc uint8 [streams * keep * 16], out_n int32
    [streams], score fp32 [streams, max_desc]).  Decode over it with
    max_desc_per_stream = keep and n_desc = out_n."""
    B, Hq = q.shape[0], q.shape[1]
    streams = B * n_kv_heads
    keep = min(int(keep), int(max_desc_per_stream))
    p = decode_params(batch=B, n_q_heads=Hq, n_kv_heads=n_kv_heads,
                      max_desc_per_stream=max_desc_per_stream)
    dev = q.device
    if out_desc is None:
        out_desc = torch.zeros(streams * keep * 16, dtype=torch.uint8, device=dev)
    if out_n is None:
        out_n = torch.empty(streams, dtype=torch.int32, device=dev)
    if score is None:
        score = torch.empty((streams, max_desc_per_stream), dtype=torch.float32, device=dev)
    kv_select_segments(p, q, summary, desc, n_desc, keep, out_desc, out_n, score)
    return out_desc, out_n, score
