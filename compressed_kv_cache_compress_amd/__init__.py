"""Python binding of libkvc (include/kvc.h): argument marshalling only.

Every step of compression and decode runs in the HIP kernels of
``libkvc.so``; this module only turns torch tensors into device pointers and
the current HIP stream.  If the library is missing the import of the entry
points fails loudly -- there is no CPU fallback.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

HEAD_DIM = 128
MAX_STRATEGIES = 32
DESC_CHOOSE = 0xFF

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration",
          -3: "no strategy fits the byte budget", -4: "workspace too small",
          -5: "pointer not 16-byte aligned", -6: "HIP launch error"}

DESC_DTYPE = np.dtype([("offset", "<u8"), ("n_tok", "<u2"), ("n_ch", "<u2"),
                       ("strategy", "u1"), ("flags", "u1"), ("seg_tokens", "<u2")])


class KvcError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status})")
        self.status = status


class Strategy(ctypes.Structure):
    _fields_ = [("n_tok", ctypes.c_uint16), ("n_ch", ctypes.c_uint16)]


class Params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", ctypes.c_uint32),
                ("n_q_heads", ctypes.c_uint32), ("n_kv_heads", ctypes.c_uint32),
                ("head_dim", ctypes.c_uint32), ("n_ctx", ctypes.c_uint32),
                ("region_begin", ctypes.c_uint32), ("region_len", ctypes.c_uint32),
                ("seg_tokens", ctypes.c_uint32), ("n_win", ctypes.c_uint32),
                ("strategies", ctypes.POINTER(Strategy)), ("n_strategies", ctypes.c_uint32),
                ("budget_bytes", ctypes.c_uint32), ("t2c_alpha", ctypes.c_uint32),
                ("t2c_gamma", ctypes.c_uint32), ("scale", ctypes.c_float),
                ("kv_stream_stride", ctypes.c_uint64), ("qw_head_stride", ctypes.c_uint64),
                ("packed_stream_stride", ctypes.c_uint64), ("packed_base_offset", ctypes.c_uint64),
                ("desc_stream_stride", ctypes.c_uint32), ("max_desc_per_stream", ctypes.c_uint32),
                ("decode_splits", ctypes.c_uint32), ("budget_scope", ctypes.c_uint32),
                ("compress_max_waves", ctypes.c_uint32), ("rotate", ctypes.c_uint32),
                ("store_logits", ctypes.c_uint32), ("rot_span", ctypes.c_uint32)]


class Layout(ctypes.Structure):
    _fields_ = [("seg_bytes", ctypes.c_uint32 * MAX_STRATEGIES), ("feasible_mask", ctypes.c_uint32),
                ("n_seg", ctypes.c_uint32), ("max_seg_bytes", ctypes.c_uint64),
                ("stream_capacity", ctypes.c_uint64), ("packed_bytes_max", ctypes.c_uint64),
                ("n_desc", ctypes.c_uint64), ("compress_ws_bytes", ctypes.c_uint64),
                ("decode_ws_bytes", ctypes.c_uint64), ("decode_splits", ctypes.c_uint32),
                ("needs_scoring", ctypes.c_uint32)]


class PipeConfig(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("mode", ctypes.c_uint32),
                ("switch_lag", ctypes.c_uint32), ("pages", ctypes.c_uint32),
                ("max_events", ctypes.c_uint32), ("prefix_desc", ctypes.c_uint32),
                ("protect", ctypes.c_uint32), ("reserved0", ctypes.c_uint32),
                ("events_offset", ctypes.c_uint64), ("pages_offset", ctypes.c_uint64),
                ("reserved", ctypes.c_uint64 * 2)]


class PipeLayout(ctypes.Structure):
    _fields_ = [("desc_per_stream", ctypes.c_uint32), ("period", ctypes.c_uint32),
                ("event_bytes", ctypes.c_uint64), ("page_bytes", ctypes.c_uint64),
                ("stream_bytes_min", ctypes.c_uint64), ("ws_bytes", ctypes.c_uint64),
                ("decode_splits", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class PipeStats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_uint64), ("tokens", ctypes.c_uint64),
                ("events_fired", ctypes.c_uint64), ("events_switched", ctypes.c_uint64),
                ("host_waits", ctypes.c_uint64), ("pending", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


PIPE_ASYNC, PIPE_SYNC, PIPE_LAG = 0, 1, 2

_lib = None


def lib():
    """The loaded libkvc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libkvc.so not built ({LIB_PATH}); run "
                              "python -m compressed_kv_cache_compress_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.kv_layout_query.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Layout)]
        L.kv_layout_query.restype = ctypes.c_int
        L.kv_compress.argtypes = [ctypes.POINTER(Params), P, P, P, P, P, P, P, P, P, P,
                                  ctypes.c_size_t, P]
        L.kv_compress.restype = ctypes.c_int
        L.kv_attend_decode.argtypes = [ctypes.POINTER(Params), P, P, P, P, P, P, P,
                                       ctypes.c_size_t, P]
        L.kv_attend_decode.restype = ctypes.c_int
        L.kv_attend_decode_noalloc.argtypes = [ctypes.POINTER(Params), P, P, P, P, P, P, P]
        L.kv_attend_decode_noalloc.restype = ctypes.c_int
        L.kv_summarize.argtypes = [ctypes.POINTER(Params), P, P, P, P, P]
        L.kv_summarize.restype = ctypes.c_int
        L.kv_select_segments.argtypes = [ctypes.POINTER(Params), P, P, P, P, ctypes.c_uint32, P,
                                         P, P, P]
        L.kv_select_segments.restype = ctypes.c_int
        u32, u64 = ctypes.c_uint32, ctypes.c_uint64
        L.kv_compress_rotated.argtypes = [ctypes.POINTER(Params), P, P, P, P, P, P, P, P, P, P, P,
                                          ctypes.c_size_t, P]
        L.kv_compress_rotated.restype = ctypes.c_int
        L.kv_attend_decode_rotated.argtypes = [ctypes.POINTER(Params), P, P, P, P, P, P, P, P,
                                               ctypes.c_size_t, P]
        L.kv_attend_decode_rotated.restype = ctypes.c_int
        L.kv_append.argtypes = [ctypes.POINTER(Params), P, P, u32, u32, u32, u64, P, P, P]
        L.kv_append.restype = ctypes.c_int
        L.kv_pipe_layout.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(PipeConfig),
                                     ctypes.POINTER(PipeLayout)]
        L.kv_pipe_layout.restype = ctypes.c_int
        L.kv_pipe_create.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(PipeConfig), P, P, P,
                                     ctypes.c_size_t, P, ctypes.POINTER(ctypes.c_void_p)]
        L.kv_pipe_create.restype = ctypes.c_int
        L.kv_pipe_step.argtypes = [P, P, P, u32, u64, P, P, P, P, P, P, P]
        L.kv_pipe_step.restype = ctypes.c_int
        L.kv_pipe_drain.argtypes = [P, P]
        L.kv_pipe_drain.restype = ctypes.c_int
        L.kv_pipe_get_stats.argtypes = [P, ctypes.POINTER(PipeStats)]
        L.kv_pipe_get_stats.restype = ctypes.c_int
        L.kv_pipe_destroy.argtypes = [P]
        L.kv_pipe_destroy.restype = ctypes.c_int
        L.kv_read_stream.argtypes = [P, u64, P, P]
        L.kv_read_stream.restype = ctypes.c_int
        L.kvc_status_str.argtypes = [ctypes.c_int]
        L.kvc_status_str.restype = ctypes.c_char_p
        L.kvc_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


class KvParams:
    """Owner of a kvc_params struct and of the host strategy array it points to."""

    def __init__(self, *, batch, n_q_heads, n_kv_heads, head_dim=HEAD_DIM, n_ctx=0,
                 region_begin=0, region_len=None, seg_tokens=0, n_win=0, strategies=(),
                 budget_bytes=0, t2c_alpha=0, t2c_gamma=0, scale=0.0, kv_stream_stride=0,
                 qw_head_stride=0, packed_stream_stride=0, packed_base_offset=0,
                 desc_stream_stride=0, max_desc_per_stream=0, decode_splits=0,
                 budget_scope=0, compress_max_waves=0, rotate=0, store_logits=0, rot_span=0):
        strategies = list(strategies)
        self._strat = (Strategy * max(1, len(strategies)))(*[Strategy(t, c) for t, c in strategies])
        if region_len is None:
            region_len = n_ctx - region_begin
        self.p = Params()
        p = self.p
        p.struct_size = ctypes.sizeof(Params)
        p.batch, p.n_q_heads, p.n_kv_heads, p.head_dim = batch, n_q_heads, n_kv_heads, head_dim
        p.n_ctx, p.region_begin, p.region_len = n_ctx, region_begin, region_len
        p.seg_tokens, p.n_win = seg_tokens, n_win
        p.strategies = ctypes.cast(self._strat, ctypes.POINTER(Strategy)) if strategies else None
        p.n_strategies = len(strategies)
        p.budget_bytes, p.t2c_alpha, p.t2c_gamma = budget_bytes, t2c_alpha, t2c_gamma
        p.scale = scale
        p.kv_stream_stride, p.qw_head_stride = kv_stream_stride, qw_head_stride
        p.packed_stream_stride, p.packed_base_offset = packed_stream_stride, packed_base_offset
        p.desc_stream_stride, p.max_desc_per_stream = desc_stream_stride, max_desc_per_stream
        p.decode_splits = decode_splits
        p.budget_scope = budget_scope
        p.compress_max_waves = compress_max_waves
        p.rotate = int(bool(rotate))
        p.store_logits = int(bool(store_logits))
        p.rot_span = rot_span
        self.strategies = strategies

    @property
    def streams(self):
        return self.p.batch * self.p.n_kv_heads


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def kv_layout_query(params, check=True):
    """Host-only layout query -> (status, Layout)."""
    L = Layout()
    st = lib().kv_layout_query(ctypes.byref(params.p), ctypes.byref(L))
    if check and st not in (0,):
        raise KvcError("kv_layout_query", st)
    return st, L


def kv_compress(params, K, V, Qwin, forced, packed, desc, used_bytes, scores, objective, ws):
    """Enqueue compression on the current stream (tensors on the GPU)."""
    st = lib().kv_compress(ctypes.byref(params.p), _ptr(K), _ptr(V), _ptr(Qwin), _ptr(forced),
                           _ptr(packed), _ptr(desc), _ptr(used_bytes), _ptr(scores),
                           _ptr(objective), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                           _stream())
    if st != 0:
        raise KvcError("kv_compress", st)


def kv_compress_rotated(params, K, V, Qwin, forced, packed, desc, used_bytes, scores, objective,
                        rot, ws):
    """Enqueue compression with the SVD rotation (params.rotate = 1)."""
    st = lib().kv_compress_rotated(ctypes.byref(params.p), _ptr(K), _ptr(V), _ptr(Qwin),
                                   _ptr(forced), _ptr(packed), _ptr(desc), _ptr(used_bytes),
                                   _ptr(scores), _ptr(objective), _ptr(rot), _ptr(ws),
                                   ws.numel() * ws.element_size() if ws is not None else 0,
                                   _stream())
    if st != 0:
        raise KvcError("kv_compress_rotated", st)


def kv_attend_decode_rotated(params, q, packed, desc, n_desc, rot, out, lse, ws):
    """Enqueue decode attention over a rotated cache (params.rotate = 1)."""
    st = lib().kv_attend_decode_rotated(ctypes.byref(params.p), _ptr(q), _ptr(packed), _ptr(desc),
                                        _ptr(n_desc), _ptr(rot), _ptr(out), _ptr(lse), _ptr(ws),
                                        ws.numel() * ws.element_size() if ws is not None else 0,
                                        _stream())
    if st != 0:
        raise KvcError("kv_attend_decode_rotated", st)


def kv_attend_decode(params, q, packed, desc, n_desc, out, lse, ws):
    """Enqueue decode attention on the current stream (tensors on the GPU)."""
    st = lib().kv_attend_decode(ctypes.byref(params.p), _ptr(q), _ptr(packed), _ptr(desc),
                                _ptr(n_desc), _ptr(out), _ptr(lse), _ptr(ws),
                                ws.numel() * ws.element_size() if ws is not None else 0, _stream())
    if st != 0:
        raise KvcError("kv_attend_decode", st)


NOALLOC_SCRATCH_BYTES = 16 << 20


def kv_attend_decode_noalloc(params, q, packed, desc, n_desc, out, lse):
    """Decode attention with the library's fixed scratch instead of a
    workspace (nothing is allocated; calls on one GPU must not overlap)."""
    st = lib().kv_attend_decode_noalloc(ctypes.byref(params.p), _ptr(q), _ptr(packed), _ptr(desc),
                                        _ptr(n_desc), _ptr(out), _ptr(lse), _stream())
    if st != 0:
        raise KvcError("kv_attend_decode_noalloc", st)


def kv_summarize(params, packed, desc, n_desc, summary):
    """Enqueue the per-descriptor key summaries on the current stream."""
    st = lib().kv_summarize(ctypes.byref(params.p), _ptr(packed), _ptr(desc), _ptr(n_desc),
                            _ptr(summary), _stream())
    if st != 0:
        raise KvcError("kv_summarize", st)


def kv_select_segments(params, q, summary, desc, n_desc, keep, out_desc, out_n, score):
    """Enqueue query-aware segment selection on the current stream."""
    st = lib().kv_select_segments(ctypes.byref(params.p), _ptr(q), _ptr(summary), _ptr(desc),
                                  _ptr(n_desc), int(keep), _ptr(out_desc), _ptr(out_n),
                                  _ptr(score), _stream())
    if st != 0:
        raise KvcError("kv_select_segments", st)


def kv_read_stream(src, nbytes, sink):
    """Enqueue the HBM read-stream reference over the first nbytes of src
    (a measurement, not a step of the method) on the current stream."""
    st = lib().kv_read_stream(_ptr(src), int(nbytes), _ptr(sink), _stream())
    if st != 0:
        raise KvcError("kv_read_stream", st)


def kv_append(params, k_new, v_new, n_new, fill, capacity, page_offset, packed, page_desc):
    """Enqueue the append of n_new tokens per stream to dense pages."""
    st = lib().kv_append(ctypes.byref(params.p), _ptr(k_new), _ptr(v_new), int(n_new), int(fill),
                         int(capacity), int(page_offset), _ptr(packed), _ptr(page_desc), _stream())
    if st != 0:
        raise KvcError("kv_append", st)


def pipe_config(*, mode=PIPE_ASYNC, switch_lag=0, pages, max_events, prefix_desc=0, protect=0,
                events_offset=0, pages_offset=0):
    c = PipeConfig()
    c.struct_size = ctypes.sizeof(PipeConfig)
    c.mode, c.switch_lag, c.pages, c.max_events = mode, switch_lag, pages, max_events
    c.prefix_desc, c.protect = prefix_desc, protect
    c.events_offset, c.pages_offset = events_offset, pages_offset
    return c


def kv_pipe_layout(params, cfg, check=True):
    """Host-only pipeline layout query -> (status, PipeLayout)."""
    L = PipeLayout()
    st = lib().kv_pipe_layout(ctypes.byref(params.p), ctypes.byref(cfg), ctypes.byref(L))
    if check and st != 0:
        raise KvcError("kv_pipe_layout", st)
    return st, L


class KvPipe:
    """Owner of a kvc_pipe handle (kv_pipe_create .. kv_pipe_destroy).  The
    tensors passed at creation are kept referenced until close()."""

    def __init__(self, params, cfg, packed, desc, ws):
        self.params, self.cfg = params, cfg
        self._keep = (packed, desc, ws)
        self.stream = _stream()
        h = ctypes.c_void_p()
        st = lib().kv_pipe_create(ctypes.byref(params.p), ctypes.byref(cfg), _ptr(packed),
                                  _ptr(desc), _ptr(ws), ws.numel() * ws.element_size(),
                                  self.stream, ctypes.byref(h))
        if st != 0:
            raise KvcError("kv_pipe_create", st)
        self.h = h

    def step(self, k_new, v_new, n_new=1, new_stride=0, win_K=None, win_V=None, win_Q=None,
             q=None, out=None, lse=None):
        st = lib().kv_pipe_step(self.h, _ptr(k_new), _ptr(v_new), int(n_new), int(new_stride),
                                _ptr(win_K), _ptr(win_V), _ptr(win_Q), _ptr(q), _ptr(out),
                                _ptr(lse), self.stream)
        if st != 0:
            raise KvcError("kv_pipe_step", st)

    def drain(self):
        st = lib().kv_pipe_drain(self.h, self.stream)
        if st != 0:
            raise KvcError("kv_pipe_drain", st)

    def stats(self):
        s = PipeStats()
        st = lib().kv_pipe_get_stats(self.h, ctypes.byref(s))
        if st != 0:
            raise KvcError("kv_pipe_get_stats", st)
        return {k: int(getattr(s, k)) for k, _ in PipeStats._fields_ if k != "reserved"}

    def close(self):
        if self.h:
            lib().kv_pipe_destroy(self.h)
            self.h = None
            self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def desc_view(t):
    """uint8 tensor of descriptors (host copy) -> numpy structured array."""
    return t.detach().cpu().numpy().view(DESC_DTYPE)
