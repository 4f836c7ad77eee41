"""ctypes wrapper of the CPU oracle ``liboracle.so`` (test infrastructure).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  It never touches the GPU library.  Every function
returns numpy arrays; bf16 data travels as uint16 bit patterns.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DESC_DTYPE = np.dtype([("offset", "<u8"), ("n_tok", "<u2"), ("n_ch", "<u2"),
                       ("strategy", "u1"), ("flags", "u1"), ("seg_tokens", "<u2")])
assert DESC_DTYPE.itemsize == 16

BUILD_CMD = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", "-std=c11", "-Wall", "-o", _LIB, _SRC, "-lm"]


def build():
    """Compile liboracle.so in place (plain gcc; no GPU code)."""
    subprocess.check_call(BUILD_CMD)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_long, ctypes.c_float
        L.orc_exp2_f32.argtypes = [P, P, i64]
        L.orc_exp2_coeffs.argtypes = [P, P]
        L.orc_normalisers.argtypes = [i32, i32, P, P, f32, P, P, i32]
        L.orc_token_scores.argtypes = [i32, i32, i32, P, P, f32, P, P, P, i32]
        L.orc_channel_topc.argtypes = [P, i32, P, P]
        L.orc_top_t.argtypes = [P, i32, i32, P]
        L.orc_token2chunk.argtypes = [P, i32, i32, i32, i32, P]
        L.orc_seg_bytes.argtypes = [i32, i32, i32]
        L.orc_seg_bytes.restype = i64
        L.orc_compress_stream.argtypes = [P, P, P, P, P, P, ctypes.c_uint64, P, P, P, P, P, P, P,
                                          i32]
        L.orc_gram.argtypes = [P, i32, P, i32]
        L.orc_jacobi.argtypes = [P, P, P]
        L.orc_rotate.argtypes = [P, i64, P, P]
        L.orc_decode_stream_rot.argtypes = [i32, P, P, P, i32, f32, P, i32, P, P]
        L.orc_compress_stream.restype = i32
        L.orc_decode_stream.argtypes = [i32, P, P, P, i32, f32, P, P]
        L.orc_max_threads.restype = i32
        L.orc_summarize_stream.argtypes = [P, P, i32, P]
        L.orc_select_stream.argtypes = [i32, P, P, P, i32, i32, P, P]
        L.orc_select_stream.restype = i32
        L.orc_stream_choose.argtypes = [P, P, i32, i32, ctypes.c_uint64, P]
        L.orc_stream_choose.restype = ctypes.c_uint32
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def max_threads():
    return lib().orc_max_threads()


def exp2(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty_like(y)
    lib().orc_exp2_f32(_p(y), _p(out), y.size)
    return out


def exp2_coeffs():
    c = np.zeros(8, np.float32)
    l2e = np.zeros(1, np.float32)
    lib().orc_exp2_coeffs(_p(c), _p(l2e))
    return c, l2e[0]


def normalisers(K, Qw, scale, n_threads=0):
    """K: [n_ctx,128] u16, Qw: [nq,128] u16 -> (m[nq], invZ[nq]) fp32."""
    K, Qw = _u16(K), _u16(Qw)
    nq = Qw.shape[0]
    m = np.zeros(nq, np.float32)
    iz = np.zeros(nq, np.float32)
    lib().orc_normalisers(K.shape[0], nq, _p(K), _p(Qw), np.float32(scale), _p(m), _p(iz),
                          n_threads or max_threads())
    return m, iz


def token_scores(K, Qw, scale, m, invZ, t0=0, nt=None, n_threads=0):
    K, Qw = _u16(K), _u16(Qw)
    nt = K.shape[0] - t0 if nt is None else nt
    s = np.zeros(nt, np.float32)
    m = np.ascontiguousarray(m, np.float32)
    invZ = np.ascontiguousarray(invZ, np.float32)
    lib().orc_token_scores(t0, nt, Qw.shape[0], _p(K), _p(Qw), np.float32(scale), _p(m),
                           _p(invZ), _p(s), n_threads or max_threads())
    return s


def channel_topc(row, c):
    """row: [128] u16 -> (mask bytes [16] u8, rho fp32)."""
    row = _u16(row)
    mask = np.zeros(16, np.uint8)
    rho = np.zeros(1, np.float32)
    lib().orc_channel_topc(_p(row), c, _p(mask), _p(rho))
    return mask, rho[0]


def top_t(s, T):
    s = np.ascontiguousarray(s, np.float32)
    keep = np.zeros(s.size, np.uint8)
    lib().orc_top_t(_p(s), s.size, T, _p(keep))
    return keep


def token2chunk(s, T, alpha, gamma):
    s = np.ascontiguousarray(s, np.float32)
    keep = np.zeros(s.size, np.uint8)
    lib().orc_token2chunk(_p(s), s.size, T, alpha, gamma, _p(keep))
    return keep


def seg_bytes(T, c, S):
    return lib().orc_seg_bytes(T, c, S)


class _Params(ctypes.Structure):
    _fields_ = [("n_ctx", ctypes.c_int), ("region_begin", ctypes.c_int),
                ("region_len", ctypes.c_int), ("S", ctypes.c_int), ("G", ctypes.c_int),
                ("W", ctypes.c_int), ("n_strat", ctypes.c_int),
                ("strat_T", ctypes.c_void_p), ("strat_c", ctypes.c_void_p),
                ("budget_bytes", ctypes.c_long), ("t2c_alpha", ctypes.c_int),
                ("t2c_gamma", ctypes.c_int), ("scale", ctypes.c_float),
                ("budget_scope", ctypes.c_int), ("rotate", ctypes.c_int),
                ("rot_span", ctypes.c_int)]


def compress_stream(K, V, Qw, *, S, strategies, budget_bytes, scale, region_begin=0,
                    region_len=None, t2c_alpha=0, t2c_gamma=0, forced=None, base_offset=0,
                    n_threads=0, budget_scope=0, rotate=False, rot_span=0):
    """Compress one stream.

    K, V: [n_ctx,128] u16; Qw: [G,W,128] u16; strategies: list of (T, c).
    budget_scope 0: every segment within budget_bytes; 1: the stream's
    segments together within n_seg * budget_bytes (Lagrangian choice).
    rotate: the region's K and V vectors are rotated (SVD) before selection,
    one R per span of rot_span tokens (0: the whole region).
    Returns dict(packed, desc, used, scores, objective, m, invZ, rot) with rot
    [n_span,2,128,128] fp32 (R_K, R_V of each span) when rotating.
    """
    K, V, Qw = _u16(K), _u16(V), _u16(Qw)
    n_ctx = K.shape[0]
    G, W = Qw.shape[0], Qw.shape[1]
    region_len = n_ctx - region_begin if region_len is None else region_len
    nseg = region_len // S
    sT = np.array([t for t, _ in strategies], np.int32)
    sc = np.array([c for _, c in strategies], np.int32)
    prm = _Params(n_ctx, region_begin, region_len, S, G, W, len(strategies),
                  sT.ctypes.data, sc.ctypes.data, int(budget_bytes), t2c_alpha, t2c_gamma,
                  np.float32(scale), int(budget_scope), int(bool(rotate)), int(rot_span))
    cap = nseg * max(seg_bytes(t, c, S) for t, c in strategies) + 16
    packed = np.zeros(cap, np.uint8)
    desc = np.zeros(nseg, DESC_DTYPE)
    used = np.zeros(1, np.uint64)
    scores = np.zeros(region_len, np.float32)
    obj = np.zeros((nseg, len(strategies)), np.float32)
    m = np.zeros(G * W, np.float32)
    iz = np.zeros(G * W, np.float32)
    f = None if forced is None else np.ascontiguousarray(forced, np.uint8)
    n_span = region_len // (rot_span or region_len) if rotate else 0
    rot = np.zeros((n_span, 2, 128, 128), np.float32) if rotate else None
    rc = lib().orc_compress_stream(ctypes.byref(prm), _p(K), _p(V), _p(Qw), _p(f), _p(packed),
                                   base_offset, _p(desc), _p(used), _p(scores), _p(obj), _p(m),
                                   _p(iz), _p(rot), n_threads or max_threads())
    if rc != 0:
        raise ValueError(f"oracle compress failed ({rc})")
    return dict(packed=packed[: int(used[0])], desc=desc, used=int(used[0]), scores=scores,
                objective=obj, m=m, invZ=iz, rot=rot)


def gram(X, n_threads=0):
    """X: [T,128] u16 -> Gram matrix [128,128] fp32, each entry one fma
    chain over the tokens in order."""
    X = _u16(X)
    C = np.zeros((128, 128), np.float32)
    lib().orc_gram(_p(X), X.shape[0], _p(C), n_threads or max_threads())
    return C


def jacobi(C):
    """Symmetric C [128,128] fp32 -> (R [128,128] eigenvectors as columns,
    eigenvalues [128], largest first), fp32 cyclic Jacobi."""
    C = np.ascontiguousarray(C, np.float32)
    R = np.zeros((128, 128), np.float32)
    ev = np.zeros(128, np.float32)
    lib().orc_jacobi(_p(C), _p(R), _p(ev))
    return R, ev


def rotate(X, R):
    """X: [T,128] u16 -> R^T x per row, rounded to bf16 (u16)."""
    X = _u16(X)
    R = np.ascontiguousarray(R, np.float32)
    Y = np.zeros_like(X)
    lib().orc_rotate(_p(X), X.shape[0], _p(R), _p(Y))
    return Y


def decode_stream_rot(q, packed, desc, scale, rot, desc_per_span=None):
    """Decode over a rotated cache: rot [n_span,2,128,128] (R_K, R_V per
    span), descriptor i in span i // desc_per_span (default: one span);
    logits against R_K^T q of the token's span, output the sum over spans of
    R_V times the span's share of the rotated output."""
    q = _u16(q)
    packed = np.ascontiguousarray(packed, np.uint8)
    desc = np.ascontiguousarray(desc, DESC_DTYPE)
    rot = np.ascontiguousarray(rot, np.float32).reshape(-1, 2, 128, 128)
    dps = int(desc_per_span or max(desc.size, 1))
    assert rot.shape[0] * dps >= desc.size
    G = q.shape[0]
    out = np.zeros((G, 128), np.float64)
    lse = np.zeros(G, np.float64)
    buf = packed if packed.size else np.zeros(16, np.uint8)
    lib().orc_decode_stream_rot(G, _p(q), _p(buf), _p(desc), desc.size, np.float32(scale),
                                _p(rot), dps, _p(out), _p(lse))
    return out, lse


def decode_stream(q, packed, desc, scale):
    """q: [G,128] u16; packed: u8 buffer the desc offsets index; -> (out fp64 [G,128], lse [G])."""
    q = _u16(q)
    packed = np.ascontiguousarray(packed, np.uint8)
    desc = np.ascontiguousarray(desc, DESC_DTYPE)
    G = q.shape[0]
    out = np.zeros((G, 128), np.float64)
    lse = np.zeros(G, np.float64)
    buf = packed if packed.size else np.zeros(16, np.uint8)
    lib().orc_decode_stream(G, _p(q), _p(buf), _p(desc), desc.size, np.float32(scale), _p(out),
                            _p(lse))
    return out, lse


def summarize_stream(packed, desc):
    """Per-descriptor key summary: [n_desc, 2, 128] u16 (bf16 max, min per channel)."""
    packed = np.ascontiguousarray(packed, np.uint8)
    desc = np.ascontiguousarray(desc, DESC_DTYPE)
    out = np.zeros((desc.size, 2, 128), np.uint16)
    buf = packed if packed.size else np.zeros(16, np.uint8)
    lib().orc_summarize_stream(_p(buf), _p(desc), desc.size, _p(out))
    return out


def select_stream(q, summary, desc, k):
    """Query-aware segment selection: (selected descriptor indices ascending,
    scores [n_desc] fp32 with -inf for empty descriptors)."""
    q = _u16(q)
    summary = np.ascontiguousarray(summary, np.uint16)
    desc = np.ascontiguousarray(desc, DESC_DTYPE)
    n = desc.size
    score = np.zeros(max(n, 1), np.float32)
    sel = np.zeros(max(n, 1), np.int32)
    m = lib().orc_select_stream(q.shape[0], _p(q), _p(summary), _p(desc), n, int(k), _p(score),
                                _p(sel))
    return sel[:m].copy(), score[:n].copy()


def stream_choose(J, nbytes, B):
    """Per-stream budget choice from objectives J [nseg, n_strat] fp32 and
    strategy bytes [n_strat]: (chosen [nseg], multiplier bit pattern)."""
    J = np.ascontiguousarray(J, np.float32)
    nb = np.ascontiguousarray(nbytes, np.int64)
    nseg, ns = J.shape
    chosen = np.zeros(max(nseg, 1), np.int32)
    u = lib().orc_stream_choose(_p(J), _p(nb), nseg, ns, int(B), _p(chosen))
    return chosen[:nseg].copy(), int(u)
