"""Shared helpers of the GPU parity tests: oracle runs over whole small
workloads, device/host layout conversions and the attention tolerance.

The attention tolerance is the one stated for the method's outputs: per
(batch, q head) row, max |o_gpu - o_ref| <= 2e-3 * ||o_ref||_2, where o_ref is
the unrounded fp64 oracle output.  Rounding the output to bf16 alone costs at
most 2^-9 |o_d| <= 1.95e-3 ||o||_2; fp32 accumulation and bf16 softmax weights
in the p.v product stay well inside the rest.
"""
import math
import sys

import numpy as np
import torch

from compressed_kv_cache_compress_amd import DESC_DTYPE, gen
from oracle import oracle as O

SCALE = np.float32(1.0 / math.sqrt(128.0))
ATT_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_compress_all(w, *, S, strategies, budget, region_begin=0, region_len=None, t2c_alpha=0,
                        t2c_gamma=0, forced=None, streams=None, capacity=None, K=None, V=None,
                        Qw=None, budget_scope=0):
    """Oracle compression of every (or the listed) stream of workload `w`.

    Returns dict stream -> oracle result, with descriptor offsets laid out as
    the library lays them out (stream s at s * capacity)."""
    B, Hkv, G = w["B"], w["Hkv"], w["G"]
    K = w["K"] if K is None else K
    V = w["V"] if V is None else V
    Qw = w["Qw"] if Qw is None else Qw
    res = {}
    todo = streams if streams is not None else range(B * Hkv)
    for s in todo:
        b, h = divmod(s, Hkv)
        Ks, Vs = gen.u16(K[b, h]), gen.u16(V[b, h])
        Qs = gen.u16(Qw[b, h * G:(h + 1) * G])
        f = None if forced is None else forced[s]
        res[s] = O.compress_stream(Ks, Vs, Qs, S=S, strategies=strategies, budget_bytes=budget,
                                   scale=SCALE, region_begin=region_begin, region_len=region_len,
                                   t2c_alpha=t2c_alpha, t2c_gamma=t2c_gamma, forced=f,
                                   base_offset=(s * capacity if capacity is not None else 0),
                                   budget_scope=budget_scope)
    return res


def assemble_cache(results, capacity, fill=0xFF):
    """Oracle segments of every stream placed in one packed buffer (stream s
    at s * capacity); unused bytes hold `fill` (0xFF bytes decode as NaN)."""
    n = max(results) + 1
    buf = np.full(n * capacity + 16, fill, np.uint8)
    descs = []
    for s in range(n):
        r = results[s]
        buf[s * capacity:s * capacity + r["used"]] = r["packed"]
        descs.append(r["desc"])
    return buf, np.stack(descs)


def to_dev_u8(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).copy()).to(device)


def desc_to_dev(d, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(d, DESC_DTYPE).view(np.uint8).reshape(-1).copy()).to(device)


def check_attention(out_gpu, lse_gpu, ref_out, ref_lse, label=""):
    """out_gpu: [rows,128] bf16 tensor; ref_out: [rows,128] fp64."""
    og = out_gpu.float().cpu().numpy().astype(np.float64).reshape(-1, 128)
    ref = np.asarray(ref_out, np.float64).reshape(-1, 128)
    norm = np.linalg.norm(ref, axis=1)
    err = np.abs(og - ref).max(axis=1)
    empty = np.isneginf(np.asarray(ref_lse).reshape(-1))
    assert np.all(og[empty] == 0), f"{label}: empty rows must be 0"
    bad = (err > ATT_TOL * norm) & ~empty
    worst = float(np.max(np.where(empty, 0, err / np.maximum(norm, 1e-300))))
    assert not bad.any(), f"{label}: {bad.sum()} rows over tolerance, worst rel {worst:.3e}"
    if lse_gpu is not None:
        lg = lse_gpu.cpu().numpy().astype(np.float64).reshape(-1)
        rl = np.asarray(ref_lse, np.float64).reshape(-1)
        assert np.all(np.isneginf(lg[empty]))
        d = np.abs(lg[~empty] - rl[~empty])
        assert np.all(d <= 1e-4 + 1e-5 * np.abs(rl[~empty])), f"{label}: lse max err {d.max():.3e}"
    return worst


def oracle_decode_all(q, buf, descs, n_desc=None):
    """q: [B,Hq,128] bf16 tensor; descs: [streams, maxd] -> (out [B*Hq,128], lse)."""
    B, Hq = q.shape[0], q.shape[1]
    streams = descs.shape[0]
    Hkv = streams // B
    G = Hq // Hkv
    outs, lses = [], []
    qn = gen.u16(q)
    for s in range(streams):
        b, h = divmod(s, Hkv)
        nd = descs.shape[1] if n_desc is None else int(n_desc[s])
        o, l = O.decode_stream(qn[b, h * G:(h + 1) * G], buf, descs[s, :nd], SCALE)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)
