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
                        Qw=None, budget_scope=0, rotate=False, rot_span=0):
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
                                   budget_scope=budget_scope, rotate=rotate, rot_span=rot_span)
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


# ---------------------------------------------------------------------------
# Incremental compression pipeline: the oracle's view of a pipeline state

def _rows_u8(a):
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


class PipelineOracle:
    """The oracle's side of a Kara pipeline run (`kara.KaraPipeline` kp,
    workload w, settings c with window, delta, protect, alpha, gamma):

      * the prefix: the prompt at full width and the events of the generated
        tokens before the pipeline's first token, each compressed by the
        oracle from its own window;
      * the pipeline's events, compressed by the oracle on demand (cached);
      * state_decode: the fp64 decode of a step's query over the prefix, the
        switched events' segments and every other appended token at full
        width.
    """

    def __init__(self, w, kp, c):
        from oracle import oracle as _O
        self.O = _O
        self.w, self.kp, self.c = w, kp, c
        self.Kh, self.Vh, self.Qh = gen.u16(w["K"]), gen.u16(w["V"]), gen.u16(w["Qall"])
        self.G = kp.Hq // kp.Hkv
        from oracle import kara as OK
        sched, _ = OK.events(kp.prompt, kp.L - kp.prompt, window=c["window"], delta=c["delta"],
                             protect=c["protect"], seg=c["delta"])
        self.T = OK.kept_tokens(c["retention_pct"], c["delta"])
        # events whose region ends by the pipeline's first token
        self.pre = [e for e in sched if e["r1"] <= kp.prompt + kp.g0]
        assert len(self.pre) == kp.n_prefix_events and self.T == kp.T
        self.cache, self.prefix_cache, self.prefix_events = {}, {}, {}

    def _event(self, s, L, w0, rb):
        """Oracle compression for stream s of the event at sequence length L
        whose window starts at w0 and whose region starts rb into it."""
        c = self.c
        b, h = divmod(s, self.kp.Hkv)
        G = self.G
        return self.O.compress_stream(
            self.Kh[b, h, w0:L], self.Vh[b, h, w0:L], self.Qh[b, h * G:(h + 1) * G, w0:L],
            S=c["delta"], strategies=[(self.T, 128)], budget_bytes=4 * c["delta"] * 128,
            scale=SCALE, region_begin=rb, region_len=c["delta"], t2c_alpha=c["alpha"],
            t2c_gamma=c["gamma"])

    def get(self, e, s, region):
        """Pipeline event e (region = its (start, end) in pipeline tokens, as
        the oracle's pipeline schedule gives it)."""
        if (e, s) not in self.cache:
            base = self.kp.prompt + self.kp.g0
            r0, r1 = base + region[0], base + region[1]
            L = r1 + self.c["protect"]
            w0 = L - self.c["window"]
            self.cache[(e, s)] = self._event(s, L, w0, r0 - w0)
        return self.cache[(e, s)]

    def prefix(self, s):
        """(parts, descs, bytes) of the prompt at full width and the prefix events."""
        if s not in self.prefix_cache:
            b, h = divmod(s, self.kp.Hkv)
            P = self.kp.prompt
            parts = [_rows_u8(self.Kh[b, h, :P]), _rows_u8(self.Vh[b, h, :P])]
            descs = [(0, P, 128, 0, 0x03, P)]
            off = 512 * P
            for ev in self.pre:
                r = self._event(s, ev["L"], ev["w0"], ev["rb"])
                self.prefix_events[(s, ev["L"])] = r
                off = self._append(parts, descs, off, r)
            self.prefix_cache[s] = (parts, descs, off)
        return self.prefix_cache[s]

    @staticmethod
    def _append(parts, descs, off, r):
        pk = np.concatenate([r["packed"], np.zeros((-r["used"]) % 16, np.uint8)])
        d = r["desc"][0]
        parts.append(pk)
        descs.append((off + int(d["offset"]), int(d["n_tok"]), int(d["n_ch"]), int(d["strategy"]),
                      int(d["flags"]), int(d["seg_tokens"])))
        return off + len(pk)

    def state_decode(self, s, entry, switched):
        from oracle import pipeline as OP
        kp = self.kp
        b, h = divmod(s, kp.Hkv)
        G = self.G
        p0, d0, off = self.prefix(s)
        parts, descs = list(p0), list(d0)
        for e in switched:
            off = self._append(parts, descs, off, self.get(e, s, entry["regions"][e]))
        base = kp.prompt + kp.g0
        for a, z in OP.state_tokens(dict(entry, switched=switched)):
            n = z - a
            parts += [_rows_u8(self.Kh[b, h, base + a:base + z]), _rows_u8(self.Vh[b, h, base + a:base + z])]
            descs.append((off, n, 128, 0, 0x03, n))
            off += 512 * n
        L = base + entry["g"]
        q = self.Qh[b, h * G:(h + 1) * G, L - 1]
        return self.O.decode_stream(q, np.concatenate(parts), np.array(descs, DESC_DTYPE), SCALE)


def run_pipeline(kp, n_steps, prefill=0, keep=None, sync=False):
    """Runs the steps, keeping (for the steps in `keep`, default all) the
    step's output and a copy of the descriptor list that step's decode read,
    both enqueued on the decode stream.  sync: the host waits for every step,
    as a serving loop does."""
    outs, lists = {}, {}
    if prefill:
        kp.step(prefill, decode=False)
    stream = torch.cuda.current_stream()
    for i in range(n_steps):
        out, lse = kp.step(1)
        if keep is None or i in keep:
            outs[i] = (out.clone(), lse.clone())
            lists[i] = kp.desc.clone()
        if sync:
            stream.synchronize()
    return outs, lists


def switched_from_list(kp, lst, streams):
    """Events whose slot holds a segment (the same for every stream), and the
    list as [streams][max_desc] descriptors."""
    d = lst.cpu().numpy().view(DESC_DTYPE).reshape(streams, kp.max_desc)
    first = kp.cfg.prefix_desc
    n = d[:, first:first + kp.cfg.max_events]["n_tok"] > 0
    assert np.all(n == n[0]), "streams disagree on the switched events"
    return [int(e) for e in np.nonzero(n[0])[0]], d


def check_pipeline_pages(kp, d, entry, switched, streams):
    """The list's page slots hold exactly the tokens the state keeps at full
    width, as paged descriptors of whole pages (the last one partly filled)."""
    from oracle import pipeline as OP
    per_page = {}
    for a, z in OP.state_tokens(dict(entry, switched=switched)):
        t = a
        while t < z:
            pg = t // kp.delta
            e = min(z, (pg + 1) * kp.delta)
            assert pg not in per_page and t == pg * kp.delta
            per_page[pg] = e - t
            t = e
    exp = {pg % kp.cfg.pages: n for pg, n in per_page.items()}
    base = kp.cfg.prefix_desc + kp.cfg.max_events
    pages = d[:, base:base + kp.cfg.pages]
    for s in range(streams):
        got = {}
        for j in range(kp.cfg.pages):
            x = pages[s, j]
            if x["n_tok"] > 0:
                assert int(x["flags"]) == 0x07 and int(x["seg_tokens"]) == kp.delta
                assert int(x["offset"]) == s * kp.stream_bytes + kp.cfg.pages_offset + \
                    j * kp.layout.page_bytes
                got[j] = int(x["n_tok"])
        assert got == exp, (s, got, exp)


def check_pipeline_finals(kp, oe, entries, streams, sample=None):
    """Every switched event's final segment (and every prefix event) is bit
    exact against the oracle's compression of that event."""
    packed = kp.packed.view(streams, -1)
    d = kp.desc.cpu().numpy().view(DESC_DTYPE).reshape(streams, kp.max_desc)
    last = entries[-1]
    for s in (range(streams) if sample is None else sample):
        row = packed[s].cpu().numpy()
        checks = [(kp.cfg.prefix_desc + e, oe.get(e, s, last["regions"][e]),
                   kp.cfg.events_offset + e * kp.layout.event_bytes) for e in range(len(last["regions"]))]
        oe.prefix(s)
        n_prompt = kp.cfg.prefix_desc - kp.n_prefix_events
        ev0 = kp.cfg.events_offset - kp.n_prefix_events * kp.layout.event_bytes
        for i, ev in enumerate(oe.pre):
            checks.append((n_prompt + i, oe.prefix_events[(s, ev["L"])],
                           ev0 + i * kp.layout.event_bytes))
        for slot, r, rel in checks:
            gd = d[s, slot]
            rd = r["desc"][0]
            assert int(gd["offset"]) == s * kp.stream_bytes + rel, (s, slot)
            for f in ("n_tok", "n_ch", "strategy", "flags", "seg_tokens"):
                assert int(gd[f]) == int(rd[f]), (s, slot, f)
            assert np.array_equal(row[rel:rel + r["used"]], r["packed"]), (s, slot)
