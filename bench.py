"""Benchmark: compressed decode attention on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: kv_compress (window scoring, per-vector channel top-c,
per-segment strategy choice, offsets, pack) followed by kv_attend_decode
(split-K decode over the packed segments + log-sum-exp merge).

Workload (default): batched long context -- B 16, GQA 32/8, head_dim 128,
context 131072, segment 128, window 64 queries per q head, budget 25 % of the
dense K+V bytes per segment, per-segment heavy-token density U(0, 2 %),
seeded synthetic bf16 data (gen.py).

Printed JSON (one line):
  value        KV tokens/s of decode attention = batch * context / median
               decode time over the timed steps (HIP events around
               kv_attend_decode on its stream; the mean is reported beside it);
               each step reads an unrelated 1 GiB buffer between compress and
               decode so the packed cache is not served from the MALL
  ms_per_step  wall time of one whole step (compress + decode); compress runs
               with store_logits = 1 (the first scoring pass keeps the logits
               for the second); compress_ms_logits_recomputed times the
               same compress with the logits recomputed
  roofline     decode (k_decode_split + k_decode_reduce) against 8 TB/s HBM;
               algorithmic bytes = descriptors + masks + values of every kept
               segment + q + out + partials written and read back
  cpu_baseline the CPU oracle (C, OpenMP) on a bounded sample, on every host
               core it may use (at most 16): compress of four streams, then
               fp64 decode of them by a thread pool
  kara         beside the headline (not part of `value`): decode over the
               Kara sliding-window cache (mostly dense prompt)
  stream_budget beside the headline (not part of `value`): the same workload
               with the byte budget shared by each stream's segments
  graph        beside the headline: decode on the Llama-3-8B-shaped layer
               (a few microseconds per call) launched eagerly and from a
               HIP graph of 20 calls
  read_stream  the achievable-bandwidth reference: kv_read_stream (a plain
               16-byte-load read of as many bytes as one decode reads)
  stage2       beside the headline (not part of `value`): query-aware
               selection of --select-pct percent of the segments
               (kv_summarize once, kv_select_segments + kv_attend_decode over
               the kept descriptors per step)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_HBM_GBS = 8000.0
PIPE_EVENT_WAVES = 1024  # waves an event kernel may keep in flight in the capped asynchronous run
EVICT_BYTES = 1 << 30    # read between compress and decode: four times the 256 MB MALL


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="batched128k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-splits", type=int, default=0, help="0 = library choice")
    ap.add_argument("--select-pct", type=float, default=12.5,
                    help="query-aware selection measured beside the headline: percent of the "
                         "segments kept (0 = off)")
    ap.add_argument("--no-kara", action="store_true",
                    help="skip the Kara sliding-window decode measurement beside the headline")
    ap.add_argument("--pipe-steps", type=int, default=512,
                    help="Kara generation steps through the compression pipeline, timed blocking "
                         "and asynchronous beside the headline (0 = off)")
    ap.add_argument("--no-rotate", action="store_true",
                    help="skip the SVD-rotation measurement beside the headline")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph decode measurement on the Llama-3-8B-shaped layer")
    ap.add_argument("--no-stream-budget", action="store_true",
                    help="skip the per-stream budget measurement beside the headline")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "decode_batched128k_traffic.md"),
                    help="summary with the measured decode HBM bytes per launch (rocprofv3 pmc)")
    return ap.parse_args()


def decode_partials(splits, rotated=False):
    """Partial rows per (b, q head) a decode writes and its merge reads: the
    four waves of a workgroup, consecutive splits of one stream, merge their
    states first when the split count is a multiple of 4 (unrotated decode)."""
    return splits if rotated or splits % 4 else splits // 4


def algorithmic_decode_bytes(desc, B, Hq, splits, rotated=False):
    n = desc["n_tok"].astype(np.int64)
    c = desc["n_ch"].astype(np.int64)
    masks = np.where(c < 128, 2 * 16 * n, 0)
    vals = 2 * 2 * n * c
    seg = (16 + masks + vals).sum()  # descriptor + masks + values (index lists unread)
    q = out = B * Hq * 128 * 2
    partials = 2 * B * Hq * decode_partials(splits, rotated) * (2 + 128) * 4
    return int(seg + q + out + partials)


def decode_source_hash():
    import hashlib
    src = os.path.join(ROOT, "compressed_kv_cache_compress_amd", "csrc", "kvc_decode.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()


def measured_traffic(path):
    """HBM bytes per decode launch from the committed counter summary, or None
    when there is none or the decode source changed since it was taken."""
    if not path or not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kvc_decode.hip sha256") != decode_source_hash():
        return None
    try:
        return int(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def bench_kara(a, kvc, stream):
    """Kara sliding-window workload (B 64, GQA 32/8, prompt 16384 dense + 127
    compressed events of 13 tokens + 64-token dense tail per stream): the
    cache is built once with kv_compress events, then decode attention over it
    is timed with HIP events on the launch stream."""
    from compressed_kv_cache_compress_amd import gen, kara
    k = gen.KARA
    dev = torch.device("cuda:0")
    w = gen.make_kara(seed=a.seed, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(128.0)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    cache = kara.build_cache(w["K"], w["V"], w["Qall"], prompt=w["prompt"], gen=w["gen"],
                             window=k["window"], delta=k["delta"], protect=k["protect"], seg=64,
                             retention_pct=k["retention_pct"], alpha=k["alpha"], gamma=k["gamma"],
                             scale=scale)
    e1.record(stream)
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    del w["K"], w["V"], w["Qall"]
    torch.cuda.empty_cache()
    B, Hq, Hkv = w["B"], w["Hq"], w["Hkv"]
    p = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_desc_per_stream=cache.max_desc,
                     scale=scale)
    _, L = kvc.kv_layout_query(p)
    dws = torch.empty(L.decode_ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    for i in range(a.warmup + a.steps):
        e = ev[i - a.warmup] if i >= a.warmup else None
        if e:
            e[0].record(stream)
        kvc.kv_attend_decode(p, w["q"], cache.packed, cache.desc, None, out, None, dws)
        if e:
            e[1].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([x[0].elapsed_time(x[1]) for x in ev])) * 1e-3
    dh = cache.desc.cpu().numpy().view(kvc.DESC_DTYPE)
    n = dh["n_tok"].astype(np.int64)
    c = dh["n_ch"].astype(np.int64)
    alg = int((16 + np.where(c < 128, 32 * n, 0) + 4 * n * c).sum()) + 2 * B * Hq * 256 + \
        2 * B * Hq * decode_partials(L.decode_splits) * 520
    L_ctx = w["prompt"] + w["gen"]
    return {"workload": "kara: B 64, GQA 32/8, prompt 16384 + 8192 generated, window 512, "
                        "retention 20 %, Token2Chunk alpha 3 gamma 16, an event every 64 steps",
            "cache_build_ms": build_ms, "events": cache.n_events, "decode_us": t * 1e6,
            "kv_tokens_per_s": B * L_ctx / t, "stored_tokens": int(n.sum()),
            "achieved_GBs": alg / t / 1e9, "pct_of_peak_hbm": 100.0 * alg / t / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": alg}


def bench_pipeline(a, kvc, stream):
    """The last generation steps of the Kara workload through the compression
    pipeline (kv_pipe_*), as a serving loop runs them: one decode step per
    token, the host waiting for each step's output (a sampler needs it), an
    event every 64 tokens.  Run three times from the same state: events
    compressed inside the step that fires them (blocking); on the pipeline's
    own stream, switched in when done (asynchronous); the same with each event
    kernel capped at PIPE_EVENT_WAVES waves in flight, so that decode keeps
    most of the GPU.  Reports each run's total time (ending with a drain, so
    every event is inside it) and the latency of single steps; the final
    caches are compared byte for byte, and one event's compression is timed
    on its own."""
    from compressed_kv_cache_compress_amd import gen, kara
    k = gen.KARA
    dev = torch.device("cuda:0")
    w = gen.make_kara(seed=a.seed, device=dev)
    n = a.pipe_steps
    prot, delta = k["protect"], k["delta"]
    start = w["gen"] - n - prot
    scale = float(np.float32(1.0 / math.sqrt(128.0)))
    runs, pipes = {}, {}
    runs_cfg = ((kvc.PIPE_SYNC, "blocking", 0), (kvc.PIPE_ASYNC, "async", 0),
                (kvc.PIPE_ASYNC, "async_capped", PIPE_EVENT_WAVES))
    for mode, name, cap in runs_cfg:
        print(f"[bench] pipeline {name}: {n} steps from generated token {start}", file=sys.stderr,
              flush=True)
        kp = kara.KaraPipeline(w["K"], w["V"], w["Qall"], prompt=w["prompt"], start=start,
                               window=k["window"], delta=delta, protect=prot,
                               retention_pct=k["retention_pct"], alpha=k["alpha"],
                               gamma=k["gamma"], scale=scale, mode=mode, steps=n + prot,
                               event_max_waves=cap)
        kp.step(prot, decode=False)
        torch.cuda.synchronize()
        lat = np.zeros(n)
        t0 = time.perf_counter()
        for i in range(n):
            t = time.perf_counter()
            kp.step(1)
            stream.synchronize()
            lat[i] = time.perf_counter() - t
        kp.pipe.drain()
        torch.cuda.synchronize()
        total = time.perf_counter() - t0
        runs[name] = dict(total_ms=total * 1e3, p50_ms=float(np.percentile(lat, 50) * 1e3),
                          p99_ms=float(np.percentile(lat, 99) * 1e3), max_ms=float(lat.max() * 1e3),
                          host_waits=kp.pipe.stats()["host_waits"],
                          events=kp.pipe.stats()["events_fired"])
        pipes[name] = kp
    a_ = pipes["blocking"]
    streams = a_.B * a_.Hkv
    lo = a_.cfg.events_offset
    hi = lo + a_.cfg.max_events * a_.layout.event_bytes
    same = all(bool(torch.equal(a_.desc, b_.desc)) and bool(torch.equal(
        a_.packed.view(streams, -1)[:, lo:hi], b_.packed.view(streams, -1)[:, lo:hi]))
        for b_ in pipes.values())
    # one event's compression on its own (same window shape, scratch output)
    pe = kvc.KvParams(batch=a_.B, n_q_heads=a_.Hq, n_kv_heads=a_.Hkv, n_ctx=k["window"],
                      region_begin=k["window"] - prot - delta, region_len=delta,
                      seg_tokens=delta, n_win=k["window"], strategies=[(a_.T, 128)],
                      budget_bytes=4 * delta * 128, t2c_alpha=k["alpha"], t2c_gamma=k["gamma"],
                      scale=scale, kv_stream_stride=a_.L * 128, qw_head_stride=a_.L * 128,
                      store_logits=1)
    _, Le = kvc.kv_layout_query(pe)
    sp = torch.empty(Le.packed_bytes_max, dtype=torch.uint8, device=dev)
    sd = torch.zeros(streams * 16, dtype=torch.uint8, device=dev)
    sw = torch.empty(Le.compress_ws_bytes, dtype=torch.uint8, device=dev)
    w0 = a_.L - k["window"]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(6)]
    for e in ev:
        e[0].record(stream)
        kvc.kv_compress(pe, w["K"][:, :, w0:], w["V"][:, :, w0:], w["Qall"][:, :, w0:], None,
                        sp, sd, None, None, None, sw)
        e[1].record(stream)
    torch.cuda.synchronize()
    t_event = float(np.mean([e[0].elapsed_time(e[1]) for e in ev[1:]]))
    for kp in pipes.values():
        kp.close()
    return {"workload": f"kara generation through the pipeline: B 64, GQA 32/8, the last {n} of "
                        "8192 generated tokens, one decode step each with the host waiting for "
                        "its output, an event every 64 tokens, 64-token protected tail, 4 pages",
            "steps": n, "event_ms": t_event, "blocking": runs["blocking"],
            "async": runs["async"], "async_capped": dict(runs["async_capped"],
                                                         event_max_waves=PIPE_EVENT_WAVES),
            "identical_final_cache": same}


ROT_SPAN = 4096  # tokens per rotation span in the per-span measurement


def _rotated_run(kvc, K, V, Qw, q, B, Hq, Hkv, N, S, W, strategies, budget, scale, stream,
                 rot_span, steps):
    """kv_compress_rotated + kv_attend_decode_rotated with one R per stream
    (rot_span 0) or per span: compress and decode times with HIP events on
    the launch stream, the objective of the chosen strategies, packed bytes
    and the bytes of the rotations themselves (fp32, 2 x 64 KB per span)."""
    p = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=N, seg_tokens=S, n_win=W,
                     strategies=strategies, budget_bytes=budget, scale=float(scale), rotate=1,
                     store_logits=1, rot_span=rot_span)
    _, L = kvc.kv_layout_query(p)
    dev = q.device
    streams = B * Hkv
    n_span = N // (rot_span or N)
    packed = torch.empty(L.packed_bytes_max, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * L.n_seg * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    obj = torch.empty((streams, L.n_seg, len(strategies)), dtype=torch.float32, device=dev)
    rot = torch.empty((streams, n_span, 2, 128, 128), dtype=torch.float32, device=dev)
    cws = torch.empty(L.compress_ws_bytes, dtype=torch.uint8, device=dev)
    dws = torch.empty(L.decode_ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(steps)]
    kvc.kv_compress_rotated(p, K, V, Qw, None, packed, desc, used, None, obj, rot, cws)
    for e in ev:
        e[0].record(stream)
        kvc.kv_compress_rotated(p, K, V, Qw, None, packed, desc, used, None, None, rot, cws)
        e[1].record(stream)
    dv = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(20)]
    for i in range(23):
        e = dv[i - 3] if i >= 3 else None
        if e:
            e[0].record(stream)
        kvc.kv_attend_decode_rotated(p, q, packed, desc, None, rot, out, None, dws)
        if e:
            e[1].record(stream)
    torch.cuda.synchronize()
    dh = desc.cpu().numpy().view(kvc.DESC_DTYPE).reshape(streams, L.n_seg)
    oh = obj.cpu().numpy()
    chosen = np.take_along_axis(oh, dh["strategy"].astype(np.int64)[..., None], axis=2)[..., 0]
    t_dec = float(np.mean([e[0].elapsed_time(e[1]) for e in dv])) * 1e-3
    alg = algorithmic_decode_bytes(dh.ravel(), B, Hq, L.decode_splits, rotated=True)
    packed_bytes = int(used.sum().item())
    rot_bytes = streams * n_span * 2 * 128 * 128 * 4
    return {"rot_span": rot_span or N, "spans_per_stream": n_span,
            "compress_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
            "decode_us": t_dec * 1e6, "kv_tokens_per_s": B * N / t_dec,
            "decode_splits": int(L.decode_splits), "achieved_GBs": alg / t_dec / 1e9,
            "packed_bytes": packed_bytes, "rotation_bytes": rot_bytes,
            "packed_plus_rotation_pct_of_dense": 100.0 * (packed_bytes + rot_bytes) / (B * Hkv * N * 512),
            "strategy_histogram": np.bincount(dh["strategy"].ravel(),
                                              minlength=len(strategies)).tolist(),
            "objective_mean": float(chosen.mean())}


def _plain_objective(kvc, K, V, Qw, B, Hq, Hkv, N, S, W, strategies, budget, scale):
    """Mean objective of the strategies plain kv_compress chooses."""
    p = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=N, seg_tokens=S, n_win=W,
                     strategies=strategies, budget_bytes=budget, scale=float(scale),
                     store_logits=1)
    _, L = kvc.kv_layout_query(p)
    dev = K.device
    streams = B * Hkv
    packed = torch.empty(L.packed_bytes_max, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * L.n_seg * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    obj = torch.empty((streams, L.n_seg, len(strategies)), dtype=torch.float32, device=dev)
    cws = torch.empty(L.compress_ws_bytes, dtype=torch.uint8, device=dev)
    kvc.kv_compress(p, K, V, Qw, None, packed, desc, used, None, obj, cws)
    torch.cuda.synchronize()
    dh = desc.cpu().numpy().view(kvc.DESC_DTYPE).reshape(streams, L.n_seg)
    chosen = np.take_along_axis(obj.cpu().numpy(), dh["strategy"].astype(np.int64)[..., None],
                                axis=2)[..., 0]
    return float(chosen.mean()), int(used.sum().item())


def bench_rotation(a, kvc, K, V, Qw, q, B, Hq, Hkv, N, S, W, strategies, budget, scale, stream,
                   plain_objective, plain_desc, steps=3):
    """The SVD rotation before channel selection (kv_compress_rotated, decoded
    by kv_attend_decode_rotated) on the headline workload with one R per
    stream, then on an off-axis copy of it (every 4096-token block of K and
    V multiplied by its own random orthogonal matrix, gen.offaxis_blocks) in
    three ways: no rotation, one R per stream, one R per 4096-token span.
    The objective (attention mass kept, weighted by the vector energy kept)
    of the chosen strategies shows what each rotation recovers; the bytes of
    the rotations are reported beside the packed bytes."""
    from compressed_kv_cache_compress_amd import gen
    pc = np.take_along_axis(plain_objective, plain_desc["strategy"].astype(np.int64)[..., None],
                            axis=2)[..., 0]
    args = (K, V, Qw, q, B, Hq, Hkv, N, S, W, strategies, budget, scale, stream)
    res = _rotated_run(kvc, *args, 0, steps)
    res["objective_mean_plain"] = float(pc.mean())
    print("[bench] rotation on the off-axis copy ...", file=sys.stderr, flush=True)
    K2 = gen.offaxis_blocks(K, ROT_SPAN, seed=a.seed + 1)
    V2 = gen.offaxis_blocks(V, ROT_SPAN, seed=a.seed + 2)
    args2 = (K2, V2) + args[2:]
    obj_plain, bytes_plain = _plain_objective(kvc, K2, V2, Qw, B, Hq, Hkv, N, S, W, strategies,
                                              budget, scale)
    off = {"workload": f"the headline workload with every {ROT_SPAN}-token block of K and V "
                       "multiplied by its own random orthogonal matrix",
           "plain": {"objective_mean": obj_plain, "packed_bytes": bytes_plain},
           "per_stream": _rotated_run(kvc, *args2, 0, steps),
           "per_span": _rotated_run(kvc, *args2, ROT_SPAN, steps)}
    del K2, V2
    torch.cuda.empty_cache()
    res["offaxis"] = off
    return res


def bench_stream_budget(a, kvc, K, V, Qw, q, B, Hq, Hkv, N, S, W, strategies, budget, scale,
                        stream, steps=3):
    """The same workload with the byte budget shared by each stream's segments
    (budget_scope = stream): compress and decode times, bytes and the chosen
    strategies; HIP events on the launch stream."""
    p = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=N, seg_tokens=S, n_win=W,
                     strategies=strategies, budget_bytes=budget, scale=float(scale),
                     budget_scope=1, store_logits=1)
    _, L = kvc.kv_layout_query(p)
    dev = q.device
    streams = B * Hkv
    packed = torch.empty(L.packed_bytes_max, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * L.n_seg * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    cws = torch.empty(L.compress_ws_bytes, dtype=torch.uint8, device=dev)
    dws = torch.empty(L.decode_ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for i in range(steps + 1):
        e = ev[i - 1] if i >= 1 else None
        if e:
            e[0].record(stream)
        kvc.kv_compress(p, K, V, Qw, None, packed, desc, used, None, None, cws)
        if e:
            e[1].record(stream)
        kvc.kv_attend_decode(p, q, packed, desc, None, out, None, dws)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    dh = desc.cpu().numpy().view(kvc.DESC_DTYPE)
    return {"budget_bytes_per_stream": int(L.n_seg) * int(budget),
            "compress_ms": float(np.mean([x[0].elapsed_time(x[1]) for x in ev])),
            "decode_us": float(np.mean([x[1].elapsed_time(x[2]) for x in ev])) * 1e3,
            "packed_bytes": int(used.sum().item()),
            "strategy_histogram": np.bincount(dh["strategy"], minlength=len(strategies)).tolist()}


def bench_graph(kvc, stream, reps=200, per_graph=20):
    """Decode on the Llama-3-8B-shaped layer (B 1, GQA 32/8, 32768 tokens,
    a few microseconds per call, so launch costs show): kv_attend_decode
    launched eagerly `reps` times, against a HIP graph holding `per_graph`
    decode calls replayed reps / per_graph times.  HIP events around each
    loop; per-call time."""
    from compressed_kv_cache_compress_amd import gen
    cfg = gen.CONFIGS["llama8b"]
    S = cfg["S"]
    dev = torch.device("cuda:0")
    w = gen.make_workload("llama8b", seed=0, device=dev)
    strategies = gen.table9(S)
    p = kvc.KvParams(batch=cfg["B"], n_q_heads=cfg["Hq"], n_kv_heads=cfg["Hkv"], n_ctx=cfg["N"],
                     seg_tokens=S, n_win=cfg["W"], strategies=strategies,
                     budget_bytes=gen.budget_bytes(cfg["budget_pct"], S),
                     scale=float(1.0 / math.sqrt(128.0)))
    _, L = kvc.kv_layout_query(p)
    streams = cfg["B"] * cfg["Hkv"]
    packed = torch.empty(L.packed_bytes_max, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * L.n_seg * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    cws = torch.empty(L.compress_ws_bytes, dtype=torch.uint8, device=dev)
    dws = torch.empty(L.decode_ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((cfg["B"], cfg["Hq"], 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg["B"], cfg["Hq"]), dtype=torch.float32, device=dev)
    kvc.kv_compress(p, w["K"], w["V"], w["Qw"], None, packed, desc, used, None, None, cws)
    torch.cuda.synchronize()
    ref = out.clone()
    kvc.kv_attend_decode(p, w["q"], packed, desc, None, ref, lse, dws)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        e0.record(s)
        for _ in range(n):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    dec = lambda: kvc.kv_attend_decode(p, w["q"], packed, desc, None, out, lse, dws)  # noqa: E731
    timed(dec, 20)
    eager_us = timed(dec, reps) / reps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            dec()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    graph_us = timed(g.replay, reps // per_graph) / reps
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.uint8), ref.view(torch.uint8)))
    del w, packed, cws, g
    torch.cuda.empty_cache()
    return {"workload": "llama8b", "decode_eager_us": eager_us, "decode_graph_us": graph_us,
            "decode_calls_per_graph": per_graph, "graph_output_equals_eager": same,
            "stored_tokens_per_stream": int(np.frombuffer(desc.cpu().numpy().tobytes(),
                                                           dtype=kvc.DESC_DTYPE)["n_tok"].astype(np.int64).sum() // streams)}


def bench_stage2(a, kvc, p, L, q, packed, desc, B, Hq, Hkv, N, stream):
    """Query-aware segment selection (decode-time stage 2) on the same cache:
    kv_summarize once, then per step kv_select_segments + kv_attend_decode
    over the kept descriptors; HIP events on the launch stream."""
    streams = B * Hkv
    n_seg = L.n_seg
    keep = max(1, int(round(n_seg * a.select_pct / 100.0)))
    dev = q.device
    summary = torch.empty((streams, n_seg, 2, 128), dtype=torch.int16, device=dev)
    out_desc = torch.zeros(streams * keep * 16, dtype=torch.uint8, device=dev)
    out_n = torch.empty(streams, dtype=torch.int32, device=dev)
    score = torch.empty((streams, n_seg), dtype=torch.float32, device=dev)
    ps = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_desc_per_stream=n_seg,
                      scale=p.p.scale)
    pd = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_desc_per_stream=keep,
                      scale=p.p.scale)
    _, Ld = kvc.kv_layout_query(pd)
    dws = torch.empty(max(Ld.decode_ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    kvc.kv_summarize(ps, packed, desc, None, summary)  # first launch loads the kernel
    e0.record(stream)
    kvc.kv_summarize(ps, packed, desc, None, summary)
    e1.record(stream)
    torch.cuda.synchronize()
    t_sum = e0.elapsed_time(e1) * 1e3
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(a.steps)]
    for i in range(a.warmup + a.steps):
        e = ev[i - a.warmup] if i >= a.warmup else None
        if e:
            e[0].record(stream)
        kvc.kv_select_segments(ps, q, summary, desc, None, keep, out_desc, out_n, score)
        if e:
            e[1].record(stream)
        kvc.kv_attend_decode(pd, q, packed, out_desc, out_n, out, None, dws)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    sel_us = float(np.mean([x[0].elapsed_time(x[1]) for x in ev])) * 1e3
    dec_us = float(np.mean([x[1].elapsed_time(x[2]) for x in ev])) * 1e3
    kd = out_desc.cpu().numpy().view(kvc.DESC_DTYPE).reshape(streams, keep)
    n = out_n.cpu().numpy()
    live = np.concatenate([kd[s, :n[s]] for s in range(streams)])
    kept_tok = int(live["n_tok"].astype(np.int64).sum())
    alg = algorithmic_decode_bytes(live, B, Hq, Ld.decode_splits)
    return {"keep_segments_per_stream": keep, "keep_pct": a.select_pct,
            "summarize_us_once": t_sum, "select_us": sel_us, "decode_us": dec_us,
            "select_plus_decode_us": sel_us + dec_us,
            "kept_tokens": kept_tok,
            "decode_algorithmic_bytes": alg,
            "decode_achieved_GBs": alg / (dec_us * 1e-6) / 1e9,
            "kv_tokens_per_s": B * N / ((sel_us + dec_us) * 1e-6)}


def bench_read_stream(kvc, buf, nbytes, stream, reps=20):
    """Achievable HBM read bandwidth on this machine: kv_read_stream (a plain
    16-byte-load stream over every CU) over as many bytes as one decode
    reads, HIP events around `reps` back-to-back launches."""
    nbytes = nbytes // 16 * 16
    sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    for _ in range(3):
        kvc.kv_read_stream(buf, nbytes, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        kvc.kv_read_stream(buf, nbytes, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    return {"kernel": "k_read_stream", "bytes": nbytes, "us": t * 1e6, "GBs": nbytes / t / 1e9,
            "pct_of_peak_hbm": 100.0 * nbytes / t / 1e9 / PEAK_HBM_GBS}


CPU_THREADS_CAP = 16  # the host share of one GPU


def host_description():
    """Host cores the oracle may use, and the CPU model."""
    try:
        n_aff = len(os.sched_getaffinity(0))
    except AttributeError:
        n_aff = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n_aff, os.cpu_count() or 1, model


def cpu_baseline(w, S, strategies, budget, scale, n_streams=4, decode_s=10.0):
    """Oracle as it stands on a bounded sample of the workload, on every host
    core it may use (at most CPU_THREADS_CAP): n_streams streams compressed
    one after the other, each by the oracle's compress with its OpenMP loops
    on all those threads; then fp64 decode of those streams by a pool of that
    many threads (each call decodes one stream; ctypes releases the GIL),
    repeated for about decode_s seconds.  The value is KV tokens decoded per
    second over the pool."""
    from concurrent.futures import ThreadPoolExecutor

    from compressed_kv_cache_compress_amd import gen
    from oracle import oracle as O
    n_aff, n_cpu, model = host_description()
    threads = max(1, min(n_aff, CPU_THREADS_CAP))
    G, Hkv = w["G"], w["Hkv"]
    streams = list(range(min(n_streams, w["K"].shape[0] * Hkv)))
    comp, t_comp = {}, 0.0
    for s in streams:
        b, h = divmod(s, Hkv)
        Ks, Vs = gen.u16(w["K"][b, h]), gen.u16(w["V"][b, h])
        Qs = gen.u16(w["Qw"][b, h * G:(h + 1) * G])
        t0 = time.perf_counter()
        comp[s] = O.compress_stream(Ks, Vs, Qs, S=S, strategies=strategies, budget_bytes=budget,
                                    scale=scale, n_threads=threads)
        t_comp += time.perf_counter() - t0
    qs = {s: gen.u16(w["q"][s // Hkv, (s % Hkv) * G:(s % Hkv + 1) * G]) for s in streams}
    n_ctx = w["K"].shape[2]

    def one(i):
        s = streams[i % len(streams)]
        O.decode_stream(qs[s], comp[s]["packed"], comp[s]["desc"], scale)
        return 1

    calls = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            calls += sum(ex.map(one, range(calls, calls + threads)))
            td = time.perf_counter() - t0
            if td > decode_s:
                break
    return dict(value=n_ctx * calls / td, unit="KV tokens/s", cores=threads, kind="oracle",
                sample=f"{len(streams)} streams (b, kv head) = {streams} of the workload, "
                       f"{n_ctx} tokens x {G} q heads each: oracle compress of each on "
                       f"{threads} OpenMP threads ({t_comp:.2f} s for all, "
                       f"{n_ctx * len(streams) / t_comp:.4g} tokens/s), then {calls} oracle fp64 "
                       f"decodes of them on a pool of {threads} threads in {td:.2f} s; host: "
                       f"{model}, nproc {n_cpu}, {n_aff} cores in the affinity mask",
                compress_tokens_per_s=n_ctx * len(streams) / t_comp, compress_threads=threads,
                host_cpu=model, host_nproc=n_cpu, host_affinity_cores=n_aff)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU (asked for {a.gpus}); the "
              "streams are independent, so batch or head sharding would need no exchange, but "
              "no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    import compressed_kv_cache_compress_amd as kvc
    from compressed_kv_cache_compress_amd import gen, runtime

    kvc.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = gen.CONFIGS[a.config]
    S, W, B, N = cfg["S"], cfg["W"], cfg["B"], cfg["N"]
    Hq, Hkv = cfg["Hq"], cfg["Hkv"]
    strategies = gen.table9(S)
    budget = gen.budget_bytes(cfg["budget_pct"], S)
    scale = np.float32(1.0 / math.sqrt(128.0))
    print(f"[bench] generating {a.config} on {dev} ...", file=sys.stderr, flush=True)
    w = gen.make_workload(a.config, seed=a.seed, device=dev)
    K, V, Qw, q = w["K"], w["V"], w["Qw"], w["q"]

    # the first scoring pass stores the window-query logits for the second
    # (17 GB of workspace at batched128k instead of recomputing 5.5e11 fma)
    p = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=N, seg_tokens=S, n_win=W,
                     strategies=strategies, budget_bytes=budget, scale=float(scale),
                     decode_splits=a.decode_splits, store_logits=1)
    _, L = kvc.kv_layout_query(p)
    streams = B * Hkv
    packed = torch.empty(L.packed_bytes_max, dtype=torch.uint8, device=dev)
    desc = torch.zeros(streams * L.n_seg * 16, dtype=torch.uint8, device=dev)
    used = torch.zeros(streams, dtype=torch.int64, device=dev)
    cws = torch.empty(L.compress_ws_bytes, dtype=torch.uint8, device=dev)
    dws = torch.empty(L.decode_ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(a.steps)]
    # between compress and decode every step reads an unrelated buffer four
    # times the Infinity Cache (MALL, 256 MB), outside the decode events, so
    # that decode reads the packed cache from HBM and not from what k_pack
    # left in the MALL
    evict = torch.ones(EVICT_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def step(e=None, evict_mall=True):
        if e:
            e[0].record(stream)
        kvc.kv_compress(p, K, V, Qw, None, packed, desc, used, None, None, cws)
        if e:
            e[1].record(stream)
        if evict_mall:
            kvc.kv_read_stream(evict, EVICT_BYTES, sink)
        if e:
            e[2].record(stream)
        kvc.kv_attend_decode(p, q, packed, desc, None, out, lse, dws)
        if e:
            e[3].record(stream)

    print(f"[bench] warmup {a.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    comp_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    # beside the headline: decode right after the pack (no eviction: part of
    # the cache may come from the MALL), and decode after decode
    ev_nc = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(10)]
    for e in ev_nc:
        step(e, evict_mall=False)
    ev_dd = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(20)]
    for e in ev_dd:
        e[0].record(stream)
        kvc.kv_attend_decode(p, q, packed, desc, None, out, lse, dws)
        e[1].record(stream)
    torch.cuda.synchronize()
    dec_after_pack_us = float(np.median([e[2].elapsed_time(e[3]) for e in ev_nc])) * 1e3
    dec_after_dec_us = float(np.median([e[0].elapsed_time(e[1]) for e in ev_dd])) * 1e3
    del evict
    # beside the headline: the same compress with the logits recomputed
    p_re = kvc.KvParams(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, n_ctx=N, seg_tokens=S, n_win=W,
                        strategies=strategies, budget_bytes=budget, scale=float(scale))
    kvc.kv_compress(p_re, K, V, Qw, None, packed, desc, used, None, None, cws)
    er = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    er[0].record(stream)
    for i in range(3):
        kvc.kv_compress(p_re, K, V, Qw, None, packed, desc, used, None, None, cws)
    er[1].record(stream)
    torch.cuda.synchronize()
    comp_re_ms = er[0].elapsed_time(er[1]) / 3
    kvc.kv_compress(p, K, V, Qw, None, packed, desc, used, None, None, cws)
    torch.cuda.synchronize()

    sbud = None
    if not a.no_stream_budget:
        sbud = bench_stream_budget(a, kvc, K, V, Qw, q, B, Hq, Hkv, N, S, W, strategies, budget,
                                   scale, stream)
    rotation = None
    if not a.no_rotate:
        print("[bench] rotation ...", file=sys.stderr, flush=True)
        pobj = torch.empty((B * Hkv, L.n_seg, len(strategies)), dtype=torch.float32, device=dev)
        kvc.kv_compress(p, K, V, Qw, None, packed, desc, used, None, pobj, cws)
        torch.cuda.synchronize()
        rotation = bench_rotation(a, kvc, K, V, Qw, q, B, Hq, Hkv, N, S, W, strategies, budget,
                                  scale, stream, pobj.cpu().numpy(),
                                  desc.cpu().numpy().view(kvc.DESC_DTYPE).reshape(B * Hkv, -1))
        del pobj
        torch.cuda.empty_cache()
    stage2 = None
    if a.select_pct > 0:
        stage2 = bench_stage2(a, kvc, p, L, q, packed, desc, B, Hq, Hkv, N, stream)

    dh = desc.cpu().numpy().view(kvc.DESC_DTYPE)
    hist = np.bincount(dh["strategy"], minlength=len(strategies)).tolist()
    alg = algorithmic_decode_bytes(dh, B, Hq, L.decode_splits)
    t_dec = float(np.median(dec_ms)) * 1e-3
    achieved = alg / t_dec / 1e9
    print("[bench] read-stream reference ...", file=sys.stderr, flush=True)
    rstream = bench_read_stream(kvc, packed, alg, stream)
    traffic = measured_traffic(a.traffic) if a.config == "batched128k" and not a.decode_splits else None
    packed_total = int(used.sum().item())
    res = {
        "metric": "compressed decode attention: KV tokens/s and achieved HBM GB/s (% of peak)",
        "value": B * N / t_dec,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": wall * 1e3 / a.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 storage, fp32 accumulate (decode: bf16 MFMA inputs); fp32 selection",
        "data": "synthetic (seeded torch generator; gen.py recipe), inputs resident in HBM",
        "config": {"workload": a.config, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": 128, "context": N, "segment": S, "window": W,
                   "budget_pct": cfg["budget_pct"], "strategies": strategies,
                   "decode_splits": L.decode_splits, "parallelism": "single GPU"},
        "decode_us": t_dec * 1e6,
        "decode_us_mall_evicted": t_dec * 1e6,
        "decode_us_mean": float(dec_ms.mean()) * 1e3,
        "decode_us_after_pack_no_eviction": dec_after_pack_us,
        "decode_us_after_decode": dec_after_dec_us,
        "frac_after_pack_no_eviction": alg / (dec_after_pack_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "decode_us_p10_p90": [float(np.percentile(dec_ms, 10) * 1e3), float(np.percentile(dec_ms, 90) * 1e3)],
        "compress_ms": float(comp_ms.mean()),
        "compress_ms_logits_recomputed": comp_re_ms,
        "achieved_GBs": achieved,
        "pct_of_peak_hbm": 100.0 * achieved / PEAK_HBM_GBS,
        "stored_tokens_per_s": float(dh["n_tok"].astype(np.int64).sum()) / t_dec,
        "packed_bytes": packed_total,
        "dense_kv_bytes": B * Hkv * N * 512,
        "strategy_histogram": hist,
        "roofline": {"kernel": "kv_attend_decode (k_decode_split + k_decode_reduce)",
                     "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg,
                     "frac_of_read_stream": achieved / rstream["GBs"]},
        "read_stream": rstream,
        "value_basis": "B*context / median decode time over the timed steps; each timed step "
                       "runs kv_compress (compress_ms), then reads an unrelated 1 GiB buffer "
                       "(outside the decode events) so that decode starts with the packed cache "
                       "out of the 256 MB Infinity Cache, then kv_attend_decode",
    }
    if stage2 is not None:
        res["stage2"] = stage2
    if rotation is not None:
        res["rotation"] = rotation
    if sbud is not None:
        res["stream_budget"] = sbud
    wc = {k: (v[:1].cpu() if torch.is_tensor(v) else v) for k, v in w.items()}
    if not a.no_kara:
        print("[bench] kara cache and decode ...", file=sys.stderr, flush=True)
        del w, K, V, Qw, packed, cws, dws
        torch.cuda.empty_cache()
        res["kara"] = bench_kara(a, kvc, stream)
    if not a.no_graph:
        print("[bench] HIP-graph decode (Llama-3-8B-shaped layer) ...", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        res["graph"] = bench_graph(kvc, stream)
    if a.pipe_steps > 0:
        torch.cuda.empty_cache()
        res["pipeline"] = bench_pipeline(a, kvc, stream)
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wc, S, strategies, budget, scale)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
