"""The Kara event schedule, pinned to hand-worked positions (CPU only).

KARA review page (arXiv 2607.01237): "What carries the argument" -- only the
recent window is scored and compressed; free-parameter ledger -- window |W|,
protected buffer |U|, retention r, compression period delta.

Two copies of the schedule exist and share no code: the oracle's
(oracle/kara.py, an event loop) and the library's host driver
(compressed_kv_cache_compress_amd/kara.py, a closed form for the first event).
Both are compared with tests/golden/kara_schedule.json, worked out by hand,
so that a one-token shift of the window, the region or the first event in
either copy fails here; the GPU tests build the expected cache from the
oracle's copy only.
"""
import json
import os

import pytest

from compressed_kv_cache_compress_amd import kara as product
from oracle import kara as OK

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kara_schedule.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _expected(c, got):
    if "events" in c:
        return c["events"]
    assert len(got) == c["n_events"]
    return [c["first"]] + [None] * (c["n_events"] - 2) + [c["last"]]


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"prompt{c['prompt']}")
def test_oracle_schedule_golden(c):
    ev, skipped = OK.events(c["prompt"], c["generated"], window=c["window"], delta=c["delta"],
                            protect=c["protect"], seg=c["seg"])
    assert len(ev) == c["n_events"]
    assert skipped == c["skipped"]
    assert OK.kept_tokens(c["retention_pct"], c["seg"]) == c["T"]
    for g, e in zip(ev, _expected(c, ev)):
        if e is not None:
            assert g == e
    # consecutive events move by one period; every region lies in its window
    for a, b in zip(ev, ev[1:]):
        assert b["L"] - a["L"] == c["delta"] and b["r0"] - a["r0"] == c["delta"]
    for e in ev:
        assert e["w0"] <= e["r0"] and e["r1"] + c["protect"] == e["L"] and e["r0"] >= c["prompt"]
    assert OK.final_tokens(c["prompt"], c["generated"], delta=c["delta"], protect=c["protect"],
                           seg=c["seg"], retention_pct=c["retention_pct"]) == c["final_tokens"]


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"prompt{c['prompt']}")
def test_library_schedule_golden(c):
    """The library's host-side event list (what kara.build_cache and
    KaraPipeline run) against the same hand-worked positions."""
    ev, T = product.event_schedule(c["prompt"], c["generated"], window=c["window"],
                                   delta=c["delta"], protect=c["protect"], seg=c["seg"],
                                   retention_pct=c["retention_pct"])
    assert T == c["T"] and len(ev) == c["n_events"]
    for (L, w0, rb), e in zip(ev, _expected(c, ev)):
        if e is not None:
            assert (L, w0, rb) == (e["L"], e["w0"], e["rb"])
