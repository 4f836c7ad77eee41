"""Kara compression events written out from the reading of the pages (test
infrastructure: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module).  It shares no code with
the library's own event list.

KARA review page: "What carries the argument" -- only the recent window is
scored and compressed; the free-parameter ledger -- window |W|, protected
buffer |U| of the newest tokens left uncompressed, retention ratio r and the
compression period delta.

Reading (stated where the pages are silent):
  * generation starts after a prompt of `prompt` tokens; the prompt itself is
    never compressed;
  * event k (k = 1, 2, ...) happens once delta * k tokens have been generated,
    at sequence length L_k = prompt + delta * k;
  * it scores the window of the last `window` positions, [L_k - window, L_k),
    with their original keys and queries;
  * it compresses the `seg` tokens just older than the protected tail:
    [L_k - protect - seg, L_k - protect);
  * an event whose region starts inside the prompt is skipped;
  * T = round(r * seg) kept tokens, rounded half up: (r% * seg + 50) div 100.
"""


def kept_tokens(retention_pct, seg):
    """Tokens an event keeps of its region: r * seg rounded half up."""
    return (retention_pct * seg + 50) // 100


def events(prompt, generated, *, window, delta, protect, seg):
    """Every event that compresses generated tokens, in firing order, as dicts
    with the sequence length L at which it fires, the window [w0, L), the
    region [r0, r1) in sequence positions and the region's first position
    inside the window (rb = r0 - w0).  `skipped` lists the lengths of the
    events whose region lies in the prompt."""
    out, skipped = [], []
    k = 1
    while delta * k <= generated:
        L = prompt + delta * k
        r1 = L - protect
        r0 = r1 - seg
        if r0 < prompt:
            skipped.append(L)
        else:
            w0 = L - window
            assert w0 >= 0 and r0 >= w0, "the window must hold the region"
            out.append(dict(L=L, w0=w0, r0=r0, r1=r1, rb=r0 - w0))
        k += 1
    return out, skipped


def final_tokens(prompt, generated, *, delta, protect, seg, retention_pct):
    """Tokens per stream once every event has run: the dense prompt, T per
    event and the dense tokens no event covers (the protected tail and any
    generated tokens past the last region)."""
    assert delta == seg, "one region per period: the regions tile the generated tokens"
    ev, _ = events(prompt, generated, window=protect + seg, delta=delta, protect=protect, seg=seg)
    T = kept_tokens(retention_pct, seg)
    covered = len(ev) * seg
    return prompt + len(ev) * T + (generated - covered)
