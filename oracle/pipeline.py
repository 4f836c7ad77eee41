"""Schedule of the incremental compression pipeline, written out from the
reading of the pages (test infrastructure: only the tests, the package's
smoke check and the benchmark's CPU-baseline leg may import this module).

MosaicKV review page, Fig. 1 and Fig. 5 captions: a segment is compressed
asynchronously once it is complete, and a switch then replaces its temporary
form with the final one without blocking decode.  KARA review page,
free-parameter ledger: compression every delta tokens, a protected buffer U
of recent tokens that stays uncompressed.

Reading (stated where the pages are silent):
  * tokens are appended one step at a time; the temporary form of a segment
    is its tokens at full width (every token, all 128 channels);
  * an event fires in the step after which the pipeline's token count g is a
    multiple of `period` with g >= protect + period; its region is tokens
    [g - protect - period, g - protect) (one page of `period` tokens);
  * deterministic switching: an event fired in step i is in effect for the
    decode of step i + lag and later (lag 0: that same step, the blocking
    order); it is also switched, at the latest, before the step that writes
    its page's memory again, i.e. the step appending token (page + pages) *
    period;
  * the decode of a step attends to the prefix, every switched event's final
    segment and every appended token whose event is not switched.
"""


def schedule(step_tokens, *, period, protect, pages, lag):
    """step_tokens: tokens appended by each step (a step stays inside one
    page).  Returns one dict per step: g (tokens after the step), fired
    (event index or None), switched (events in effect for the step's decode,
    in firing order), regions (event -> (first token, end))."""
    regions = []      # event -> (start, end)
    fire_step = []    # event -> step that fired it
    out = []
    g = 0
    for i, n in enumerate(step_tokens):
        assert n >= 1 and g % period + n <= period, "a step stays inside one page"
        first = g  # first token appended by this step
        g += n
        fired = None
        if g % period == 0 and g >= protect + period:
            fired = len(regions)
            regions.append((g - protect - period, g - protect))
            fire_step.append(i)
        switched = []
        for e, (r0, _) in enumerate(regions):
            reuse_token = (r0 // period + pages) * period
            if fire_step[e] + lag <= i or first >= reuse_token:
                switched.append(e)
        out.append(dict(g=g, fired=fired, switched=switched, regions=dict(enumerate(regions))))
    return out


def state_tokens(entry):
    """Token ranges of the pipeline's own tokens that a step's decode sees at
    full width: every appended token outside the switched regions, as
    (start, end) ranges in order."""
    g = entry["g"]
    cut = sorted(entry["regions"][e] for e in entry["switched"])
    ranges, t = [], 0
    for r0, r1 in cut:
        if r0 > t:
            ranges.append((t, r0))
        t = max(t, r1)
    if g > t:
        ranges.append((t, g))
    return ranges
