// kvc_pipe.cpp -- host side of the incremental, asynchronous compression
// pipeline (MosaicKV review page: Fig. 1 and Fig. 5 captions, compression
// off the decode path with a non-blocking switch from the temporary to the
// final form of a segment; Fig. 7 caption, double compression buffering.
// KARA review page, free-parameter ledger: period delta, protected buffer U).
//
// Per stream the decode list is [prefix | event slots | page slots]:
//   * tokens are appended to dense pages (kv_append) on the decode stream;
//   * when a page is complete and `protect` tokens follow it, its event is
//     fired: kv_compress of that page's tokens, scored by the window, runs on
//     the pipeline's own stream and writes the final segment into the next
//     event slot's bytes and a staged descriptor;
//   * the switch (one kernel on the decode stream) copies the staged
//     descriptor into the event slot and empties the page slot, so every
//     decode sees either the page or the final segment, never both;
//   * a page's memory is reused `pages` pages later, after its switch.
// The host never blocks unless a page is needed again before its event has
// finished (counted in host_waits).  No device memory is allocated here.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>

#include "kvc_internal.h"

using namespace kvc;

namespace {

constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
bool pow2(uint64_t x) { return x && !(x & (x - 1)); }
bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvc_status streams_of(const kvc_params* p, int* streams) {
  if (!p || p->struct_size != sizeof(kvc_params)) return KVC_E_INVALID;
  if (p->head_dim != KVC_HEAD_DIM) return KVC_E_UNSUPPORTED;
  if (p->batch == 0 || p->n_kv_heads == 0) return KVC_E_INVALID;
  const uint64_t s = (uint64_t)p->batch * p->n_kv_heads;
  if (s > 65535u) return KVC_E_UNSUPPORTED;
  *streams = (int)s;
  return KVC_OK;
}

struct Resolved {
  kvc_layout cl;          // kv_layout_query of the event compression (+ decode list)
  kvc_pipe_layout pl;
  int streams;
};

kvc_status resolve(const kvc_params* p, const kvc_pipe_config* c, Resolved* r) {
  if (!c || c->struct_size != sizeof(kvc_pipe_config)) return KVC_E_INVALID;
  kvc_status st = streams_of(p, &r->streams);
  if (st != KVC_OK) return st;
  const uint32_t period = p->seg_tokens;
  if (!pow2(period) || c->protect % period) return KVC_E_INVALID;
  if (p->region_len != period || p->n_ctx < c->protect + period ||
      p->region_begin != p->n_ctx - c->protect - period)
    return KVC_E_INVALID;
  const uint32_t kp = c->protect / period;
  if (c->pages < kp + 2 || c->pages > 4096 || c->max_events == 0) return KVC_E_INVALID;
  if (c->mode > KVC_PIPE_LAG) return KVC_E_INVALID;
  if (c->mode == KVC_PIPE_LAG && (uint64_t)c->switch_lag > (uint64_t)(c->pages - kp - 1) * period)
    return KVC_E_INVALID;
  const uint64_t per = (uint64_t)c->prefix_desc + c->max_events + c->pages;
  if (per > 65535u) return KVC_E_UNSUPPORTED;
  if (p->desc_stream_stride && p->desc_stream_stride != per) return KVC_E_INVALID;
  if (c->events_offset % 16 || c->pages_offset % 16) return KVC_E_ALIGN;
  kvc_params q = *p;
  q.max_desc_per_stream = (uint32_t)per;
  std::memset(&r->cl, 0, sizeof r->cl);
  st = kv_layout_query(&q, &r->cl);
  if (st != KVC_OK) return st;
  kvc_pipe_layout& L = r->pl;
  std::memset(&L, 0, sizeof L);
  L.desc_per_stream = (uint32_t)per;
  L.period = period;
  L.event_bytes = align_up(r->cl.max_seg_bytes, 16);
  L.page_bytes = 2ull * period * KVC_HEAD_DIM * 2;
  const uint64_t ev_end = c->events_offset + (uint64_t)c->max_events * L.event_bytes;
  const uint64_t pg_end = c->pages_offset + (uint64_t)c->pages * L.page_bytes;
  if (c->events_offset < pg_end && c->pages_offset < ev_end) return KVC_E_INVALID;  // overlap
  L.stream_bytes_min = align_up(ev_end > pg_end ? ev_end : pg_end, 16);
  L.ws_bytes = align_up(r->cl.compress_ws_bytes, kAlign) +
               align_up((uint64_t)c->pages * r->streams * sizeof(kvc_seg_desc), kAlign) +
               align_up(r->cl.decode_ws_bytes, kAlign);
  L.decode_splits = r->cl.decode_splits;
  return KVC_OK;
}

}  // namespace

struct kvc_pipe {
  kvc_params ev;                         // event compression (strategies point at strat)
  kvc_strategy strat[KVC_MAX_STRATEGIES];
  kvc_params dec;                        // decode over the list
  kvc_pipe_config cfg;
  Resolved r;
  uint8_t* packed;
  kvc_seg_desc* list;
  uint8_t* cws;                          // event compression workspace
  kvc_seg_desc* staged;                  // [pages][streams]
  uint8_t* dws;                          // decode workspace
  hipStream_t dstream;                   // the caller's decode stream
  hipStream_t cstream;                   // the pipeline's compression stream
  hipEvent_t* ready;                     // [pages]: window inputs ready (decode stream)
  hipEvent_t* done;                      // [pages]: event compressed (compression stream)
  uint64_t g, steps, fired, switched, host_waits;
  bool broken;                           // a HIP call failed inside a step: only destroy is valid
  struct Pending {
    uint64_t event, step, page;          // event number, step that fired it, its page number
  };
  std::deque<Pending> pending;           // fired, not yet switched, oldest first
};

namespace {

uint32_t page_slot(const kvc_pipe* pp, uint64_t page) {
  return pp->cfg.prefix_desc + pp->cfg.max_events + (uint32_t)(page % pp->cfg.pages);
}

// Switches the oldest pending event on the decode stream.  wait_host: the
// page is needed now, so an event the host has not seen finish is waited for.
kvc_status switch_front(kvc_pipe* pp, bool wait_host) {
  const kvc_pipe::Pending e = pp->pending.front();
  const int ring = (int)(e.event % pp->cfg.pages);
  if (wait_host) {
    const hipError_t q = hipEventQuery(pp->done[ring]);
    if (q == hipErrorNotReady) {
      ++pp->host_waits;
      if (hipEventSynchronize(pp->done[ring]) != hipSuccess) return KVC_E_HIP;
    } else if (q != hipSuccess) {
      return KVC_E_HIP;
    }
  }
  // orders the switch after the compression on the device in every mode
  if (hipStreamWaitEvent(pp->dstream, pp->done[ring], 0) != hipSuccess) return KVC_E_HIP;
  SwitchPlan sp;
  sp.streams = pp->r.streams;
  sp.dstride = pp->r.pl.desc_per_stream;
  sp.final_slot = (int)(pp->cfg.prefix_desc + e.event);
  sp.clear_slot = (int)page_slot(pp, e.page);
  sp.staged = pp->staged + (uint64_t)ring * pp->r.streams;
  sp.list = pp->list;
  if (launch_switch(sp, pp->dstream) != hipSuccess) return KVC_E_HIP;
  pp->pending.pop_front();
  ++pp->switched;
  return KVC_OK;
}

void release(kvc_pipe* pp) {
  if (!pp) return;
  if (pp->cstream) (void)hipStreamSynchronize(pp->cstream);
  for (uint32_t i = 0; pp->ready && i < pp->cfg.pages; ++i)
    if (pp->ready[i]) (void)hipEventDestroy(pp->ready[i]);
  for (uint32_t i = 0; pp->done && i < pp->cfg.pages; ++i)
    if (pp->done[i]) (void)hipEventDestroy(pp->done[i]);
  delete[] pp->ready;
  delete[] pp->done;
  if (pp->cstream) (void)hipStreamDestroy(pp->cstream);
  delete pp;
}

}  // namespace

extern "C" {

kvc_status kv_append(const kvc_params* p, const uint16_t* k_new, const uint16_t* v_new,
                     uint32_t n_new, uint32_t fill, uint32_t capacity, uint64_t page_offset,
                     void* packed, kvc_seg_desc* page_desc, hipStream_t stream) {
  int streams;
  kvc_status st = streams_of(p, &streams);
  if (st != KVC_OK) return st;
  if (!k_new || !v_new || !packed || !page_desc || n_new == 0) return KVC_E_INVALID;
  if (!pow2(capacity) || capacity > 32768u || (uint64_t)fill + n_new > capacity)
    return KVC_E_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(packed) || !aligned16(page_desc))
    return KVC_E_ALIGN;
  if (page_offset % 16 || p->packed_stream_stride % 16 || p->kv_stream_stride % 8)
    return KVC_E_ALIGN;
  const uint64_t page_bytes = 2ull * capacity * KVC_HEAD_DIM * 2;
  if (streams > 1 && p->packed_stream_stride < page_bytes) return KVC_E_INVALID;
  const uint64_t src = p->kv_stream_stride ? p->kv_stream_stride : (uint64_t)n_new * KVC_HEAD_DIM;
  if (streams > 1 && src < (uint64_t)n_new * KVC_HEAD_DIM) return KVC_E_INVALID;
  AppendPlan a;
  a.streams = streams;
  a.n_new = (int)n_new;
  a.fill = (int)fill;
  a.capacity = (int)capacity;
  a.src_stride = src;
  a.page_offset = page_offset;
  a.pstride = p->packed_stream_stride;
  a.dstride = p->desc_stream_stride ? p->desc_stream_stride : 1u;
  a.k = k_new;
  a.v = v_new;
  a.packed = static_cast<uint8_t*>(packed);
  a.desc = page_desc;
  if (launch_append(a, stream) != hipSuccess) return KVC_E_HIP;
  return KVC_OK;
}

kvc_status kv_pipe_layout(const kvc_params* p, const kvc_pipe_config* cfg, kvc_pipe_layout* out) {
  if (!out) return KVC_E_INVALID;
  std::memset(out, 0, sizeof *out);
  Resolved r;
  const kvc_status st = resolve(p, cfg, &r);
  if (st != KVC_OK) return st;
  *out = r.pl;
  return KVC_OK;
}

kvc_status kv_pipe_create(const kvc_params* p, const kvc_pipe_config* cfg, void* packed,
                          kvc_seg_desc* desc, void* ws, size_t ws_bytes, hipStream_t stream,
                          kvc_pipe** out) {
  if (!out) return KVC_E_INVALID;
  *out = nullptr;
  Resolved r;
  kvc_status st = resolve(p, cfg, &r);
  if (st != KVC_OK) return st;
  if (!packed || !desc || !ws) return KVC_E_INVALID;
  if (!aligned16(packed) || !aligned16(desc) || !aligned16(ws)) return KVC_E_ALIGN;
  if (p->packed_stream_stride < r.pl.stream_bytes_min || p->packed_stream_stride % 16)
    return KVC_E_INVALID;
  if (ws_bytes < r.pl.ws_bytes) return KVC_E_WORKSPACE;
  if (p->n_strategies > KVC_MAX_STRATEGIES || !p->strategies) return KVC_E_INVALID;
  kvc_pipe* pp = new (std::nothrow) kvc_pipe();
  if (!pp) return KVC_E_INVALID;
  pp->cfg = *cfg;
  pp->r = r;
  pp->ev = *p;
  std::memcpy(pp->strat, p->strategies, sizeof(kvc_strategy) * p->n_strategies);
  pp->ev.strategies = pp->strat;
  pp->ev.desc_stream_stride = 1;          // staged descriptors: one per stream
  pp->ev.max_desc_per_stream = 0;
  std::memset(&pp->dec, 0, sizeof pp->dec);
  pp->dec.struct_size = sizeof(kvc_params);
  pp->dec.batch = p->batch;
  pp->dec.n_q_heads = p->n_q_heads;
  pp->dec.n_kv_heads = p->n_kv_heads;
  pp->dec.head_dim = p->head_dim;
  pp->dec.scale = p->scale;
  pp->dec.max_desc_per_stream = r.pl.desc_per_stream;
  pp->dec.decode_splits = p->decode_splits;
  pp->packed = static_cast<uint8_t*>(packed);
  pp->list = desc;
  uint8_t* w = static_cast<uint8_t*>(ws);
  pp->cws = w;
  w += align_up(r.cl.compress_ws_bytes, kAlign);
  pp->staged = reinterpret_cast<kvc_seg_desc*>(w);
  w += align_up((uint64_t)cfg->pages * r.streams * sizeof(kvc_seg_desc), kAlign);
  pp->dws = w;
  pp->dstream = stream;
  pp->ready = new (std::nothrow) hipEvent_t[cfg->pages]();
  pp->done = new (std::nothrow) hipEvent_t[cfg->pages]();
  if (!pp->ready || !pp->done) {
    release(pp);
    return KVC_E_INVALID;
  }
  bool ok = hipStreamCreateWithFlags(&pp->cstream, hipStreamNonBlocking) == hipSuccess;
  for (uint32_t i = 0; ok && i < cfg->pages; ++i)
    ok = hipEventCreateWithFlags(&pp->ready[i], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&pp->done[i], hipEventDisableTiming) == hipSuccess;
  ClearPlan c;
  c.streams = r.streams;
  c.first = (int)cfg->prefix_desc;
  c.count = (int)(cfg->max_events + cfg->pages);
  c.dstride = r.pl.desc_per_stream;
  c.list = desc;
  if (!ok || launch_clear(c, stream) != hipSuccess) {
    release(pp);
    return KVC_E_HIP;
  }
  *out = pp;
  return KVC_OK;
}

namespace {
kvc_status step_impl(kvc_pipe* pp, const uint16_t* k_new, const uint16_t* v_new, uint32_t n_new,
                     uint64_t new_stride, const uint16_t* win_K, const uint16_t* win_V,
                     const uint16_t* win_Q, const uint16_t* q, uint16_t* out, float* lse,
                     hipStream_t stream, bool* enqueued);
}  // namespace

kvc_status kv_pipe_step(kvc_pipe* pp, const uint16_t* k_new, const uint16_t* v_new,
                        uint32_t n_new, uint64_t new_stride, const uint16_t* win_K,
                        const uint16_t* win_V, const uint16_t* win_Q, const uint16_t* q,
                        uint16_t* out, float* lse, hipStream_t stream) {
  if (!pp) return KVC_E_INVALID;
  if (pp->broken) return KVC_E_HIP;
  bool enqueued = false;
  const kvc_status st = step_impl(pp, k_new, v_new, n_new, new_stride, win_K, win_V, win_Q, q,
                                  out, lse, stream, &enqueued);
  if (st != KVC_OK && enqueued) pp->broken = true;  // part of the step is on the stream
  return st;
}

kvc_status kv_pipe_drain(kvc_pipe* pp, hipStream_t stream) {
  if (!pp || stream != pp->dstream) return KVC_E_INVALID;
  if (pp->broken) return KVC_E_HIP;
  while (!pp->pending.empty()) {
    const kvc_status st = switch_front(pp, false);
    if (st != KVC_OK) {
      pp->broken = true;
      return st;
    }
  }
  return KVC_OK;
}

kvc_status kv_pipe_get_stats(const kvc_pipe* pp, kvc_pipe_stats* out) {
  if (!pp || !out) return KVC_E_INVALID;
  std::memset(out, 0, sizeof *out);
  out->steps = pp->steps;
  out->tokens = pp->g;
  out->events_fired = pp->fired;
  out->events_switched = pp->switched;
  out->host_waits = pp->host_waits;
  out->pending = (uint32_t)pp->pending.size();
  return KVC_OK;
}

kvc_status kv_pipe_destroy(kvc_pipe* pp) {
  release(pp);
  return KVC_OK;
}

}  // extern "C"

namespace {

// One step; every check that can fail without a HIP error comes before the
// first enqueue, and *enqueued records whether anything reached the stream.
kvc_status step_impl(kvc_pipe* pp, const uint16_t* k_new, const uint16_t* v_new, uint32_t n_new,
                     uint64_t new_stride, const uint16_t* win_K, const uint16_t* win_V,
                     const uint16_t* win_Q, const uint16_t* q, uint16_t* out, float* lse,
                     hipStream_t stream, bool* enqueued) {
  if (stream != pp->dstream || !k_new || !v_new || n_new == 0) return KVC_E_INVALID;
  const kvc_pipe_config& c = pp->cfg;
  const uint32_t period = pp->r.pl.period;
  const uint64_t fill = pp->g % period;
  if (fill + n_new > period) return KVC_E_INVALID;  // a step stays inside one page
  const uint64_t g1 = pp->g + n_new;
  const bool fire = g1 % period == 0 && g1 >= (uint64_t)c.protect + period;
  if (fire && (!win_K || !win_V || !win_Q || pp->fired >= c.max_events)) return KVC_E_INVALID;
  if (out && !q) return KVC_E_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(win_K) || !aligned16(win_V) ||
      !aligned16(win_Q) || !aligned16(q) || !aligned16(out))
    return KVC_E_ALIGN;
  if (new_stride % 8) return KVC_E_ALIGN;
  if (pp->r.streams > 1 && new_stride && new_stride < (uint64_t)n_new * KVC_HEAD_DIM)
    return KVC_E_INVALID;

  const uint64_t page = pp->g / period;
  *enqueued = true;
  // 1. the page about to be written again must have been switched out
  if (fill == 0 && page >= c.pages) {
    const uint64_t old = page - c.pages;
    while (!pp->pending.empty() && pp->pending.front().page <= old) {
      const kvc_status st = switch_front(pp, c.mode == KVC_PIPE_ASYNC);
      if (st != KVC_OK) return st;
    }
  }
  // 2. switches that are due
  if (c.mode == KVC_PIPE_ASYNC) {
    while (!pp->pending.empty()) {
      const hipError_t e = hipEventQuery(pp->done[pp->pending.front().event % c.pages]);
      if (e == hipErrorNotReady) break;
      if (e != hipSuccess) return KVC_E_HIP;
      const kvc_status st = switch_front(pp, false);
      if (st != KVC_OK) return st;
    }
  } else if (c.mode == KVC_PIPE_LAG) {
    while (!pp->pending.empty() && pp->steps >= pp->pending.front().step + c.switch_lag) {
      const kvc_status st = switch_front(pp, false);
      if (st != KVC_OK) return st;
    }
  }
  // 3. append this step's tokens
  kvc_params ap = pp->ev;
  ap.kv_stream_stride = new_stride;
  ap.desc_stream_stride = pp->r.pl.desc_per_stream;
  kvc_status st = kv_append(&ap, k_new, v_new, n_new, (uint32_t)fill, period,
                            c.pages_offset + (page % c.pages) * pp->r.pl.page_bytes, pp->packed,
                            pp->list + page_slot(pp, page), stream);
  if (st != KVC_OK) return st;
  // 4. fire the event of the page `protect` tokens back
  if (fire) {
    const uint64_t e = pp->fired;
    const int ring = (int)(e % c.pages);
    const uint64_t region_page = (g1 - c.protect - period) / period;
    kvc_params ep = pp->ev;
    ep.packed_base_offset = c.events_offset + e * pp->r.pl.event_bytes;
    const bool sync = c.mode == KVC_PIPE_SYNC;
    const hipStream_t cs = sync ? stream : pp->cstream;
    if (!sync) {
      if (hipEventRecord(pp->ready[ring], stream) != hipSuccess ||
          hipStreamWaitEvent(cs, pp->ready[ring], 0) != hipSuccess)
        return KVC_E_HIP;
    }
    st = kv_compress(&ep, win_K, win_V, win_Q, nullptr, pp->packed + ep.packed_base_offset,
                     pp->staged + (uint64_t)ring * pp->r.streams, nullptr, nullptr, nullptr,
                     pp->cws, pp->r.cl.compress_ws_bytes, cs);
    if (st != KVC_OK) return st;
    if (hipEventRecord(pp->done[ring], cs) != hipSuccess) return KVC_E_HIP;
    ++pp->fired;
    pp->pending.push_back({e, pp->steps, region_page});
    if (sync || (c.mode == KVC_PIPE_LAG && c.switch_lag == 0)) {
      st = switch_front(pp, false);
      if (st != KVC_OK) return st;
    }
  }
  // 5. decode over the list
  if (out) {
    st = kv_attend_decode(&pp->dec, q, pp->packed, pp->list, nullptr, out, lse, pp->dws,
                          pp->r.cl.decode_ws_bytes, stream);
    if (st != KVC_OK) return st;
  }
  pp->g = g1;
  ++pp->steps;
  return KVC_OK;
}

}  // namespace

