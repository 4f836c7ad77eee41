// kvc_host.cpp -- host side of libkvc: argument validation, byte costs and
// feasible strategies, workspace carve-up, split-K sizing, kernel launches.
// No device memory is allocated and no call synchronises.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace {

using namespace kvc;

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
bool pow2(uint32_t x) { return x && !(x & (x - 1)); }
bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Shape {
  int batch, hq, hkv, G, streams;
};

kvc_status check_shape(const kvc_params* p, Shape* s) {
  if (!p || p->struct_size != sizeof(kvc_params)) return KVC_E_INVALID;
  if (p->head_dim != KVC_HEAD_DIM) return KVC_E_UNSUPPORTED;
  if (p->batch == 0 || p->n_q_heads == 0 || p->n_kv_heads == 0) return KVC_E_INVALID;
  if (p->n_q_heads % p->n_kv_heads) return KVC_E_INVALID;
  const uint32_t G = p->n_q_heads / p->n_kv_heads;
  if (G > 16) return KVC_E_UNSUPPORTED;
  if ((uint64_t)p->batch * p->n_q_heads > (1u << 24)) return KVC_E_UNSUPPORTED;
  if ((uint64_t)p->batch * p->n_kv_heads > 65535u) return KVC_E_UNSUPPORTED;  // grid.y
  s->batch = (int)p->batch;
  s->hq = (int)p->n_q_heads;
  s->hkv = (int)p->n_kv_heads;
  s->G = (int)G;
  s->streams = (int)(p->batch * p->n_kv_heads);
  return KVC_OK;
}

float eff_scale(const kvc_params* p) {
  return p->scale != 0.0f ? p->scale : (float)(1.0 / std::sqrt((double)p->head_dim));
}

// Fills the compression part of the layout.  Returns KVC_E_BUDGET when no
// strategy fits (layout still filled).
kvc_status compress_layout(const kvc_params* p, const Shape& sh, kvc_layout* L, int* nc_out,
                           int* cvals, int* su) {
  if (p->n_strategies == 0 || p->n_strategies > KVC_MAX_STRATEGIES || !p->strategies)
    return KVC_E_INVALID;
  if (p->budget_scope > KVC_BUDGET_STREAM) return KVC_E_INVALID;
  if (p->rotate > 1 || p->store_logits > 1) return KVC_E_INVALID;
  const bool stream_scope = p->budget_scope == KVC_BUDGET_STREAM;
  const uint32_t S = p->seg_tokens;
  if (!pow2(S) || S < 16 || S > 256) return KVC_E_INVALID;
  if (p->rot_span && (!p->rotate || p->rot_span % 64 || p->rot_span % S ||
                      p->region_len % p->rot_span))
    return KVC_E_INVALID;
  if (p->n_ctx == 0 || p->n_ctx % BLK || p->n_ctx > (1u << 22)) return KVC_E_INVALID;
  if (p->region_len == 0 || p->region_len % S) return KVC_E_INVALID;
  if ((uint64_t)p->region_begin + p->region_len > p->n_ctx) return KVC_E_INVALID;
  int nc = 0;
  bool t2c_used = false;
  uint32_t feas = 0, nfeas = 0;
  uint64_t maxb = 0;
  bool partial = false;
  for (uint32_t i = 0; i < p->n_strategies; ++i) {
    const kvc_strategy& st = p->strategies[i];
    if (st.n_tok > S) return KVC_E_INVALID;
    if (st.n_tok > 0) {
      if (st.n_ch < 8 || st.n_ch > KVC_HEAD_DIM || st.n_ch % 8) return KVC_E_INVALID;
      if (st.n_tok < S) {
        t2c_used = true;
        if (p->t2c_alpha > 0 && p->t2c_alpha >= st.n_tok) return KVC_E_INVALID;
      }
    }
    su[i] = 0;
    if (st.n_tok > 0 && st.n_ch < KVC_HEAD_DIM) {
      int u = 0;
      while (u < nc && cvals[u] != st.n_ch) ++u;
      if (u == nc) {
        if (nc == MAX_NC) return KVC_E_UNSUPPORTED;
        cvals[nc++] = st.n_ch;
      }
      su[i] = u;
    }
    const uint32_t by = seg_bytes(st.n_tok, st.n_tok ? st.n_ch : 0, S);
    L->seg_bytes[i] = by;
    const uint64_t cap = stream_scope ? (uint64_t)p->budget_bytes * (p->region_len / S)
                                      : (uint64_t)p->budget_bytes;
    if (by <= cap) {
      feas |= 1u << i;
      ++nfeas;
      if (by > maxb) maxb = by;
      if (st.n_tok > 0 && st.n_tok < S) partial = true;
    }
  }
  if (p->t2c_alpha > 0 && t2c_used && p->t2c_gamma < 2) return KVC_E_INVALID;
  *nc_out = nc;
  const uint64_t n_seg = p->region_len / S;
  L->feasible_mask = feas;
  L->n_seg = (uint32_t)n_seg;
  L->max_seg_bytes = maxb;
  uint64_t stream_max = n_seg * maxb;
  if (stream_scope) {
    // the smallest strategy must fit every segment; the stream never writes
    // more than n_seg * budget_bytes
    uint32_t mn = 0xFFFFFFFFu;
    for (uint32_t i = 0; i < p->n_strategies; ++i) mn = L->seg_bytes[i] < mn ? L->seg_bytes[i] : mn;
    if (mn > p->budget_bytes) nfeas = 0;
    if (n_seg * p->budget_bytes < stream_max) stream_max = n_seg * p->budget_bytes;
  }
  L->stream_capacity = align_up(stream_max, kAlign);
  L->packed_bytes_max = (uint64_t)sh.streams * L->stream_capacity;
  L->n_desc = (uint64_t)sh.streams * n_seg;
  L->needs_scoring = (partial || nfeas > 1) ? 1u : 0u;
  if (L->needs_scoring && p->n_win == 0) return KVC_E_INVALID;
  // workspace: partials, normalisers, scores, masks, energy shares, keep bits
  const uint64_t nq = (uint64_t)sh.G * (p->n_win ? p->n_win : 1);
  const uint64_t nblk = p->n_ctx / BLK;
  uint64_t ws = 0;
  ws += 2 * align_up((uint64_t)sh.streams * nq * nblk * 4, kAlign);
  ws += 2 * align_up((uint64_t)sh.streams * nq * 4, kAlign);
  ws += align_up((uint64_t)sh.streams * p->region_len * 4, kAlign);
  ws += align_up((uint64_t)sh.streams * p->region_len * (uint64_t)nc * 2 * 16, kAlign);
  ws += align_up((uint64_t)sh.streams * p->region_len * (uint64_t)nc * 2 * 4, kAlign);
  ws += align_up((uint64_t)sh.streams * n_seg * ((S + 31) / 32) * 4, kAlign);
  // window queries converted to fp32 once per call
  if (p->n_win) ws += align_up((uint64_t)sh.streams * nq * KVC_HEAD_DIM * 4, kAlign);
  // store_logits: every window-query logit of the domain
  if (p->n_win && p->store_logits) ws += align_up((uint64_t)sh.streams * nq * p->n_ctx * 4, kAlign);
  // stream scope: keep sets and objectives of every strategy
  if (stream_scope) {
    ws += align_up((uint64_t)sh.streams * n_seg * p->n_strategies * ((S + 31) / 32) * 4, kAlign);
    ws += align_up((uint64_t)sh.streams * n_seg * p->n_strategies * 4, kAlign);
  }
  // rotation: the Gram matrix of every span and side, the rotated region vectors
  if (p->rotate) {
    const uint64_t n_span = p->rot_span ? p->region_len / p->rot_span : 1;
    ws += align_up((uint64_t)sh.streams * n_span * 2 * KVC_HEAD_DIM * KVC_HEAD_DIM * 4, kAlign);
    ws += 2 * align_up((uint64_t)sh.streams * p->region_len * KVC_HEAD_DIM * 2, kAlign);
  }
  L->compress_ws_bytes = ws;
  return nfeas ? KVC_OK : KVC_E_BUDGET;
}

// Rotation spans of a decode list: descriptor i is in span i / span_desc
// (one span holding every descriptor when the cache has no rotation spans).
struct DecodeSpans {
  uint32_t n_span, span_desc;
};
DecodeSpans decode_spans(const kvc_params* p, uint32_t maxd) {
  DecodeSpans d{1u, maxd};
  if (p->rotate && p->rot_span && p->seg_tokens && p->rot_span % p->seg_tokens == 0) {
    d.span_desc = p->rot_span / p->seg_tokens;
    d.n_span = (maxd + d.span_desc - 1) / d.span_desc;
  }
  return d;
}

constexpr uint32_t kMaxSplits = 65536;  // split-K factor per stream (a caller's value included)

// 0 when the caller's split count cannot be used.
uint32_t choose_splits(const kvc_params* p, const Shape& sh, uint32_t maxd) {
  const DecodeSpans sp = decode_spans(p, maxd);
  if (p->decode_splits) {
    if (p->decode_splits > kMaxSplits || p->decode_splits % sp.n_span) return 0;
    return p->decode_splits;
  }
  // one wave per (stream, split); a CU holds 12 decode waves for groups of up
  // to 4 q heads and 8 for larger groups (LDS and registers): fill 256 CUs
  // once, with at least one descriptor per split
  const uint32_t waves = sh.G <= 4 ? 3072u : 2048u;
  uint32_t want = (waves + (uint32_t)sh.streams - 1) / (uint32_t)sh.streams;
  if (want > maxd) want = maxd;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  // with rotation spans, every split stays inside one span: per splits per
  // span, chosen (up to 8, at most a span's descriptors) so that the waves
  // fill whole rounds of the CU slots (rounds per unit of work,
  // ceil(items * per / waves) / per, is smallest)
  if (sp.n_span > 1) {
    const uint64_t items = (uint64_t)sh.streams * sp.n_span;
    uint32_t per = 1;
    double best = 1e30;
    for (uint32_t c = 1; c <= 8 && c <= sp.span_desc; ++c) {
      const double rounds = (double)((items * c + waves - 1) / waves) / (double)c;
      if (rounds < best - 1e-9) {
        best = rounds;
        per = c;
      }
    }
    want = sp.n_span * per;
  }
  return want;
}

// false when the split count is unusable (caller's value out of range, or
// more (stream, split) items than an int holds).
bool decode_layout(const kvc_params* p, const Shape& sh, uint32_t maxd, kvc_layout* L) {
  const uint32_t splits = choose_splits(p, sh, maxd ? maxd : 1);
  if (splits == 0 || (uint64_t)sh.streams * splits > 0x7FFFFFFFull) return false;
  L->decode_splits = splits;
  const uint64_t rows = (uint64_t)sh.batch * sh.hq * splits;
  L->decode_ws_bytes = align_up(rows * 2 * 4, kAlign) + align_up(rows * KVC_HEAD_DIM * 4, kAlign);
  // rotated cache: the rotated queries' two bf16 parts and each span's
  // rotated-back share of the output (fp32), per row and span
  if (p->rotate) {
    const uint64_t n_span = decode_spans(p, maxd ? maxd : 1).n_span;
    const uint64_t per = (uint64_t)sh.batch * sh.hq * n_span * KVC_HEAD_DIM;
    L->decode_ws_bytes += 2 * align_up(per * 2, kAlign) + align_up(per * 4, kAlign);
  }
  return true;
}

uint32_t decode_maxd(const kvc_params* p) {
  if (p->max_desc_per_stream) return p->max_desc_per_stream;
  if (p->seg_tokens && p->region_len) return p->region_len / p->seg_tokens;
  return 0;
}

}  // namespace

extern "C" {

int kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_E_INVALID: return "invalid argument";
    case KVC_E_UNSUPPORTED: return "unsupported configuration";
    case KVC_E_BUDGET: return "no strategy fits the byte budget";
    case KVC_E_WORKSPACE: return "workspace too small";
    case KVC_E_ALIGN: return "pointer not 16-byte aligned";
    case KVC_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

kvc_status kv_layout_query(const kvc_params* p, kvc_layout* out) {
  if (!out) return KVC_E_INVALID;
  std::memset(out, 0, sizeof(*out));
  Shape sh;
  kvc_status st = check_shape(p, &sh);
  if (st != KVC_OK) return st;
  kvc_status cs = KVC_OK;
  if (p->n_strategies > 0) {
    int nc, cvals[MAX_NC], su[KVC_MAX_STRATEGIES];
    cs = compress_layout(p, sh, out, &nc, cvals, su);
    if (cs != KVC_OK && cs != KVC_E_BUDGET) return cs;
  }
  const uint32_t maxd = decode_maxd(p);
  if (maxd) {
    if (!decode_layout(p, sh, maxd, out)) return KVC_E_INVALID;
  } else if (p->n_strategies == 0) {
    return KVC_E_INVALID;
  }
  return cs;
}

}  // extern "C"

namespace {

kvc_status compress_impl(const kvc_params* p, const uint16_t* K, const uint16_t* V,
                         const uint16_t* Qwin, const uint8_t* forced_strategy, void* packed,
                         kvc_seg_desc* desc, uint64_t* used_bytes, float* scores,
                         float* objective, float* rot, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  Shape sh;
  kvc_status st = check_shape(p, &sh);
  if (st != KVC_OK) return st;
  if ((p->rotate != 0) != (rot != nullptr)) return KVC_E_INVALID;
  if (!aligned16(rot)) return KVC_E_ALIGN;
  kvc_layout L;
  std::memset(&L, 0, sizeof L);
  CompressPlan c;
  std::memset(&c, 0, sizeof c);
  st = compress_layout(p, sh, &L, &c.nc, c.cvals, c.su);
  if (st != KVC_OK) return st;
  const bool scoring = L.needs_scoring || scores || objective;
  if (!K || !V || !packed || !desc || (scoring && (!Qwin || !p->n_win))) return KVC_E_INVALID;
  if (!aligned16(K) || !aligned16(V) || !aligned16(Qwin) || !aligned16(packed) ||
      !aligned16(desc) || !aligned16(ws))
    return KVC_E_ALIGN;
  if (p->packed_base_offset % 16 || (p->packed_stream_stride && p->packed_stream_stride % 16))
    return KVC_E_ALIGN;
  if (p->kv_stream_stride % 8 || p->qw_head_stride % 8) return KVC_E_ALIGN;
  if (ws_bytes < L.compress_ws_bytes || (L.compress_ws_bytes && !ws)) return KVC_E_WORKSPACE;
  const bool stream_scope = p->budget_scope == KVC_BUDGET_STREAM;
  if (stream_scope && forced_strategy) return KVC_E_INVALID;
  const uint64_t pstride = p->packed_stream_stride ? p->packed_stream_stride : L.stream_capacity;
  const uint64_t stream_max =
      stream_scope ? (uint64_t)L.n_seg * p->budget_bytes : L.n_seg * L.max_seg_bytes;
  if (pstride < stream_max) return KVC_E_INVALID;
  const uint32_t dstride = p->desc_stream_stride ? p->desc_stream_stride : L.n_seg;
  if (dstride < L.n_seg) return KVC_E_INVALID;

  c.batch = sh.batch;
  c.hq = sh.hq;
  c.hkv = sh.hkv;
  c.G = sh.G;
  c.streams = sh.streams;
  c.n_ctx = (int)p->n_ctx;
  c.region_begin = (int)p->region_begin;
  c.region_len = (int)p->region_len;
  c.S = (int)p->seg_tokens;
  c.W = (int)(p->n_win ? p->n_win : 1);
  c.nq = c.G * c.W;
  c.nblk = (int)(p->n_ctx / BLK);
  c.n_seg = (int)L.n_seg;
  c.scale = eff_scale(p);
  c.kv_stride = p->kv_stream_stride ? p->kv_stream_stride : (uint64_t)p->n_ctx * KVC_HEAD_DIM;
  c.qw_stride = p->qw_head_stride ? p->qw_head_stride : (uint64_t)c.W * KVC_HEAD_DIM;
  c.pstride = pstride;
  c.pbase = p->packed_base_offset;
  c.dstride = dstride;
  c.n_strat = (int)p->n_strategies;
  for (uint32_t i = 0; i < p->n_strategies; ++i) {
    c.sT[i] = p->strategies[i].n_tok;
    c.sc[i] = p->strategies[i].n_tok ? p->strategies[i].n_ch : 0;
  }
  c.feasible_mask = L.feasible_mask;
  c.t2c_alpha = (int)p->t2c_alpha;
  c.t2c_gamma = (int)p->t2c_gamma;
  c.scoring = scoring;
  c.max_waves = p->compress_max_waves;
  c.K = K;
  c.V = V;
  c.Qw = Qwin;
  c.forced = forced_strategy;
  c.packed = static_cast<uint8_t*>(packed);
  c.desc = desc;
  c.used = used_bytes;
  c.scores_out = scores;
  c.objective = objective;
  // workspace carve-up (same order and sizes as compress_layout)
  uint8_t* w = static_cast<uint8_t*>(ws);
  auto take = [&](uint64_t bytes) {
    uint8_t* r = w;
    w += align_up(bytes, kAlign);
    return r;
  };
  const uint64_t S64 = (uint64_t)c.streams;
  c.part_m = reinterpret_cast<float*>(take(S64 * c.nq * c.nblk * 4));
  c.part_z = reinterpret_cast<float*>(take(S64 * c.nq * c.nblk * 4));
  c.norm_m = reinterpret_cast<float*>(take(S64 * c.nq * 4));
  c.norm_iz = reinterpret_cast<float*>(take(S64 * c.nq * 4));
  c.scores = reinterpret_cast<float*>(take(S64 * c.region_len * 4));
  c.masks = reinterpret_cast<uint32_t*>(take(S64 * c.region_len * (uint64_t)c.nc * 2 * 16));
  c.rho = reinterpret_cast<float*>(take(S64 * c.region_len * (uint64_t)c.nc * 2 * 4));
  c.keep = reinterpret_cast<uint32_t*>(take(S64 * c.n_seg * ((c.S + 31) / 32) * 4));
  c.qf = p->n_win ? reinterpret_cast<float*>(take(S64 * c.nq * D * 4)) : nullptr;
  c.logits = p->n_win && p->store_logits
                 ? reinterpret_cast<float*>(take(S64 * c.nq * (uint64_t)p->n_ctx * 4))
                 : nullptr;
  c.stream_budget = stream_scope;
  c.stream_bytes = (uint64_t)L.n_seg * p->budget_bytes;
  for (int i = 0; i < KVC_MAX_STRATEGIES; ++i) c.seg_bytes[i] = L.seg_bytes[i];
  c.keep_all = nullptr;
  c.J_all = nullptr;
  if (stream_scope) {
    c.keep_all = reinterpret_cast<uint32_t*>(
        take(S64 * c.n_seg * (uint64_t)c.n_strat * ((c.S + 31) / 32) * 4));
    c.J_all = reinterpret_cast<float*>(take(S64 * c.n_seg * (uint64_t)c.n_strat * 4));
  }
  c.rotate = p->rotate != 0;
  c.rot = rot;
  c.gram = nullptr;
  c.YK = c.YV = nullptr;
  if (c.rotate) {
    c.span_len = p->rot_span ? (int)p->rot_span : c.region_len;
    c.n_span = c.region_len / c.span_len;
    c.gram = reinterpret_cast<float*>(take(S64 * (uint64_t)c.n_span * 2 * D * D * 4));
    c.YK = reinterpret_cast<uint16_t*>(take(S64 * c.region_len * D * 2));
    c.YV = reinterpret_cast<uint16_t*>(take(S64 * c.region_len * D * 2));
  }
  if (launch_compress(c, stream) != hipSuccess) return KVC_E_HIP;
  return KVC_OK;
}

kvc_status decode_impl(const kvc_params* p, const uint16_t* q, const void* packed,
                       const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                       const float* rot, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t stream);

}  // namespace

extern "C" {

kvc_status kv_compress(const kvc_params* p, const uint16_t* K, const uint16_t* V,
                       const uint16_t* Qwin, const uint8_t* forced_strategy, void* packed,
                       kvc_seg_desc* desc, uint64_t* used_bytes, float* scores, float* objective,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  if (p && p->struct_size == sizeof(kvc_params) && p->rotate) return KVC_E_INVALID;
  return compress_impl(p, K, V, Qwin, forced_strategy, packed, desc, used_bytes, scores,
                       objective, nullptr, ws, ws_bytes, stream);
}

kvc_status kv_compress_rotated(const kvc_params* p, const uint16_t* K, const uint16_t* V,
                               const uint16_t* Qwin, const uint8_t* forced_strategy, void* packed,
                               kvc_seg_desc* desc, uint64_t* used_bytes, float* scores,
                               float* objective, float* rot, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!p || p->struct_size != sizeof(kvc_params) || p->rotate != 1 || !rot) return KVC_E_INVALID;
  return compress_impl(p, K, V, Qwin, forced_strategy, packed, desc, used_bytes, scores,
                       objective, rot, ws, ws_bytes, stream);
}

kvc_status kv_attend_decode(const kvc_params* p, const uint16_t* q, const void* packed,
                            const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                            uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (p && p->struct_size == sizeof(kvc_params) && p->rotate) return KVC_E_INVALID;
  return decode_impl(p, q, packed, desc, n_desc_per_stream, nullptr, out, lse, ws, ws_bytes,
                     stream);
}

kvc_status kv_attend_decode_noalloc(const kvc_params* p, const uint16_t* q, const void* packed,
                                    const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                                    uint16_t* out, float* lse, hipStream_t stream) {
  if (p && p->struct_size == sizeof(kvc_params) && p->rotate) return KVC_E_INVALID;
  Shape sh;
  kvc_status st = check_shape(p, &sh);
  if (st != KVC_OK) return st;
  const uint32_t maxd = decode_maxd(p);
  if (maxd == 0) return KVC_E_INVALID;
  kvc_layout L;
  std::memset(&L, 0, sizeof L);
  if (!decode_layout(p, sh, maxd, &L)) return KVC_E_INVALID;
  if (L.decode_ws_bytes > KVC_NOALLOC_SCRATCH_BYTES) return KVC_E_WORKSPACE;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess || !ws) return KVC_E_HIP;
  return decode_impl(p, q, packed, desc, n_desc_per_stream, nullptr, out, lse, ws,
                     KVC_NOALLOC_SCRATCH_BYTES, stream);
}

kvc_status kv_attend_decode_rotated(const kvc_params* p, const uint16_t* q, const void* packed,
                                    const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                                    const float* rot, uint16_t* out, float* lse, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (!p || p->struct_size != sizeof(kvc_params) || p->rotate != 1 || !rot) return KVC_E_INVALID;
  return decode_impl(p, q, packed, desc, n_desc_per_stream, rot, out, lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

kvc_status decode_impl(const kvc_params* p, const uint16_t* q, const void* packed,
                       const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                       const float* rot, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  Shape sh;
  kvc_status st = check_shape(p, &sh);
  if (st != KVC_OK) return st;
  if (!aligned16(rot)) return KVC_E_ALIGN;
  const uint32_t maxd = decode_maxd(p);
  if (maxd == 0 || !q || !out || !desc || !packed) return KVC_E_INVALID;
  if (!aligned16(q) || !aligned16(packed) || !aligned16(desc) || !aligned16(out) || !aligned16(ws))
    return KVC_E_ALIGN;
  if (p->rot_span && (!p->rotate || !p->seg_tokens || p->rot_span % p->seg_tokens))
    return KVC_E_INVALID;
  kvc_layout L;
  std::memset(&L, 0, sizeof L);
  if (!decode_layout(p, sh, maxd, &L)) return KVC_E_INVALID;
  if (ws_bytes < L.decode_ws_bytes || !ws) return KVC_E_WORKSPACE;
  DecodePlan d;
  d.batch = sh.batch;
  d.hq = sh.hq;
  d.hkv = sh.hkv;
  d.G = sh.G;
  d.streams = sh.streams;
  d.maxd = (int)maxd;
  d.splits = (int)L.decode_splits;
  d.scale = eff_scale(p);
  d.q = q;
  d.packed = static_cast<const uint8_t*>(packed);
  d.desc = desc;
  d.n_desc = n_desc_per_stream;
  d.out = out;
  d.lse = lse;
  const uint64_t rows = (uint64_t)sh.batch * sh.hq * d.splits;
  uint8_t* w = static_cast<uint8_t*>(ws);
  d.part_ml = reinterpret_cast<float*>(w);
  w += align_up(rows * 2 * 4, kAlign);
  d.part_acc = reinterpret_cast<float*>(w);
  w += align_up(rows * KVC_HEAD_DIM * 4, kAlign);
  d.rot = rot;
  d.qhi = d.qlo = nullptr;
  d.span_out = nullptr;
  d.n_span = 1;
  d.span_desc = 0;
  d.spl = d.splits;
  if (rot) {
    const DecodeSpans sp = decode_spans(p, maxd);
    d.n_span = (int)sp.n_span;
    if (sp.n_span > 1) {
      d.span_desc = (int)sp.span_desc;
      d.spl = d.splits / d.n_span;
    }
    const uint64_t per = (uint64_t)sh.batch * sh.hq * sp.n_span * KVC_HEAD_DIM;
    const uint64_t qb = align_up(per * 2, kAlign);
    d.qhi = reinterpret_cast<uint16_t*>(w);
    d.qlo = reinterpret_cast<uint16_t*>(w + qb);
    d.span_out = reinterpret_cast<float*>(w + 2 * qb);
  }
  if (launch_decode(d, stream) != hipSuccess) return KVC_E_HIP;
  return KVC_OK;
}

}  // namespace

extern "C" {

kvc_status kv_summarize(const kvc_params* p, const void* packed, const kvc_seg_desc* desc,
                        const uint32_t* n_desc_per_stream, uint16_t* summary, hipStream_t stream) {
  Shape sh;
  kvc_status st = check_shape(p, &sh);
  if (st != KVC_OK) return st;
  const uint32_t maxd = decode_maxd(p);
  if (maxd == 0 || maxd > 65535u || !packed || !desc || !summary) return KVC_E_INVALID;
  if (!aligned16(packed) || !aligned16(desc) || !aligned16(summary)) return KVC_E_ALIGN;
  SummaryPlan sp;
  sp.streams = sh.streams;
  sp.maxd = (int)maxd;
  sp.packed = static_cast<const uint8_t*>(packed);
  sp.desc = desc;
  sp.n_desc = n_desc_per_stream;
  sp.summary = summary;
  if (launch_summarize(sp, stream) != hipSuccess) return KVC_E_HIP;
  return KVC_OK;
}

kvc_status kv_read_stream(const void* src, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0) return KVC_E_INVALID;
  if (!aligned16(src) || !aligned16(sink)) return KVC_E_ALIGN;
  if (launch_read_stream(src, bytes, sink, stream) != hipSuccess) return KVC_E_HIP;
  return KVC_OK;
}

kvc_status kv_select_segments(const kvc_params* p, const uint16_t* q, const uint16_t* summary,
                              const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                              uint32_t keep, kvc_seg_desc* out_desc, uint32_t* out_n, float* score,
                              hipStream_t stream) {
  Shape sh;
  kvc_status st = check_shape(p, &sh);
  if (st != KVC_OK) return st;
  const uint32_t maxd = decode_maxd(p);
  if (maxd == 0 || keep == 0 || !q || !summary || !desc || !out_desc || !out_n || !score)
    return KVC_E_INVALID;
  if (maxd > (uint32_t)SEL_MAXD) return KVC_E_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(summary) || !aligned16(desc) || !aligned16(out_desc) ||
      !aligned16(score))
    return KVC_E_ALIGN;
  SelectPlan sp;
  sp.streams = sh.streams;
  sp.hkv = sh.hkv;
  sp.hq = sh.hq;
  sp.G = sh.G;
  sp.maxd = (int)maxd;
  sp.keep = (int)(keep < maxd ? keep : maxd);
  sp.q = q;
  sp.summary = summary;
  sp.desc = desc;
  sp.n_desc = n_desc_per_stream;
  sp.out_desc = out_desc;
  sp.out_n = out_n;
  sp.score = score;
  if (launch_select(sp, stream) != hipSuccess) return KVC_E_HIP;
  return KVC_OK;
}

}  // extern "C"
