// kvc_select.hip -- gfx950 kernels of query-aware segment selection at decode
// time (MosaicKV review page: Fig. 6 caption, stage 2 runs during the decode
// stage before each attention layer; Sec. 5.3, PackedAttention performs
// sequence compression in each decode attention layer; Fig. 8, token
// selection rates of 6.25 % and 12.5 %).
//
//   summarize  per descriptor: channel-wise maximum and minimum of its
//              decoded keys (a dropped channel counts as 0, -0 as +0)
//   scores     per descriptor and q head of the group: the bound
//              sum_ch max(q kmax, q kmin) >= q.k of every kept key; a
//              descriptor's score is its largest bound
//   topk       per stream: the k best descriptors (score desc, index asc),
//              written in index order
//
// Scores are pairwise-tree fp32 sums over channels of exact products (bf16 x
// bf16), so the kept set is a deterministic function of the inputs.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// grid (max_desc, streams), 64 threads: lane = channel pair (2 lane, 2 lane + 1).
__global__ __launch_bounds__(64) void k_summarize(SummaryPlan p) {
  const int d = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int nd = p.n_desc ? min((int)p.n_desc[s], p.maxd) : p.maxd;
  uint32_t* out = reinterpret_cast<uint32_t*>(p.summary + ((uint64_t)s * p.maxd + d) * 2 * D);
  const kvc_seg_desc ds = p.desc[(uint64_t)s * p.maxd + d];
  const int T = d < nd ? (int)ds.n_tok : 0;
  if (T == 0) {
    out[lane] = 0u;
    out[64 + lane] = 0u;
    return;
  }
  const int c = ds.n_ch;
  const uint8_t* base = p.packed + ds.offset;
  const bool hm = c < D;
  // a paged descriptor's parts are sized for seg_tokens tokens
  const int TL = (ds.flags & KVC_DESC_PAGED) ? (int)ds.seg_tokens : T;
  const uint8_t* kval = base + (hm ? 16 * TL : 0);
  float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY;
  const int ch = 2 * lane, wd = lane >> 4, bit = ch & 31;
  for (int t = 0; t < T; ++t) {
    uint32_t v0 = 0u, v1 = 0u;
    if (hm) {
      const uint4 m = *reinterpret_cast<const uint4*>(base + 16 * t);
      const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
      uint32_t w = mw[0], below = 0u;
      if (wd >= 1) { below += __popc(mw[0]); w = mw[1]; }
      if (wd >= 2) { below += __popc(mw[1]); w = mw[2]; }
      if (wd >= 3) { below += __popc(mw[2]); w = mw[3]; }
      const uint32_t r0 = below + __popc(w & ((1u << bit) - 1u));
      const bool on0 = (w >> bit) & 1u, on1 = (w >> (bit + 1)) & 1u;
      const uint16_t* row = reinterpret_cast<const uint16_t*>(kval + (size_t)2 * c * t);
      if (on0) v0 = row[r0];
      if (on1) v1 = row[r0 + (on0 ? 1u : 0u)];
    } else {
      const uint32_t w = reinterpret_cast<const uint32_t*>(kval + (size_t)256 * t)[lane];
      v0 = w & 0xFFFFu;
      v1 = w >> 16;
    }
    const float x0 = bf2f(v0) + 0.0f, x1 = bf2f(v1) + 0.0f;  // -0 -> +0
    mx0 = fmaxf(mx0, x0);
    mx1 = fmaxf(mx1, x1);
    mn0 = fminf(mn0, x0);
    mn1 = fminf(mn1, x1);
  }
  // every candidate is a bf16 value, so the top halves are exact
  out[lane] = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xFFFF0000u);
  out[64 + lane] = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xFFFF0000u);
}

// Order-preserving map of an fp32 to uint32 (larger float -> larger key).
// Every finite score maps above float_key(-inf); empty descriptors get key 0.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static_assert(sizeof(kvc_seg_desc) == 16, "descriptors move as one 16-byte word");

constexpr int SCORE_ITERS = 4;  // descriptor groups of 4 per wave and pass

// Scores of NI descriptors dd[i] of stream s, one per 16-lane row (lane cb of
// the row holding channels 8cb .. 8cb+7): max over the group's q heads of
// the pairwise-tree sum over channels of max(q kmax, q kmin) + 0 (8 channels
// in the lane, then the row), -inf for an empty descriptor or one past nd.
// Every load comes first (clamped indices): a store between them, which the
// compiler must assume could alias, would make each wait for it.
template <int NI>
__device__ __forceinline__ void score_rows(const SelectPlan& p, int s, int cb, int nd,
                                           const int (&dd)[NI], float (&out)[NI]) {
  const int b = s / p.hkv, h = s - b * p.hkv;
  const int G = p.G;
  const uint16_t* qg = p.q + (uint64_t)(b * p.hq + h * G) * D + 8 * cb;
  uint32_t ntok[NI];
  uint4 sa[NI], sc[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int di = min(dd[it], p.maxd - 1);
    ntok[it] = p.desc[(uint64_t)s * p.maxd + di].n_tok;
    const uint16_t* sm = p.summary + ((uint64_t)s * p.maxd + di) * 2 * D + 8 * cb;
    sa[it] = *reinterpret_cast<const uint4*>(sm);
    sc[it] = *reinterpret_cast<const uint4*>(sm + D);
  }
  float best[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) best[it] = -INFINITY;
  for (int g = 0; g < G; ++g) {
    const uint4 qv = *reinterpret_cast<const uint4*>(qg + (uint64_t)g * D);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const uint32_t aw[4] = {sa[it].x, sa[it].y, sa[it].z, sa[it].w};
      const uint32_t cw[4] = {sc[it].x, sc[it].y, sc[it].z, sc[it].w};
      float t[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float q0 = bf2f(qw[k] & 0xFFFFu), q1 = bf2f(qw[k] >> 16);
        t[2 * k] = fmaxf(q0 * bf2f(aw[k] & 0xFFFFu), q0 * bf2f(cw[k] & 0xFFFFu)) + 0.0f;
        t[2 * k + 1] = fmaxf(q1 * bf2f(aw[k] >> 16), q1 * bf2f(cw[k] >> 16)) + 0.0f;
      }
      const float v = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
      best[it] = fmaxf(best[it], row16_sum(v));
    }
  }
#pragma unroll
  for (int it = 0; it < NI; ++it)
    out[it] = (dd[it] < nd && ntok[it] > 0) ? best[it] : -INFINITY;
}

// grid (ceil(maxd / (16 * SCORE_ITERS)), streams), 256 threads: four rows
// per wave, SCORE_ITERS descriptors per row.
__global__ __launch_bounds__(256) void k_select_scores(SelectPlan p) {
  const int s = blockIdx.y, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = lane >> 4, cb = lane & 15;
  const int nd = p.n_desc ? min((int)p.n_desc[s], p.maxd) : p.maxd;
  int dd[SCORE_ITERS];
#pragma unroll
  for (int it = 0; it < SCORE_ITERS; ++it)
    dd[it] = ((blockIdx.x * SCORE_ITERS + it) * 4 + wv) * 4 + row;
  float sc[SCORE_ITERS];
  score_rows<SCORE_ITERS>(p, s, cb, nd, dd, sc);
#pragma unroll
  for (int it = 0; it < SCORE_ITERS; ++it)
    if (cb == 0 && dd[it] < p.maxd) p.score[(uint64_t)s * p.maxd + dd[it]] = sc[it];
}

// Sum of a small non-negative integer over the 64 lanes of a full wave
// (exact: every partial sum stays below 2^24), returned wave-uniform.
__device__ __forceinline__ uint32_t wave_count(uint32_t v) {
  return (uint32_t)tree_sum64((float)v);
}

// One wave: the keep best live descriptors of stream s by (score desc,
// index asc), written in index order.  KPL keys per lane in registers
// (descriptor d = 64 i + lane in slot i; maxd <= 64 KPL); counts are ballots
// counted on the scalar unit, ranks are ballots and mbcnt, so there is no
// barrier.  `score` is the stream's row (global memory or LDS).
template <int KPL>
__device__ __forceinline__ void topk_wave(const SelectPlan& p, int s, int lane,
                                          const float* score) {
  const int maxd = p.maxd;
  const kvc_seg_desc* dl = p.desc + (uint64_t)s * maxd;
  // short lists: every descriptor is loaded before any store (a store that
  // might alias would make the loads after it wait), overlapping the search
  constexpr bool PRELOAD = KPL <= 16;
  uint4 dv[PRELOAD ? KPL : 1];
  if constexpr (PRELOAD) {
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      dv[i] = *reinterpret_cast<const uint4*>(dl + min(64 * i + lane, maxd - 1));
  }
  uint32_t key[KPL];
  uint32_t live = 0u;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int d = 64 * i + lane;
    const float f = d < maxd ? score[d] : -INFINITY;
    key[i] = f > -INFINITY ? float_key(f) : 0u;  // 0: empty, below every live key
    live += key[i] != 0u ? 1u : 0u;
  }
  const uint32_t kk = min((uint32_t)p.keep, wave_count(live));
  // kk-th largest key, bit by bit from the top
  uint32_t tau = 0u;
  if (kk > 0) {
    for (int bt = 31; bt >= 0; --bt) {
      const uint32_t cand = tau | (1u << bt);
      // keys at or above cand over the wave: one ballot per slot, counted on
      // the scalar unit (no cross-lane reduction in the chain)
      uint32_t c = 0u;
#pragma unroll
      for (int i = 0; i < KPL; ++i) c += (uint32_t)__popcll(__ballot(key[i] >= cand));
      if (c >= kk) tau = cand;
    }
  }
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < KPL; ++i) c += (kk > 0 && key[i] > tau) ? 1u : 0u;
  const uint32_t need = kk - wave_count(c);
  // compaction in index order: keys above tau, then the first `need` equal to tau
  uint4* od = reinterpret_cast<uint4*>(p.out_desc + (uint64_t)s * p.keep);
  uint32_t eq_before = 0u, out_before = 0u;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (kk > 0 && 64 * i < maxd) {  // wave-uniform
      const uint32_t k = key[i];
      const bool eq = k != 0u && k == tau;
      const uint64_t be = __ballot(eq);
      const bool on = k != 0u && (k > tau || (eq && eq_before + lanes_below(be) < need));
      eq_before += (uint32_t)__popcll(be);
      const uint64_t bo = __ballot(on);
      if (on) {
        uint4 v;
        if constexpr (PRELOAD)
          v = dv[i];
        else
          v = *reinterpret_cast<const uint4*>(dl + 64 * i + lane);
        od[out_before + lanes_below(bo)] = v;
      }
      out_before += (uint32_t)__popcll(bo);
    }
  }
  if (lane == 0) p.out_n[s] = kk;
}

// grid (streams), one wave.
template <int KPL>
__global__ __launch_bounds__(64) void k_select_topk(SelectPlan p) {
  topk_wave<KPL>(p, blockIdx.x, threadIdx.x, p.score + (uint64_t)blockIdx.x * p.maxd);
}

hipError_t launch_summarize(const SummaryPlan& p, hipStream_t st) {
  hipLaunchKernelGGL(k_summarize, dim3(p.maxd, p.streams), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_select(const SelectPlan& p, hipStream_t st) {
  const int per_block = 16 * SCORE_ITERS;
  hipLaunchKernelGGL(k_select_scores, dim3((p.maxd + per_block - 1) / per_block, p.streams),
                     dim3(256), 0, st, p);
  if (p.maxd <= 1024)
    hipLaunchKernelGGL(k_select_topk<16>, dim3(p.streams), dim3(64), 0, st, p);
  else if (p.maxd <= 4096)
    hipLaunchKernelGGL(k_select_topk<64>, dim3(p.streams), dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL(k_select_topk<SEL_MAXD / 64>, dim3(p.streams), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace kvc
