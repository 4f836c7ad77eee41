// kvc_compress.hip -- gfx950 kernels of segment-wise two-dimensional KV-cache
// compression (MosaicKV review page: abstract, Fig. 5 and Fig. 6 captions;
// KARA review page: "What carries the argument", Fig. 3 caption).
//
// Pipeline per call (every kernel on the caller's stream):
//   score_partials  per 64-token block of the domain and per window query:
//                   the logits (stored for the later passes when asked) and
//                   their block maximum m_b
//   score_max       per window query: global max m = max of the m_b
//   score_expsum    per block and window query: pairwise sum z_b of
//                   exp(l - m) over the block's 64 tokens
//   score_normalise per window query: Z = pairwise sum of the z_b over the
//                   blocks (zero-padded to a power of two), i.e. the
//                   pairwise sum of exp(l - m) over the whole domain; 1/Z
//   token_scores    per region token: sum over the group's window queries of
//                   exp(l - m) / Z, accumulated one query at a time
//   channel_select  per region K and V vector and per channel count c < 128:
//                   top-c magnitude mask and kept energy share
//   segment_choose  per segment: top-T (or Token2Chunk) per strategy,
//                   objective, choice under the byte budget, descriptor
//   offsets_scan    per stream: exclusive scan of segment bytes
//   pack            per segment: masks, values, index list
//
// Selection outputs are bit-exact functions of the inputs: every float that
// feeds a comparison is produced by correctly rounded fp32 operations in a
// fixed order (fma chains over ascending channels, pairwise trees with
// adjacent pairs first, sequential sums over queries), built with
// -ffp-contract=off and without packed fp32 math.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// ---------------------------------------------------------------------------
// Window scoring.
// ---------------------------------------------------------------------------

// Loads one key row (128 bf16) of this lane into fp32 registers.
__device__ __forceinline__ void load_row_f32(const uint16_t* __restrict__ row, float* kf) {
  const uint4* r4 = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 v = r4[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      kf[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
      kf[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}

// Shapes and inputs of the scoring kernels; outputs and workspace arrays are
// separate restrict-qualified arguments (so uniform loads become scalar).
struct ScoreArgs {
  const uint16_t* K;
  const uint16_t* Qw;
  uint64_t kv_stride, qw_stride;
  int hkv, hq, G, W, nq, nblk, n_ctx, region_begin, region_len;
  int qper;  // window queries per wave of score_partials (at most 64, a multiple of 4)
  float scale;
};

// Work units of a logical grid (gx, gy, gz), walked by a 1-D launch that
// may be capped below the unit count: workgroup b takes units b, b +
// gridDim.x, ...; unit u is (u % gx, u / gx % gy, u / (gx gy)).  Every unit
// is computed by exactly one workgroup whatever the cap, so results do not
// depend on it.
struct Units {
  uint32_t gx, gy, total;
};
__device__ __forceinline__ void unit_xyz(const Units& g, uint32_t u, int& x, int& y, int& z) {
  x = (int)(u % g.gx);
  const uint32_t r = u / g.gx;
  y = (int)(r % g.gy);
  z = (int)(r / g.gy);
}

// Window queries to fp32, [stream][g * W + w][128], so that the scoring
// kernels read them with scalar loads and no per-use conversion.
// grid (G * W, streams), 64 threads: lane = channel pair.
__global__ __launch_bounds__(64) void k_q_convert(ScoreArgs a, Units un, float* __restrict__ qf) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int qi, s, z_;
    unit_xyz(un, u, qi, s, z_);
    const int b = s / a.hkv, h = s - b * a.hkv;
    const int g = qi / a.W, w = qi - g * a.W;
    const uint16_t* src = a.Qw + (uint64_t)(b * a.hq + h * a.G + g) * a.qw_stride + (uint64_t)w * D;
    const uint32_t v = reinterpret_cast<const uint32_t*>(src)[lane];
    float2 o;
    o.x = __uint_as_float(v << 16);
    o.y = __uint_as_float(v & 0xFFFF0000u);
    reinterpret_cast<float2*>(qf + ((uint64_t)s * a.nq + qi) * D)[lane] = o;
  }
}

constexpr int QB = 8;  // window queries scored together (independent fma chains)

// Logits of NQ consecutive window queries (rows qr, qr + 128, ...) against
// this lane's key: one fma chain per query over ascending channels, times
// scale.
template <int NQ>
__device__ __forceinline__ void logits(const float* __restrict__ qr, const float* kf, float scale,
                                       float* l) {
  float acc[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int ch = 0; ch < D; ++ch)
#pragma unroll
    for (int j = 0; j < NQ; ++j) acc[j] = __builtin_fmaf(qr[j * D + ch], kf[ch], acc[j]);
#pragma unroll
  for (int j = 0; j < NQ; ++j) l[j] = acc[j] * scale;
}

// Logits and block maximum of NQ window queries q0.. over the 64 tokens of a
// block (lane = token).  With `lg`, the logits are also stored,
// [stream][query][domain token], for the later passes.
template <int NQ>
__device__ __forceinline__ void block_max(const float* __restrict__ qs, int q0, const float* kf,
                                          const ScoreArgs& a, int s, int blk, int lane,
                                          float* __restrict__ part_m, float* __restrict__ lg) {
  float l[NQ], mb[NQ];
  logits<NQ>(qs + (uint64_t)q0 * D, kf, a.scale, l);
  if (lg) {
    const uint32_t t = (uint32_t)(blk * BLK + lane);
#pragma unroll
    for (int j = 0; j < NQ; ++j) (lg + ((uint64_t)s * a.nq + q0 + j) * a.n_ctx)[t] = l[j];
  }
#pragma unroll
  for (int j = 0; j < NQ; ++j) mb[j] = l[j];
  max64_n_last<NQ>(mb);
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) part_m[((uint64_t)s * a.nq + q0 + j) * a.nblk + blk] = mb[j];
  }
}

// grid (nblk, streams, ceil(nq / qper)), 64 threads: lane = token of the
// 64-token block; wave z handles window queries z * qper .. (z + 1) * qper - 1
// (each (query, block) result is computed by exactly one wave, so the split
// changes no result; it fills the chip when a domain has few blocks and keeps
// the window queries read at one time within the scalar cache).
__global__ __launch_bounds__(64) void k_score_partials(ScoreArgs a, Units un,
                                                       const float* __restrict__ qf,
                                                       float* __restrict__ part_m,
                                                       float* __restrict__ lg) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int blk, s, zq;
    unit_xyz(un, u, blk, s, zq);
    const int t = blk * BLK + lane;
    float kf[D];
    load_row_f32(a.K + (uint64_t)s * a.kv_stride + (uint64_t)t * D, kf);
    const float* qs = qf + (uint64_t)s * a.nq * D;
    int q0 = zq * a.qper;
    const int q1 = min(a.nq, q0 + a.qper);
    for (; q0 + QB <= q1; q0 += QB) block_max<QB>(qs, q0, kf, a, s, blk, lane, part_m, lg);
    for (; q0 < q1; ++q0) block_max<1>(qs, q0, kf, a, s, blk, lane, part_m, lg);
  }
}

// grid (nq, streams), 64 threads: m = max of the block maxima of a query.
__global__ __launch_bounds__(64) void k_score_max(ScoreArgs a, Units un,
                                                  const float* __restrict__ part_m,
                                                  float* __restrict__ norm_m) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int qi, s, z_;
    unit_xyz(un, u, qi, s, z_);
    const float* pm = part_m + ((uint64_t)s * a.nq + qi) * a.nblk;
    float mx = -INFINITY;
    for (int b = lane; b < a.nblk; b += 64) mx = fmax_nn(mx, pm[b]);
    const float m = max64(mx);
    if (lane == 0) norm_m[(uint64_t)s * a.nq + qi] = m;
  }
}

// z_b of NQ queries q0.. from their logits l (lane = token): pairwise sum of
// exp(l - m) over the block, stored by lane 63.
template <int NQ>
__device__ __forceinline__ void block_expsum(const float* l, int q0, const ScoreArgs& a, int s,
                                             int blk, int lane, const float* __restrict__ nm,
                                             float* __restrict__ part_z) {
  float z[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) z[j] = spec_exp2((l[j] - nm[q0 + j]) * KVC_LOG2E);
  tree_sum64_n_last<NQ>(z);
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) part_z[((uint64_t)s * a.nq + q0 + j) * a.nblk + blk] = z[j];
  }
}

// grid as k_score_partials: the block sums z_b with the global maximum,
// logits recomputed (same fma chains, so the same values).
__global__ __launch_bounds__(64) void k_score_expsum(ScoreArgs a, Units un,
                                                     const float* __restrict__ qf,
                                                     const float* __restrict__ norm_m,
                                                     float* __restrict__ part_z) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int blk, s, zq;
    unit_xyz(un, u, blk, s, zq);
    const int t = blk * BLK + lane;
    float kf[D];
    load_row_f32(a.K + (uint64_t)s * a.kv_stride + (uint64_t)t * D, kf);
    const float* qs = qf + (uint64_t)s * a.nq * D;
    const float* nm = norm_m + (uint64_t)s * a.nq;
    int q0 = zq * a.qper;
    const int q1 = min(a.nq, q0 + a.qper);
    for (; q0 + QB <= q1; q0 += QB) {
      float l[QB];
      logits<QB>(qs + (uint64_t)q0 * D, kf, a.scale, l);
      block_expsum<QB>(l, q0, a, s, blk, lane, nm, part_z);
    }
    for (; q0 < q1; ++q0) {
      float l;
      logits<1>(qs + (uint64_t)q0 * D, kf, a.scale, &l);
      block_expsum<1>(&l, q0, a, s, blk, lane, nm, part_z);
    }
  }
}

// The same block sums from the stored logits ([stream][query][domain
// token]), LQ queries loaded at a time.
constexpr int LQ = 16;
__global__ __launch_bounds__(64) void k_score_expsum_stored(ScoreArgs a, Units un,
                                                            const float* __restrict__ lg,
                                                            const float* __restrict__ norm_m,
                                                            float* __restrict__ part_z) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int blk, s, zq;
    unit_xyz(un, u, blk, s, zq);
    const float* lr = lg + (uint64_t)s * a.nq * a.n_ctx + (uint32_t)(blk * BLK + lane);
    const float* nm = norm_m + (uint64_t)s * a.nq;
    int q0 = zq * a.qper;
    const int q1 = min(a.nq, q0 + a.qper);
    for (; q0 + LQ <= q1; q0 += LQ) {
      float l[LQ];
#pragma unroll
      for (int j = 0; j < LQ; ++j) l[j] = lr[(uint64_t)(q0 + j) * a.n_ctx];
      block_expsum<LQ>(l, q0, a, s, blk, lane, nm, part_z);
    }
    for (; q0 < q1; ++q0) {
      const float l = lr[(uint64_t)q0 * a.n_ctx];
      block_expsum<1>(&l, q0, a, s, blk, lane, nm, part_z);
    }
  }
}

// grid (nq, streams), 64 threads.  Z = pairwise tree over the blocks
// (zero-padded to a power of two) of z_b: groups of 64 consecutive blocks are
// summed across lanes, then the group sums are combined pairwise in LDS.
// Every block holds 64 tokens, so this is the pairwise tree over the domain's
// tokens.
constexpr int NORM_GROUPS = (1 << 22) / BLK / 64;  // n_ctx <= 2^22
__global__ __launch_bounds__(64) void k_score_normalise(ScoreArgs a, Units un,
                                                        const float* __restrict__ part_z,
                                                        float* __restrict__ norm_iz) {
  __shared__ float grp[NORM_GROUPS];
  const int lane = threadIdx.x;
  // one wave: its LDS accesses execute in issue order, also across units
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int qi, s, z_;
    unit_xyz(un, u, qi, s, z_);
    const float* pz = part_z + ((uint64_t)s * a.nq + qi) * a.nblk;
    const int ng = (a.nblk + 63) / 64;
    int np = 1;
    while (np < ng) np <<= 1;
    for (int i = 0; i < ng; ++i) {
      const int b = 64 * i + lane;
      const float t = tree_sum64(b < a.nblk ? pz[b] : 0.0f);
      if (lane == 0) grp[i] = t;
    }
    for (int i = ng + lane; i < np; i += 64) grp[i] = 0.0f;
    // in-order LDS within the wave: level w reads [0, 2w) before writing [0, w)
    for (int w = np >> 1; w >= 1; w >>= 1)
      for (int j = lane; j < w; j += 64) grp[j] = grp[2 * j] + grp[2 * j + 1];
    if (lane == 0) norm_iz[(uint64_t)s * a.nq + qi] = 1.0f / grp[0];
  }
}

// Adds the probabilities NQ window queries q0.. give this lane's key to sc,
// in query order.
template <int NQ>
__device__ __forceinline__ void add_scores(const float* __restrict__ qs, int q0, const float* kf,
                                           float scale, const float* __restrict__ nm,
                                           const float* __restrict__ ni, float& sc) {
  float l[NQ];
  logits<NQ>(qs + (uint64_t)q0 * D, kf, scale, l);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const float e = spec_exp2((l[j] - nm[q0 + j]) * KVC_LOG2E);
    sc = sc + e * ni[q0 + j];
  }
}

// grid (ceil(region_len/64), streams), 64 threads: lane = region token.  The
// score is accumulated one window query at a time, in query order.
__global__ __launch_bounds__(64) void k_token_scores(ScoreArgs a, Units un,
                                                     const float* __restrict__ qf,
                                                     const float* __restrict__ norm_m,
                                                     const float* __restrict__ norm_iz,
                                                     float* __restrict__ scores,
                                                     float* __restrict__ scores_out) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
  int bx, s, z_;
  unit_xyz(un, u, bx, s, z_);
  const int tr = bx * 64 + lane;
  const bool valid = tr < a.region_len;
  const int t = a.region_begin + (valid ? tr : 0);
  float kf[D];
  load_row_f32(a.K + (uint64_t)s * a.kv_stride + (uint64_t)t * D, kf);
  const float* qs = qf + (uint64_t)s * a.nq * D;
  const float* nm = norm_m + (uint64_t)s * a.nq;
  const float* ni = norm_iz + (uint64_t)s * a.nq;
  float sc = 0.0f;
  int q0 = 0;
  for (; q0 + QB <= a.nq; q0 += QB) add_scores<QB>(qs, q0, kf, a.scale, nm, ni, sc);
  for (; q0 < a.nq; ++q0) add_scores<1>(qs, q0, kf, a.scale, nm, ni, sc);
  if (valid) {
    scores[(uint64_t)s * a.region_len + tr] = sc;
    if (scores_out) scores_out[(uint64_t)s * a.region_len + tr] = sc;
  }
  }
}

// The same scores from the logits the first pass stored ([stream][query]
// [domain token]): each term is computed from the same logit by the same
// operations, in the same query order, so the scores are identical.  Logits
// are loaded LQ queries at a time so that a wave keeps several loads in
// flight.  grid (ceil(region_len/64), streams), 64 threads: lane = token.
__global__ __launch_bounds__(64) void k_token_scores_stored(ScoreArgs a, Units un,
                                                            const float* __restrict__ lg,
                                                            const float* __restrict__ norm_m,
                                                            const float* __restrict__ norm_iz,
                                                            float* __restrict__ scores,
                                                            float* __restrict__ scores_out) {
  const int lane = threadIdx.x;
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int bx, s, z_;
    unit_xyz(un, u, bx, s, z_);
    const int tr = bx * 64 + lane;
    const bool valid = tr < a.region_len;
    const float* lr = lg + (uint64_t)s * a.nq * a.n_ctx + (uint32_t)(a.region_begin + (valid ? tr : 0));
    const float* nm = norm_m + (uint64_t)s * a.nq;
    const float* ni = norm_iz + (uint64_t)s * a.nq;
    float sc = 0.0f;
    int q0 = 0;
    for (; q0 + LQ <= a.nq; q0 += LQ) {
      float l[LQ];
#pragma unroll
      for (int j = 0; j < LQ; ++j) l[j] = lr[(uint64_t)(q0 + j) * a.n_ctx];
#pragma unroll
      for (int j = 0; j < LQ; ++j) {
        const float e = spec_exp2((l[j] - nm[q0 + j]) * KVC_LOG2E);
        sc = sc + e * ni[q0 + j];
      }
    }
    for (; q0 < a.nq; ++q0) {
      const float e = spec_exp2((lr[(uint64_t)q0 * a.n_ctx] - nm[q0]) * KVC_LOG2E);
      sc = sc + e * ni[q0];
    }
    if (valid) {
      scores[(uint64_t)s * a.region_len + tr] = sc;
      if (scores_out) scores_out[(uint64_t)s * a.region_len + tr] = sc;
    }
  }
}

// The same scores when the region has few tokens (one wave per 64 region
// tokens would leave most of the chip idle): TW waves share the 64 tokens,
// wave w computing the terms fl(exp(l - m) / Z) of queries q0 + QB w ..
// q0 + QB w + QB - 1 of each round of TW * QB queries into LDS, and wave 0
// adding the round's terms to the score in query order.  Terms and their
// order are those of k_token_scores, so the scores are identical.  grid
// (ceil(region_len/64), streams), 64 * TW threads.
template <int TW>
__global__ __launch_bounds__(64 * TW) void k_token_scores_shared(
    ScoreArgs a, Units un, const float* __restrict__ qf, const float* __restrict__ norm_m,
    const float* __restrict__ norm_iz, float* __restrict__ scores, float* __restrict__ scores_out) {
  constexpr int R = TW * QB;  // queries per round
  __shared__ float term[2][R][64];
  // the wave index made visibly uniform, so that query rows are scalar loads
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
  int bx, s, z_;
  unit_xyz(un, u, bx, s, z_);
  const int tr = bx * 64 + lane;
  const bool valid = tr < a.region_len;
  const int t = a.region_begin + (valid ? tr : 0);
  float kf[D];
  load_row_f32(a.K + (uint64_t)s * a.kv_stride + (uint64_t)t * D, kf);
  const float* qs = qf + (uint64_t)s * a.nq * D;
  const float* nm = norm_m + (uint64_t)s * a.nq;
  const float* ni = norm_iz + (uint64_t)s * a.nq;
  float sc = 0.0f;
  int buf = 0;
  // a round's buffer is rewritten two rounds later, after every wave has
  // passed the next barrier, which wave 0 reaches only after adding it
  for (int q0 = 0; q0 < a.nq; q0 += R, buf ^= 1) {
    const int qw = q0 + wv * QB;
    if (qw + QB <= a.nq) {
      float l[QB];
      logits<QB>(qs + (uint64_t)qw * D, kf, a.scale, l);
#pragma unroll
      for (int j = 0; j < QB; ++j)
        term[buf][wv * QB + j][lane] = spec_exp2((l[j] - nm[qw + j]) * KVC_LOG2E) * ni[qw + j];
    } else {
      for (int j = 0; j < QB && qw + j < a.nq; ++j) {
        float l1;
        logits<1>(qs + (uint64_t)(qw + j) * D, kf, a.scale, &l1);
        term[buf][wv * QB + j][lane] = spec_exp2((l1 - nm[qw + j]) * KVC_LOG2E) * ni[qw + j];
      }
    }
    __syncthreads();
    if (wv == 0) {
      const int n = min(R, a.nq - q0);
      for (int j = 0; j < n; ++j) sc = sc + term[buf][j][lane];
    }
  }
  if (wv == 0 && valid) {
    scores[(uint64_t)s * a.region_len + tr] = sc;
    if (scores_out) scores_out[(uint64_t)s * a.region_len + tr] = sc;
  }
  __syncthreads();  // the next unit's first round rewrites a buffer wave 0 may still be adding
  }
}

// ---------------------------------------------------------------------------
// Per-vector channel selection (Stage-1): 16 lanes per K or V vector.
// ---------------------------------------------------------------------------
struct SelectArgs {
  const uint16_t* K;
  const uint16_t* V;
  uint32_t* masks;
  float* rho;
  uint64_t kv_stride;
  int region_begin, region_len, nc;
  int cvals[MAX_NC];
};

constexpr int SEL_TOKENS = 16;  // tokens per block (x2 vectors, 8 per wave)

// NC = number of distinct channel counts; the NC threshold searches of a
// vector run interleaved (independent chains).
// A wave takes four vectors, one per 16-lane DPP row, and lane j of a row
// holds channels 8j..8j+7.  The c-th largest key is found bit by bit from
// the top: per-lane compares summed across the row with DPP (vector ALU
// only; a ballot-and-popcount search with one vector per wave keeps the
// shared scalar unit busy instead and measured 5 % slower).  Ties at the
// threshold go to the lower channels (an exclusive prefix count across the
// row).  Energies are pairwise trees: in-lane over 8 channels, then across
// the row, i.e. the pairwise tree over the 128 channels in index order.
__device__ __forceinline__ uint32_t row16_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true);
  return v;
}
// row16_sum_u32 of N values, each step applied to all before the next, so
// that one value's DPP move fills the wait states after another's
template <int N>
__device__ __forceinline__ void row16_sum_u32_n(uint32_t* v) {
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[j], 0xB1, 0xF, 0xF, true);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[j], 0x4E, 0xF, 0xF, true);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[j], 0x141, 0xF, 0xF, true);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[j], 0x140, 0xF, 0xF, true);
}
// exclusive prefix sum over the lanes of a 16-lane row (row_shr 1, 2, 4, 8;
// lanes shifted in from outside the row read 0)
__device__ __forceinline__ uint32_t row16_excl_scan_u32(uint32_t v) {
  uint32_t x = v;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
  return x - v;
}
typedef __attribute__((ext_vector_type(2))) uint16_t u16x2;
__device__ __forceinline__ float tree8(const float* v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Ascending bitonic sort of the 128 keys of every 16-lane row.  Key x of a
// row sits in lane x >> 3 of the row, dword x & 3, half (x >> 2) & 1 of k,
// so the stages with partner x ^ 1 and x ^ 2 pair whole dwords, x ^ 4 pairs
// the two halves of a dword and x ^ 8m pairs lanes m apart.  In each phase
// the blocks that sort downwards hold complemented keys (key ^ 0x7FFF
// reverses the order of 15-bit keys), so every compare-exchange puts the
// minimum at the lower index.  The c-th largest key of a row is then key
// 128 - c, whatever order equal keys end in.
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
// dwords a (lower keys) and b
__device__ __forceinline__ void cx_dwords(uint32_t& a, uint32_t& b) {
  const uint32_t m = pk_min_u16(a, b);
  b = pk_max_u16(a, b);
  a = m;
}
// the two halves of x (the low half holds the lower key)
__device__ __forceinline__ uint32_t cx_halves(uint32_t x) {
  // the swapped operand folds into the packed instructions' operand selects
  const u16x2 v = __builtin_bit_cast(u16x2, x);
  const u16x2 sw = __builtin_shufflevector(v, v, 1, 0);
  const uint32_t mn = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(v, sw));
  const uint32_t mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, sw));
  return (mn & 0xFFFFu) | (mx & 0xFFFF0000u);
}
// the same dword of the row's lane l ^ M (M = 1, 2, 4, 8)
template <int M>
__device__ __forceinline__ uint32_t row_partner(uint32_t x) {
  const int xi = (int)x;
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, true);
  if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, true);
  if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, xi, 0x128, 0xF, 0xF, true);
  // M == 4: lanes 0-3 and 8-11 of the row read 4 lanes up (row_shl:4),
  // lanes 4-7 and 12-15 4 lanes down (row_shr:4)
  const int t = __builtin_amdgcn_update_dpp(xi, xi, 0x104, 0xF, 0x5, false);
  return (uint32_t)__builtin_amdgcn_update_dpp(t, xi, 0x114, 0xF, 0xA, false);
}
// Lanes with bit M (of the row) hold complemented keys during this stage.
// Each lane takes the minimum of its own value and its partner's value
// complemented: the lower lane gets the minimum of the two keys, the upper
// lane the complement of their maximum.  The partner's move folds into the
// exclusive or (v_xor_b32_dpp), so a stage is two instructions per dword.
template <int M>
__device__ __forceinline__ void cx_lanes_c(uint32_t* k, uint32_t fv) {
#pragma unroll
  for (int d = 0; d < 4; ++d) k[d] = pk_min_u16(k[d], row_partner<M>(k[d]) ^ fv);
}
__device__ __forceinline__ void xor_all(uint32_t* k, uint32_t f) {
#pragma unroll
  for (int d = 0; d < 4; ++d) k[d] ^= f;
}
__device__ __forceinline__ void cx_in_lane(uint32_t* k, bool halves) {
  if (halves) {
#pragma unroll
    for (int d = 0; d < 4; ++d) k[d] = cx_halves(k[d]);
  }
  cx_dwords(k[0], k[2]);
  cx_dwords(k[1], k[3]);
  cx_dwords(k[0], k[1]);
  cx_dwords(k[2], k[3]);
}
__device__ __forceinline__ void row_sort128_u16(uint32_t* k, int lane) {
  constexpr uint32_t F = 0x7FFF7FFFu;
  const bool l1 = lane & 1, l2 = lane & 2, l4 = lane & 4, l8 = lane & 8;
  // phase 2: down where x & 2 (dwords 2, 3)
  k[2] ^= F;
  k[3] ^= F;
  cx_dwords(k[0], k[1]);
  cx_dwords(k[2], k[3]);
  // phase 4: down where x & 4 (high halves)
  k[0] ^= 0x7FFF0000u;
  k[1] ^= 0x7FFF0000u;
  k[2] ^= 0x00007FFFu;
  k[3] ^= 0x00007FFFu;
  cx_in_lane(k, false);
  // phases 8 .. 64: down where lane bit 0, 1, 2, 3 of the row is set; the
  // exclusive ors below move between the stored forms: direction flip of
  // the phase, complemented upper lanes of each lane stage, plain keys for
  // the in-lane stages
  const uint32_t c1 = l1 ? F : 0u, c2 = l2 ? F : 0u, c4 = l4 ? F : 0u, c8 = l8 ? F : 0u;
  // the complement mask in a vector register, so that the partner's move
  // folds into the exclusive or (a DPP operation takes no literal)
  uint32_t fv = F;
  asm volatile("" : "+v"(fv));
  xor_all(k, 0x7FFF0000u ^ c1);
  cx_in_lane(k, true);
  xor_all(k, c2);  // phase 16: key ^ c2, upper lanes of x ^ 8 complemented
  cx_lanes_c<1>(k, fv);
  xor_all(k, c1);
  cx_in_lane(k, true);
  xor_all(k, c4);  // phase 32
  cx_lanes_c<2>(k, fv);
  xor_all(k, c2 ^ c1);
  cx_lanes_c<1>(k, fv);
  xor_all(k, c1);
  cx_in_lane(k, true);
  xor_all(k, c8);  // phase 64
  cx_lanes_c<4>(k, fv);
  xor_all(k, c4 ^ c2);
  cx_lanes_c<2>(k, fv);
  xor_all(k, c2 ^ c1);
  cx_lanes_c<1>(k, fv);
  xor_all(k, c1);
  cx_in_lane(k, true);
  // phase 128, all upwards: key ^ c8 is already the form for x ^ 64
  cx_lanes_c<8>(k, fv);
  xor_all(k, c8 ^ c4);
  cx_lanes_c<4>(k, fv);
  xor_all(k, c4 ^ c2);
  cx_lanes_c<2>(k, fv);
  xor_all(k, c2 ^ c1);
  cx_lanes_c<1>(k, fv);
  xor_all(k, c1);
  cx_in_lane(k, true);
}

template <int NC>
__device__ __forceinline__ void select_unit_rows(const SelectArgs& a, int bx, int s) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rw = lane >> 4, j = lane & 15;
  // the unit's 2 * SEL_TOKENS vectors, 16 per pass (4 waves x 4 rows)
  for (int r0 = 0; r0 < 2 * SEL_TOKENS; r0 += 16) {
    const int r = r0 + 4 * wv + rw;
    const int tr = bx * SEL_TOKENS + (r >> 1);
    const int kv = r & 1;
    const bool valid = tr < a.region_len;  // uniform per row
    const uint16_t* row = (kv ? a.V : a.K) + (uint64_t)s * a.kv_stride +
                          (uint64_t)(a.region_begin + (valid ? tr : 0)) * D;
    const uint4 w = *reinterpret_cast<const uint4*>(row + 8 * j);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t k[8];
    float q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b = (wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      k[e] = b & 0x7FFFu;
      const float x = bf2f(b);
      q[e] = x * x;
    }
    const float Eall = row16_sum(tree8(q));
    // keys two to a dword: (key - cand) per 16-bit half has bit 15 set
    // exactly when key < cand (both are below 2^15), so one packed subtract
    // and a popcount of the two sign bits count two keys
    u16x2 k2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k2[i] = __builtin_bit_cast(u16x2, wd[i] & 0x7FFF7FFFu);
    uint32_t tau[NC];
    if constexpr (NC >= 2) {
      // one sort serves every channel count: c is a multiple of 8, so the
      // c-th largest key is the low half of dword 0 in lane 16 - c / 8
      uint32_t ks[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ks[i] = __builtin_bit_cast(uint32_t, k2[i]);
      row_sort128_u16(ks, lane);
#pragma unroll
      for (int v = 0; v < NC; ++v)
        tau[v] = (uint32_t)__shfl((int)(ks[0] & 0xFFFFu), (lane & 48) | (16 - a.cvals[v] / 8), 64);
    } else {
#pragma unroll
      for (int v = 0; v < NC; ++v) tau[v] = 0;
      for (int bit = 14; bit >= 0; --bit) {
        uint32_t cand[NC], lt[NC];
#pragma unroll
        for (int v = 0; v < NC; ++v) {
          cand[v] = tau[v] | (1u << bit);
          const u16x2 c2 = {(uint16_t)cand[v], (uint16_t)cand[v]};
          lt[v] = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            lt[v] += (uint32_t)__popc(__builtin_bit_cast(uint32_t, (u16x2)(k2[i] - c2)) & 0x80008000u);
        }
        row16_sum_u32_n<NC>(lt);  // keys below cand, of 128
#pragma unroll
        for (int v = 0; v < NC; ++v) tau[v] = (D - lt[v] >= (uint32_t)a.cvals[v]) ? cand[v] : tau[v];
      }
    }
    float ec_mine = 0.0f;  // kept energy of channel count j (lanes j < NC of the row)
#pragma unroll
    for (int v = 0; v < NC; ++v) {
      const uint32_t c = (uint32_t)a.cvals[v];
      // counts of keys above and below the threshold from the packed keys
      // (sign bit of each 16-bit difference), so that no per-key flag has
      // to live across both loops
      const u16x2 t2 = {(uint16_t)tau[v], (uint16_t)tau[v]};
      uint32_t gt = 0, lt = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gt += (uint32_t)__popc(__builtin_bit_cast(uint32_t, (u16x2)(t2 - k2[i])) & 0x80008000u);
        lt += (uint32_t)__popc(__builtin_bit_cast(uint32_t, (u16x2)(k2[i] - t2)) & 0x80008000u);
      }
      const uint32_t need = c - row16_sum_u32(gt);
      uint32_t rk = row16_excl_scan_u32(8u - gt - lt);  // ties in lower channels of the row
      uint32_t mb = 0;
      float qs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool eq = k[e] == tau[v];
        const bool sel = (k[e] > tau[v]) | (eq & (rk < need));
        rk += eq ? 1u : 0u;
        mb |= sel ? (1u << e) : 0u;
        qs[e] = sel ? q[e] : 0.0f;
      }
      const float Ec = row16_sum(tree8(qs));
      ec_mine = j == v ? Ec : ec_mine;
      if (valid) {
        const uint64_t o = (((uint64_t)s * a.region_len + tr) * a.nc + v) * 2 + kv;
        reinterpret_cast<uint8_t*>(a.masks)[o * 16 + j] = (uint8_t)mb;
      }
    }
    // lane j < NC of the row divides for channel count j: one division
    // sequence for all counts
    if (valid && j < NC) {
      const uint64_t o = (((uint64_t)s * a.region_len + tr) * a.nc + j) * 2 + kv;
      a.rho[o] = (Eall == 0.0f) ? 1.0f : ec_mine / Eall;
    }
  }
}

// grid: units of SEL_TOKENS tokens of a stream (K and V vectors), 256 threads.
template <int NC>
__global__ __launch_bounds__(256) void k_channel_select(SelectArgs a, Units un) {
  for (uint32_t u = blockIdx.x; u < un.total; u += gridDim.x) {
    int bx, s, z_;
    unit_xyz(un, u, bx, s, z_);
    select_unit_rows<NC>(a, bx, s);
  }
}

// ---------------------------------------------------------------------------
// Per-segment strategy choice.
// ---------------------------------------------------------------------------
struct ChooseArgs {
  const float* scores;
  const float* rho;
  const uint8_t* forced;
  kvc_seg_desc* desc;
  uint32_t* keep;
  float* objective;
  int region_len, S, n_seg, nc, n_strat, t2c_alpha, t2c_gamma;
  uint32_t dstride, feasible_mask;
  bool have_scores;
  uint32_t* keep_all;  // stream scope: keep sets of every strategy, else null
  float* J_all;        // stream scope: objectives of every strategy, else null
  int sT[KVC_MAX_STRATEGIES], sc[KVC_MAX_STRATEGIES], su[KVC_MAX_STRATEGIES];
};

// Keys of the segment's tokens: slot j of lane l is token 64*j + l.  Returns
// per slot whether the token is among the T best by (score desc, position asc).
__device__ __forceinline__ void top_t_flags(const uint32_t* key, const bool* valid, int NJ, int T,
                                            bool* out) {
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    uint32_t cnt = 0;
    for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(valid[j] && key[j] >= cand));
    if (cnt >= (uint32_t)T) tau = cand;
  }
  uint32_t ngt = 0;
  for (int j = 0; j < NJ; ++j) ngt += __popcll(__ballot(valid[j] && key[j] > tau));
  const uint32_t need = (uint32_t)T - ngt;
  uint32_t before = 0;
  for (int j = 0; j < NJ; ++j) {
    const uint64_t e = __ballot(valid[j] && key[j] == tau);
    const uint32_t rk = before + lanes_below(e);
    out[j] = valid[j] && (key[j] > tau || (key[j] == tau && rk < need));
    before += (uint32_t)__popcll(e);
  }
}

// Token2Chunk on one lane, from the top-(T-alpha) flags in `fl` (bytes, one
// per token); leaves exactly T flags set.
// a, ck: LDS scratch of >= S ints; done: >= S bytes.
__device__ void token2chunk_lane(const float* s, uint8_t* fl, int S, int T, int alpha, int gamma,
                                 int* a, int* ck, uint8_t* done) {
  int m = 0;
  for (int i = 0; i < S; ++i)
    if (fl[i]) a[m++] = i;
  int nc = 0;
  for (int k = 0; k + 1 < m; ++k) {
    const int gap = a[k + 1] - a[k] - 1;
    if (gap >= 1 && a[k + 1] - a[k] + 1 <= gamma) ck[nc++] = k;
  }
  for (int j = 0; j < nc; ++j) done[j] = 0;
  int used = 0;
  for (int it = 0; it < nc; ++it) {
    int best = -1, bg = 0;
    float bv = 0.0f;
    for (int j = 0; j < nc; ++j) {
      if (done[j]) continue;
      const int k = ck[j];
      const float v = s[a[k]] + s[a[k + 1]];
      const int g = a[k + 1] - a[k] - 1;
      if (best < 0 || v > bv || (v == bv && (g < bg || (g == bg && k < ck[best])))) {
        best = j;
        bv = v;
        bg = g;
      }
    }
    done[best] = 1;
    if (used + bg <= alpha) {
      const int k = ck[best];
      for (int t = a[k] + 1; t < a[k + 1]; ++t) fl[t] = 1;
      used += bg;
    }
  }
  int have = 0;
  for (int i = 0; i < S; ++i) have += fl[i];
  while (have < T) {
    int best = -1;
    for (int i = 0; i < S; ++i) {
      if (fl[i]) continue;
      if (best < 0 || s[i] > s[best]) best = i;  // first index wins ties
    }
    fl[best] = 1;
    ++have;
  }
}

// grid (n_seg, streams), 64 threads.
__global__ __launch_bounds__(64) void k_segment_choose(ChooseArgs a) {
  const int sg = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int S = a.S;
  const int NJ = S >= 64 ? S / 64 : 1;
  const int width = S >= 64 ? 64 : S;
  __shared__ float s_sc[256];
  __shared__ uint8_t s_fl[256];
  __shared__ int s_a[256], s_ck[256];
  __shared__ uint8_t s_done[256];
  __shared__ float s_J[KVC_MAX_STRATEGIES];
  __shared__ uint32_t s_keep[KVC_MAX_STRATEGIES][8];
  float sc[4];
  uint32_t key[4];
  bool valid[4];
  for (int j = 0; j < NJ; ++j) {
    const int t = 64 * j + lane;
    valid[j] = t < S;
    sc[j] = (valid[j] && a.have_scores) ? a.scores[(uint64_t)s * a.region_len + sg * S + t] : 0.0f;
    key[j] = __float_as_uint(sc[j]);
    if (valid[j]) s_sc[t] = sc[j];
  }
  __syncthreads();
  // Without the objective output only feasible strategies matter (and a
  // forced one, which is feasible or else replaced by the choice).  Keep
  // sets depend on T only, so consecutive strategies with the same T share
  // them.
  int last_T = -1;
  bool kp[4] = {false, false, false, false};
  for (int i = 0; i < a.n_strat; ++i) {
    if (!a.objective && !a.J_all && !((a.feasible_mask >> i) & 1u)) continue;
    const int T = a.sT[i], c = a.sc[i];
    if (T == last_T) {
      // same keep set as the previous strategy computed
    } else if (T == 0) {
      for (int j = 0; j < NJ; ++j) kp[j] = false;
    } else if (T >= S) {
      for (int j = 0; j < NJ; ++j) kp[j] = valid[j];
    } else if (a.t2c_alpha > 0) {
      top_t_flags(key, valid, NJ, T - a.t2c_alpha, kp);
      for (int j = 0; j < NJ; ++j)
        if (valid[j]) s_fl[64 * j + lane] = kp[j] ? 1 : 0;
      __syncthreads();
      if (lane == 0) token2chunk_lane(s_sc, s_fl, S, T, a.t2c_alpha, a.t2c_gamma, s_a, s_ck, s_done);
      __syncthreads();
      for (int j = 0; j < NJ; ++j) kp[j] = valid[j] && s_fl[64 * j + lane];
      __syncthreads();
    } else {
      top_t_flags(key, valid, NJ, T, kp);
    }
    last_T = T;
    // objective: pairwise tree over the segment's slots
    float tj[4];
    for (int j = 0; j < NJ; ++j) {
      float term = 0.0f;
      if (kp[j] && a.have_scores) {
        float rk = 1.0f, rv = 1.0f;
        if (c < D) {
          const uint64_t o = (((uint64_t)s * a.region_len + sg * S + 64 * j + lane) * a.nc + a.su[i]) * 2;
          rk = a.rho[o];
          rv = a.rho[o + 1];
        }
        term = sc[j] * (0.5f * (rk + rv));
      }
      tj[j] = width == 64 ? tree_sum64(term) : tree_sum_lanes(term, width);
    }
    float J;
    if (NJ == 1)
      J = tj[0];
    else if (NJ == 2)
      J = tj[0] + tj[1];
    else
      J = (tj[0] + tj[1]) + (tj[2] + tj[3]);
    for (int j = 0; j < NJ; ++j) {
      const uint64_t bal = __ballot(kp[j]);
      if (lane == 0) {
        s_keep[i][2 * j] = (uint32_t)bal;
        s_keep[i][2 * j + 1] = (uint32_t)(bal >> 32);
      }
    }
    if (lane == 0) s_J[i] = J;
  }
  __syncthreads();
  if (a.J_all) {
    // stream scope: every strategy's keep set and objective; k_stream_choose
    // chooses and writes the descriptor
    const uint64_t si = (uint64_t)s * a.n_seg + sg;
    const int nw = (S + 31) / 32;
    for (int i = lane; i < a.n_strat; i += 64) a.J_all[si * a.n_strat + i] = s_J[i];
    for (int e = lane; e < a.n_strat * nw; e += 64)
      a.keep_all[si * a.n_strat * nw + e] = s_keep[e / nw][e % nw];
    if (a.objective)
      for (int i = lane; i < a.n_strat; i += 64) a.objective[si * a.n_strat + i] = s_J[i];
    return;
  }
  if (lane == 0) {
    const uint64_t si = (uint64_t)s * a.n_seg + sg;
    int best = -1;
    uint8_t rej = 0;
    const uint8_t f = a.forced ? a.forced[si] : (uint8_t)KVC_DESC_CHOOSE;
    if (f < a.n_strat && ((a.feasible_mask >> f) & 1u)) {
      best = f;
    } else {
      if (a.forced && f != KVC_DESC_CHOOSE) rej = 0x80;
      for (int i = 0; i < a.n_strat; ++i) {
        if (!((a.feasible_mask >> i) & 1u)) continue;
        if (best < 0 || s_J[i] > s_J[best]) best = i;
      }
    }
    const int T = a.sT[best], c = a.sc[best];
    kvc_seg_desc d;
    d.offset = 0;
    d.n_tok = (uint16_t)T;
    d.n_ch = (uint16_t)(T > 0 ? c : 0);
    d.strategy = (uint8_t)best;
    d.flags = (uint8_t)(rej | (T >= S ? 1 : 0) | (c >= D ? 2 : 0));
    d.seg_tokens = (uint16_t)S;
    a.desc[(uint64_t)s * a.dstride + sg] = d;
    const int nw = (S + 31) / 32;
    for (int w = 0; w < nw; ++w) a.keep[si * nw + w] = s_keep[best][w];
    if (a.objective)
      for (int i = 0; i < a.n_strat; ++i) a.objective[si * a.n_strat + i] = s_J[i];
  }
}

// ---------------------------------------------------------------------------
// Per-stream budget: multiple-choice knapsack over the stream's segments by
// Lagrangian relaxation (MosaicKV abstract and Fig. 5 caption: strategies per
// segment under the memory target).  Every segment takes
// argmax_i fl(J_i - fl(lambda * bytes_i)) (ties to the lower index); lambda
// is the smallest fp32 value, by binary search over its bit patterns
// 0 .. 2^97, whose total fits the stream's bytes.
// ---------------------------------------------------------------------------
struct StreamChooseArgs {
  const float* J_all;
  const uint32_t* keep_all;
  kvc_seg_desc* desc;
  uint32_t* keep;
  uint64_t stream_bytes;
  uint32_t dstride;
  int n_seg, n_strat, S;
  int sT[KVC_MAX_STRATEGIES], sc[KVC_MAX_STRATEGIES];
  uint32_t seg_bytes[KVC_MAX_STRATEGIES];
};

constexpr int SC_THREADS = 256;

__device__ __forceinline__ int lagrange_best(const float* J, const StreamChooseArgs& a, float lambda) {
  int best = 0;
  float bv = J[0] - lambda * (float)a.seg_bytes[0];
  for (int i = 1; i < a.n_strat; ++i) {
    const float v = J[i] - lambda * (float)a.seg_bytes[i];
    if (v > bv) {
      bv = v;
      best = i;
    }
  }
  return best;
}

// Total bytes of the Lagrangian choice at lambda (block-wide, every thread
// gets it).
__device__ __forceinline__ uint64_t lagrange_total(const StreamChooseArgs& a, const float* Js,
                                                   float lambda, unsigned long long* tot) {
  uint64_t mine = 0;
  for (int sg = threadIdx.x; sg < a.n_seg; sg += SC_THREADS)
    mine += a.seg_bytes[lagrange_best(Js + (uint64_t)sg * a.n_strat, a, lambda)];
  if (threadIdx.x == 0) *tot = 0ull;
  __syncthreads();
  atomicAdd(tot, (unsigned long long)mine);
  __syncthreads();
  const uint64_t r = *tot;
  __syncthreads();
  return r;
}

// grid (streams), 256 threads.
__global__ __launch_bounds__(SC_THREADS) void k_stream_choose(StreamChooseArgs a) {
  __shared__ unsigned long long tot;
  const int s = blockIdx.x;
  const float* Js = a.J_all + (uint64_t)s * a.n_seg * a.n_strat;
  uint32_t u = 0u;
  if (lagrange_total(a, Js, 0.0f, &tot) > a.stream_bytes) {
    const uint32_t top = 0x70000000u;  // 2^97: every segment takes its smallest strategy
    u = top;
    if (lagrange_total(a, Js, __uint_as_float(top), &tot) <= a.stream_bytes) {
      uint32_t lo = 0u, hi = top;  // total(lo) > budget, total(hi) <= budget
      while (hi - lo > 1u) {
        const uint32_t mid = lo + (hi - lo) / 2u;
        if (lagrange_total(a, Js, __uint_as_float(mid), &tot) <= a.stream_bytes)
          hi = mid;
        else
          lo = mid;
      }
      u = hi;
    }
  }
  const float lambda = __uint_as_float(u);
  const int nw = (a.S + 31) / 32;
  for (int sg = threadIdx.x; sg < a.n_seg; sg += SC_THREADS) {
    const uint64_t si = (uint64_t)s * a.n_seg + sg;
    const int best = lagrange_best(Js + (uint64_t)sg * a.n_strat, a, lambda);
    const int T = a.sT[best], c = a.sc[best];
    kvc_seg_desc d;
    d.offset = 0;
    d.n_tok = (uint16_t)T;
    d.n_ch = (uint16_t)(T > 0 ? c : 0);
    d.strategy = (uint8_t)best;
    d.flags = (uint8_t)((T >= a.S ? 1 : 0) | (c >= D ? 2 : 0));
    d.seg_tokens = (uint16_t)a.S;
    a.desc[(uint64_t)s * a.dstride + sg] = d;
    for (int w = 0; w < nw; ++w) a.keep[si * nw + w] = a.keep_all[(si * a.n_strat + best) * nw + w];
  }
}

// ---------------------------------------------------------------------------
// Offsets: per-stream exclusive scan of the chosen segments' bytes.
// ---------------------------------------------------------------------------
struct ScanArgs {
  kvc_seg_desc* desc;
  uint64_t* used;
  uint64_t pstride, pbase;
  uint32_t dstride;
  int n_seg, S;
};

__global__ __launch_bounds__(64) void k_offsets_scan(ScanArgs a) {
  const int s = blockIdx.x, lane = threadIdx.x;
  uint64_t run = 0;
  for (int b0 = 0; b0 < a.n_seg; b0 += 64) {
    const int i = b0 + lane;
    kvc_seg_desc* d = a.desc + (uint64_t)s * a.dstride + i;
    const uint32_t by = (i < a.n_seg) ? seg_bytes(d->n_tok, d->n_ch, a.S) : 0u;
    uint32_t inc = by;
    for (int m = 1; m < 64; m <<= 1) {
      const uint32_t o = __shfl_up(inc, m, 64);
      if (lane >= m) inc += o;
    }
    if (i < a.n_seg) d->offset = a.pbase + (uint64_t)s * a.pstride + run + (inc - by);
    run += __shfl(inc, 63, 64);
  }
  if (lane == 0 && a.used) a.used[s] = run;
}

// ---------------------------------------------------------------------------
// Pack: one block per segment.
// ---------------------------------------------------------------------------
struct PackArgs {
  const uint16_t* K;
  const uint16_t* V;
  const uint32_t* masks;
  const uint32_t* keep;
  const kvc_seg_desc* desc;
  uint8_t* packed;
  uint64_t kv_stride, pstride, pbase;
  uint32_t dstride;
  int region_begin, region_len, S, n_seg, nc;
  int su[KVC_MAX_STRATEGIES];
};

__global__ __launch_bounds__(256) void k_pack(PackArgs a) {
  const int sg = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const kvc_seg_desc d = a.desc[(uint64_t)s * a.dstride + sg];
  const int T = d.n_tok, c = d.n_ch, S = a.S;
  if (T == 0) return;
  const uint64_t local = d.offset - a.pbase - (uint64_t)s * a.pstride;
  uint8_t* out = a.packed + (uint64_t)s * a.pstride + local;
  __shared__ uint16_t s_idx[256];
  if (wv == 0) {
    const int nw = (S + 31) / 32;
    const uint32_t* kw = a.keep + ((uint64_t)s * a.n_seg + sg) * nw;
    uint32_t before = 0;
    for (int j = 0; j * 64 < S; ++j) {
      const int t = 64 * j + lane;
      const bool on = t < S && ((kw[t >> 5] >> (t & 31)) & 1u);
      const uint64_t bal = __ballot(on);
      if (on) s_idx[before + lanes_below(bal)] = (uint16_t)t;
      before += (uint32_t)__popcll(bal);
    }
  }
  __syncthreads();
  const bool hasmask = c < D;
  const int u = a.su[d.strategy];
  const uint32_t kmask = 0, kval = hasmask ? 16u * T : 0u;
  const uint32_t vmask = kval + 2u * T * c, vval = vmask + (hasmask ? 16u * T : 0u);
  const uint32_t idxo = vval + 2u * T * c;
  // values: 16 lanes per kept row (lane q: channels 8q..8q+7, one 16-byte
  // load), four rows per wave; a masked row is compacted in LDS (each lane
  // drops its kept values at the row's running rank, an exclusive prefix of
  // the per-lane counts) and written out in 16-byte pieces
  __shared__ uint4 s_row[16][D / 8 + 1];
  __shared__ uint32_t s_vm[4][32];  // one transposed V block's mask bits per wave
  __shared__ __align__(16) uint16_t s_vv[4][8 * (D - 8)];  // and its values (c <= 120)
  const int rr = 4 * wv + (lane >> 4), q = lane & 15;
  for (int part = 0; part < 2; ++part) {
    const uint16_t* X = part ? a.V : a.K;
    const uint32_t mo = part ? vmask : kmask, vo = part ? vval : kval;
    if (part == 1 && hasmask) {
      // V of a masked segment: transposed blocks of 8 kept tokens, wave wv
      // takes blocks wv, wv + 4, ...  Lane l holds channels l (h 0) and
      // 64 + l (h 1): its 2 nb mask bits (bit nb h + t: token t keeps the
      // channel) go to bit 2 nb l of the block's mask bytes, its kept values
      // (h, t order) to the block's value bytes at the running rank, an
      // exclusive prefix of the lanes' counts.
      const uint16_t* Xs = X + (uint64_t)s * a.kv_stride + (uint64_t)a.region_begin * D;
      for (int bk = wv; 8 * bk < T; bk += 4) {
        const int nb = min(8, T - 8 * bk);
        uint32_t field = 0;
        uint16_t v0[8], v1[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          v0[t] = 0;
          v1[t] = 0;
          if (t < nb) {
            const int tr = sg * S + s_idx[8 * bk + t];
            const uint64_t o = (((uint64_t)s * a.region_len + tr) * a.nc + u) * 2 + 1;
            const uint4 m = reinterpret_cast<const uint4*>(a.masks)[o];
            const uint32_t b0 = ((lane < 32 ? m.x : m.y) >> (lane & 31)) & 1u;
            const uint32_t b1 = ((lane < 32 ? m.z : m.w) >> (lane & 31)) & 1u;
            field |= (b0 << t) | (b1 << (nb + t));
            const uint16_t* row = Xs + (uint64_t)tr * D;
            v0[t] = row[lane];
            v1[t] = row[64 + lane];
          }
        }
        const uint32_t cnt = (uint32_t)__popc(field);
        uint32_t k = wave_incl_scan_u32(cnt) - cnt;
        // the block's values are gathered in LDS (the wave's own words,
        // written and read in order by the same wave) and written out in
        // 16-byte pieces: 2 c nb bytes, a multiple of 16
        uint16_t* sv = s_vv[wv];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (t < nb && ((field >> t) & 1u)) sv[k++] = v0[t];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (t < nb && ((field >> (nb + t)) & 1u)) sv[k++] = v1[t];
        const int n16 = (2 * c * nb) / 16;
        uint4* bv = reinterpret_cast<uint4*>(out + vo + (uint64_t)16 * c * bk);
        for (int i = lane; i < n16; i += 64) bv[i] = reinterpret_cast<const uint4*>(sv)[i];
        // mask bits: 2 nb bits at bit 2 nb l, assembled in LDS (the wave's
        // own words, written and read in order by the same wave)
        if (lane < 32) s_vm[wv][lane] = 0u;
        const uint32_t bit = 2u * (uint32_t)nb * (uint32_t)lane;
        if (field) {
          atomicOr(&s_vm[wv][bit >> 5], field << (bit & 31u));
          if ((bit & 31u) + 2u * (uint32_t)nb > 32u)
            atomicOr(&s_vm[wv][(bit >> 5) + 1u], field >> (32u - (bit & 31u)));
        }
        if (lane < 4 * nb)
          reinterpret_cast<uint32_t*>(out + mo + (uint64_t)128 * bk)[lane] = s_vm[wv][lane];
      }
      continue;
    }
    if (hasmask) {
      for (int j = tid; j < T; j += 256) {
        const uint64_t o = (((uint64_t)s * a.region_len + sg * S + s_idx[j]) * a.nc + u) * 2 + part;
        reinterpret_cast<uint4*>(out + mo)[j] = reinterpret_cast<const uint4*>(a.masks)[o];
      }
    }
    for (int j0 = 0; j0 < T; j0 += 16) {
      const int j = j0 + rr;
      const bool live = j < T;
      const int tr = sg * S + s_idx[live ? j : 0];
      const uint16_t* row = X + (uint64_t)s * a.kv_stride + (uint64_t)(a.region_begin + tr) * D;
      const uint4 w = *reinterpret_cast<const uint4*>(row + 8 * q);
      if (!hasmask) {
        if (live) reinterpret_cast<uint4*>(out + vo + (uint64_t)j * 2 * D)[q] = w;
        continue;
      }
      const uint64_t o = (((uint64_t)s * a.region_len + tr) * a.nc + u) * 2 + part;
      const uint4 m = reinterpret_cast<const uint4*>(a.masks)[o];
      const uint32_t mw = q < 4 ? m.x : q < 8 ? m.y : q < 12 ? m.z : m.w;
      const uint32_t mb = live ? (mw >> (8 * (q & 3))) & 0xFFu : 0u;
      uint32_t rank = row16_excl_scan_u32((uint32_t)__popc(mb));
      uint16_t* dst = reinterpret_cast<uint16_t*>(&s_row[rr][0]);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((mb >> e) & 1u) {
          dst[rank] = (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
          ++rank;
        }
      }
      // the row's LDS writes and reads are by the same wave, in order
      if (live && q < c / 8)
        reinterpret_cast<uint4*>(out + vo + (uint64_t)j * 2 * c)[q] = s_row[rr][q];
    }
  }
  if (T < S) {
    const uint32_t nidx = ((2u * T + 15u) / 16u) * 8u;  // u16 slots incl. padding
    uint16_t* oi = reinterpret_cast<uint16_t*>(out + idxo);
    for (uint32_t j = tid; j < nidx; j += 256) oi[j] = j < (uint32_t)T ? s_idx[j] : (uint16_t)0;
  }
}

// ---------------------------------------------------------------------------
// 1-D launch over the units, at most max_waves / waves_per_group workgroups
// (at least one) when max_waves > 0.
static dim3 capped(const Units& u, uint32_t waves_per_group, uint32_t max_waves) {
  uint32_t n = u.total;
  if (max_waves) {
    const uint32_t cap = max_waves / waves_per_group > 0 ? max_waves / waves_per_group : 1u;
    if (n > cap) n = cap;
  }
  return dim3(n);
}

hipError_t launch_compress(const CompressPlan& p, hipStream_t st) {
  if (p.scoring) {
    ScoreArgs sa;
    sa.K = p.K;
    sa.Qw = p.Qw;
    sa.kv_stride = p.kv_stride;
    sa.qw_stride = p.qw_stride;
    sa.hkv = p.hkv;
    sa.hq = p.hq;
    sa.G = p.G;
    sa.W = p.W;
    sa.nq = p.nq;
    sa.nblk = p.nblk;
    sa.n_ctx = p.nblk * BLK;
    sa.region_begin = p.region_begin;
    sa.region_len = p.region_len;
    sa.scale = p.scale;
    // at least SCORE_WAVES waves per scoring kernel when the shape allows
    constexpr int64_t SCORE_WAVES = 16384;
    const int64_t pw = (int64_t)p.nblk * p.streams;
    int qsplit = (int)((SCORE_WAVES + pw - 1) / pw);
    // and at most 64 window queries per wave: the waves resident together
    // then read one 32 KB window of the fp32 queries, most of which the
    // scalar cache holds (all 256 queries of a stream, 128 KB, mostly miss
    // it); the key rows are read once per wave, nq / 64 times in all
    if (qsplit < (p.nq + 63) / 64) qsplit = (p.nq + 63) / 64;
    const int max_split = (p.nq + 4 * QB - 1) / (4 * QB);  // keep >= 4 rounds of QB per wave
    if (qsplit > max_split) qsplit = max_split;
    if (qsplit < 1) qsplit = 1;
    sa.qper = (((p.nq + qsplit - 1) / qsplit + QB - 1) / QB) * QB;
    qsplit = (p.nq + sa.qper - 1) / sa.qper;
    const Units uq{(uint32_t)p.nq, (uint32_t)p.streams, (uint32_t)p.nq * p.streams};
    const Units up{(uint32_t)p.nblk, (uint32_t)p.streams, (uint32_t)(p.nblk * p.streams * qsplit)};
    hipLaunchKernelGGL(k_q_convert, capped(uq, 1, p.max_waves), dim3(64), 0, st, sa, uq, p.qf);
    hipLaunchKernelGGL(k_score_partials, capped(up, 1, p.max_waves), dim3(64), 0, st, sa, up,
                       (const float*)p.qf, p.part_m, p.logits);
    hipLaunchKernelGGL(k_score_max, capped(uq, 1, p.max_waves), dim3(64), 0, st, sa, uq,
                       (const float*)p.part_m, p.norm_m);
    if (p.logits)
      hipLaunchKernelGGL(k_score_expsum_stored, capped(up, 1, p.max_waves), dim3(64), 0, st, sa,
                         up, (const float*)p.logits, (const float*)p.norm_m, p.part_z);
    else
      hipLaunchKernelGGL(k_score_expsum, capped(up, 1, p.max_waves), dim3(64), 0, st, sa, up,
                         (const float*)p.qf, (const float*)p.norm_m, p.part_z);
    hipLaunchKernelGGL(k_score_normalise, capped(uq, 1, p.max_waves), dim3(64), 0, st, sa, uq,
                       (const float*)p.part_z, p.norm_iz);
    const uint32_t tx = (uint32_t)(p.region_len + 63) / 64;
    const Units ut{tx, (uint32_t)p.streams, tx * (uint32_t)p.streams};
    if (p.logits)
      hipLaunchKernelGGL(k_token_scores_stored, capped(ut, 1, p.max_waves), dim3(64), 0, st, sa,
                         ut, (const float*)p.logits, (const float*)p.norm_m,
                         (const float*)p.norm_iz, p.scores, p.scores_out);
    else if ((int64_t)ut.total * 4 <= SCORE_WAVES && p.nq >= 8 * QB)
      hipLaunchKernelGGL(k_token_scores_shared<8>, capped(ut, 8, p.max_waves), dim3(512), 0, st,
                         sa, ut, (const float*)p.qf, (const float*)p.norm_m,
                         (const float*)p.norm_iz, p.scores, p.scores_out);
    else
      hipLaunchKernelGGL(k_token_scores, capped(ut, 1, p.max_waves), dim3(64), 0, st, sa, ut,
                         (const float*)p.qf, (const float*)p.norm_m, (const float*)p.norm_iz,
                         p.scores, p.scores_out);
  }
  // selection and packing read the rotated region vectors when rotating
  const uint16_t* selK = p.K;
  const uint16_t* selV = p.V;
  uint64_t sel_stride = p.kv_stride;
  int sel_begin = p.region_begin;
  if (p.rotate) {
    RotatePlan rp;
    rp.K = p.K;
    rp.V = p.V;
    rp.kv_stride = p.kv_stride;
    rp.region_begin = p.region_begin;
    rp.region_len = p.region_len;
    rp.streams = p.streams;
    rp.n_span = p.n_span;
    rp.span_len = p.span_len;
    rp.gram = p.gram;
    rp.rot = p.rot;
    rp.YK = p.YK;
    rp.YV = p.YV;
    const hipError_t e = launch_rotate(rp, st);
    if (e != hipSuccess) return e;
    selK = p.YK;
    selV = p.YV;
    sel_stride = (uint64_t)p.region_len * D;
    sel_begin = 0;
  }
  if (p.nc > 0) {
    SelectArgs se;
    se.K = selK;
    se.V = selV;
    se.masks = p.masks;
    se.rho = p.rho;
    se.kv_stride = sel_stride;
    se.region_begin = sel_begin;
    se.region_len = p.region_len;
    se.nc = p.nc;
    for (int i = 0; i < MAX_NC; ++i) se.cvals[i] = p.cvals[i];
    const uint32_t sx = (uint32_t)(p.region_len + SEL_TOKENS - 1) / SEL_TOKENS;
    const Units us{sx, (uint32_t)p.streams, sx * (uint32_t)p.streams};
    const dim3 grid = capped(us, 4, p.max_waves);
    switch (p.nc) {
      case 1: hipLaunchKernelGGL(k_channel_select<1>, grid, dim3(256), 0, st, se, us); break;
      case 2: hipLaunchKernelGGL(k_channel_select<2>, grid, dim3(256), 0, st, se, us); break;
      case 3: hipLaunchKernelGGL(k_channel_select<3>, grid, dim3(256), 0, st, se, us); break;
      case 4: hipLaunchKernelGGL(k_channel_select<4>, grid, dim3(256), 0, st, se, us); break;
      case 5: hipLaunchKernelGGL(k_channel_select<5>, grid, dim3(256), 0, st, se, us); break;
      case 6: hipLaunchKernelGGL(k_channel_select<6>, grid, dim3(256), 0, st, se, us); break;
      case 7: hipLaunchKernelGGL(k_channel_select<7>, grid, dim3(256), 0, st, se, us); break;
      default: hipLaunchKernelGGL(k_channel_select<8>, grid, dim3(256), 0, st, se, us); break;
    }
  }
  ChooseArgs ca;
  ca.scores = p.scores;
  ca.rho = p.rho;
  ca.forced = p.forced;
  ca.desc = p.desc;
  ca.keep = p.keep;
  ca.objective = p.objective;
  ca.region_len = p.region_len;
  ca.S = p.S;
  ca.n_seg = p.n_seg;
  ca.nc = p.nc;
  ca.n_strat = p.n_strat;
  ca.t2c_alpha = p.t2c_alpha;
  ca.t2c_gamma = p.t2c_gamma;
  ca.dstride = p.dstride;
  ca.feasible_mask = p.feasible_mask;
  ca.have_scores = p.scoring;
  for (int i = 0; i < KVC_MAX_STRATEGIES; ++i) {
    ca.sT[i] = p.sT[i];
    ca.sc[i] = p.sc[i];
    ca.su[i] = p.su[i];
  }
  ca.keep_all = p.stream_budget ? p.keep_all : nullptr;
  ca.J_all = p.stream_budget ? p.J_all : nullptr;
  hipLaunchKernelGGL(k_segment_choose, dim3(p.n_seg, p.streams), dim3(64), 0, st, ca);
  if (p.stream_budget) {
    StreamChooseArgs sa;
    sa.J_all = p.J_all;
    sa.keep_all = p.keep_all;
    sa.desc = p.desc;
    sa.keep = p.keep;
    sa.stream_bytes = p.stream_bytes;
    sa.dstride = p.dstride;
    sa.n_seg = p.n_seg;
    sa.n_strat = p.n_strat;
    sa.S = p.S;
    for (int i = 0; i < KVC_MAX_STRATEGIES; ++i) {
      sa.sT[i] = p.sT[i];
      sa.sc[i] = p.sc[i];
      sa.seg_bytes[i] = p.seg_bytes[i];
    }
    hipLaunchKernelGGL(k_stream_choose, dim3(p.streams), dim3(SC_THREADS), 0, st, sa);
  }
  ScanArgs sc;
  sc.desc = p.desc;
  sc.used = p.used;
  sc.pstride = p.pstride;
  sc.pbase = p.pbase;
  sc.dstride = p.dstride;
  sc.n_seg = p.n_seg;
  sc.S = p.S;
  hipLaunchKernelGGL(k_offsets_scan, dim3(p.streams), dim3(64), 0, st, sc);
  PackArgs pa;
  pa.K = selK;
  pa.V = selV;
  pa.masks = p.masks;
  pa.keep = p.keep;
  pa.desc = p.desc;
  pa.packed = p.packed;
  pa.kv_stride = sel_stride;
  pa.pstride = p.pstride;
  pa.pbase = p.pbase;
  pa.dstride = p.dstride;
  pa.region_begin = sel_begin;
  pa.region_len = p.region_len;
  pa.S = p.S;
  pa.n_seg = p.n_seg;
  pa.nc = p.nc;
  for (int i = 0; i < KVC_MAX_STRATEGIES; ++i) pa.su[i] = p.su[i];
  hipLaunchKernelGGL(k_pack, dim3(p.n_seg, p.streams), dim3(256), 0, st, pa);
  return hipGetLastError();
}

}  // namespace kvc
