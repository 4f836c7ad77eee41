// kvc_decode.hip -- gfx950 decode attention over compressed KV segments
// (MosaicKV review page, Fig. 6 caption: PackedAttention over the packed KV
// format).  One wave per (stream, split): the split's descriptors are
// streamed through LDS in chunks of 16 kept tokens; each kept vector is
// expanded from (bitmask, compact bf16 values) to a dense 128-channel row,
// q.k and p.v run on MFMA (bf16 inputs, fp32 accumulation), and the softmax
// is online in base 2.  A second kernel merges the splits (log-sum-exp) and
// rounds the output to bf16.
//
// MFMA row mapping: the q head h of the group occupies A-row
// 4*(h & 3) + (h >> 2), so in the 16x16 accumulator layout (lane l, item j
// <-> row 4*(l>>4)+j, column l&15) lane l's item j belongs to head 4*j+(l>>4)
// and to token/channel l&15 -- for G <= 4 every head's scores and outputs sit
// in item 0 of its own 16-lane row.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int CT = 16;                       // kept tokens per chunk
constexpr int STAGE_BYTES = CT * 16 + CT * 256;  // masks + values of one chunk

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* packed;
  const kvc_seg_desc* desc;
  const uint32_t* n_desc;
  float* part_ml;
  float* part_acc;
  int hkv, hq, G, maxd, splits;
  float sl2;  // scale * log2(e)
};

// Copies `bytes` (multiple of 16) from global to LDS with the wave's lanes.
__device__ __forceinline__ void stage16(uint4* dst, const uint8_t* src, uint32_t bytes, int lane) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  for (uint32_t i = lane; i < bytes / 16; i += 64) dst[i] = s4[i];
}

// Dense channels 32*kk + 8*grp .. +7 of token `tok` of the staged chunk.
// Staged chunk: masks [nt][16 B] (if hasmask) then values [nt][c] bf16.
__device__ __forceinline__ u16x8_t expand8(const uint8_t* st, int tok, int kk, int grp, int nt,
                                           int c, bool hasmask) {
  u16x8_t r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (tok >= nt) return r;
  if (!hasmask) {
    return *reinterpret_cast<const u16x8_t*>(st + tok * 256 + 2 * (32 * kk + 8 * grp));
  }
  const uint32_t* m = reinterpret_cast<const uint32_t*>(st + 16 * tok);
  const uint16_t* vals = reinterpret_cast<const uint16_t*>(st + 16 * nt + 2 * c * tok);
  uint32_t rk = 0;
  for (int w = 0; w < kk; ++w) rk += __popc(m[w]);
  const uint32_t mw = m[kk];
  rk += __popc(mw & ((1u << (8 * grp)) - 1u));
  const uint32_t byte = (mw >> (8 * grp)) & 0xFFu;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((byte >> i) & 1u) {
      r[i] = vals[rk];
      ++rk;
    }
  }
  return r;
}

template <int JG>
__global__ __launch_bounds__(64) void k_decode_split(DecodeArgs a) {
  const int sp = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int grp = lane >> 4, col = lane & 15;
  const int b = s / a.hkv, h = s - b * a.hkv;
  __shared__ uint4 kst[STAGE_BYTES / 16];
  __shared__ uint4 vst[STAGE_BYTES / 16];
  __shared__ uint16_t vt[D * CT];   // dense V of the chunk, [channel][token]
  __shared__ uint16_t pl[16 * CT];  // probabilities, [head][token]

  for (int i = lane; i < 16 * CT; i += 64) pl[i] = 0;

  // A operand of the score MFMA: row col holds head hh (zero if none)
  const int hh = 4 * (col & 3) + (col >> 2);
  const bool hh_ok = hh < a.G;
  const uint16_t* qh = a.q + ((uint64_t)(b * a.hq + h * a.G + (hh_ok ? hh : 0))) * D;
  bf16x8_t qa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (hh_ok) v = *reinterpret_cast<const u16x8_t*>(qh + 32 * kk + 8 * grp);
    qa[kk] = __builtin_bit_cast(bf16x8_t, v);
  }

  f32x4_t O[8];
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) O[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[JG], l_run[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
  }

  const int nd = a.n_desc ? min((int)a.n_desc[s], a.maxd) : a.maxd;
  const int d0 = (int)(((int64_t)sp * nd) / a.splits);
  const int d1 = (int)(((int64_t)(sp + 1) * nd) / a.splits);
  const kvc_seg_desc* dl = a.desc + (uint64_t)s * a.maxd;
  const uint8_t* kst8 = reinterpret_cast<const uint8_t*>(kst);
  const uint8_t* vst8 = reinterpret_cast<const uint8_t*>(vst);

  for (int di = d0; di < d1; ++di) {
    const kvc_seg_desc d = dl[di];
    const int T = d.n_tok, c = d.n_ch;
    if (T == 0) continue;
    const bool hasmask = c < D;
    const uint8_t* base = a.packed + d.offset;
    const uint32_t mb = hasmask ? 16u * T : 0u;
    const uint8_t* kval = base + mb;
    const uint8_t* vmask = kval + 2u * T * c;
    const uint8_t* vval = vmask + mb;
    for (int t0 = 0; t0 < T; t0 += CT) {
      const int nt = min(CT, T - t0);
      __syncthreads();
      if (hasmask) {
        stage16(kst, base + 16 * t0, 16 * nt, lane);
        stage16(vst, vmask + 16 * t0, 16 * nt, lane);
      }
      stage16(kst + (hasmask ? nt : 0), kval + 2 * c * t0, 2 * c * nt, lane);
      stage16(vst + (hasmask ? nt : 0), vval + 2 * c * t0, 2 * c * nt, lane);
      __syncthreads();

      // scores of the chunk: S^T = Q Kd^T
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u16x8_t kb = expand8(kst8, col, kk, grp, nt, c, hasmask);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8_t, kb),
                                                       sacc, 0, 0, 0);
      }
      // online softmax, one head per (16-lane row, item j)
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        const int hd = 4 * j + grp;
        const bool ok = col < nt && hd < a.G;
        const float x = ok ? sacc[j] * a.sl2 : -INFINITY;
        float cm = x;
        cm = fmaxf(cm, __shfl_xor(cm, 1, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 2, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 4, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 8, 64));
        const float mn = fmaxf(m_run[j], cm);
        float alpha = 1.0f, p = 0.0f;
        if (mn != -INFINITY) {
          alpha = exp2f(m_run[j] - mn);
          p = exp2f(x - mn);
        }
        float rs = p;
        rs += __shfl_xor(rs, 1, 64);
        rs += __shfl_xor(rs, 2, 64);
        rs += __shfl_xor(rs, 4, 64);
        rs += __shfl_xor(rs, 8, 64);
        l_run[j] = l_run[j] * alpha + rs;
        m_run[j] = mn;
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) O[nn][j] *= alpha;
        if (hd < a.G) pl[hd * CT + col] = (uint16_t)f2bf(p);
      }
      // dense V of the chunk, transposed into LDS
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u16x8_t vb = expand8(vst8, col, kk, grp, nt, c, hasmask);
#pragma unroll
        for (int i = 0; i < 8; ++i) vt[(32 * kk + 8 * grp + i) * CT + col] = vb[i];
      }
      __syncthreads();
      // O += P Vd
      s16x4_t pa = {0, 0, 0, 0};
      if (hh_ok) pa = *reinterpret_cast<const s16x4_t*>(pl + hh * CT + 4 * grp);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        const s16x4_t vb = *reinterpret_cast<const s16x4_t*>(vt + (16 * nn + col) * CT + 4 * grp);
        O[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[nn], 0, 0, 0);
      }
    }
  }

  // partial state of this split
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    const int hd = 4 * j + grp;
    if (hd < a.G) {
      const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + hd) * a.splits + sp;
      if (col == 0) {
        a.part_ml[2 * pi] = m_run[j];
        a.part_ml[2 * pi + 1] = l_run[j];
      }
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) a.part_acc[pi * D + 16 * nn + col] = O[nn][j];
    }
  }
}

// grid (batch*n_q_heads), 128 threads: lane = channel.
__global__ __launch_bounds__(128) void k_decode_reduce(const float* __restrict__ part_ml,
                                                       const float* __restrict__ part_acc,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse, int splits) {
  const int r = blockIdx.x, ch = threadIdx.x;
  const float* ml = part_ml + (uint64_t)r * splits * 2;
  float M = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, ml[2 * sp]);
  if (M == -INFINITY) {
    out[(uint64_t)r * D + ch] = 0;
    if (lse && ch == 0) lse[r] = -INFINITY;
    return;
  }
  float L = 0.0f, acc = 0.0f;
  for (int sp = 0; sp < splits; ++sp) {
    const float w = exp2f(ml[2 * sp] - M);
    L += ml[2 * sp + 1] * w;
    acc += part_acc[((uint64_t)r * splits + sp) * D + ch] * w;
  }
  out[(uint64_t)r * D + ch] = (uint16_t)f2bf(acc / L);
  if (lse && ch == 0) lse[r] = (M + log2f(L)) * 0.69314718055994530942f;
}

hipError_t launch_decode(const DecodePlan& p, hipStream_t st) {
  DecodeArgs a;
  a.q = p.q;
  a.packed = p.packed;
  a.desc = p.desc;
  a.n_desc = p.n_desc;
  a.part_ml = p.part_ml;
  a.part_acc = p.part_acc;
  a.hkv = p.hkv;
  a.hq = p.hq;
  a.G = p.G;
  a.maxd = p.maxd;
  a.splits = p.splits;
  a.sl2 = p.scale * KVC_LOG2E;
  const dim3 grid(p.splits, p.streams);
  if (p.G <= 4)
    hipLaunchKernelGGL(k_decode_split<1>, grid, dim3(64), 0, st, a);
  else if (p.G <= 8)
    hipLaunchKernelGGL(k_decode_split<2>, grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(k_decode_split<4>, grid, dim3(64), 0, st, a);
  hipLaunchKernelGGL(k_decode_reduce, dim3(p.batch * p.hq), dim3(128), 0, st, p.part_ml, p.part_acc,
                     p.out, p.lse, p.splits);
  return hipGetLastError();
}

}  // namespace kvc
