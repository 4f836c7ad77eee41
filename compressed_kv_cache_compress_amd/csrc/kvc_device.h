// kvc_device.h -- device helpers for the gfx950 kernels: bf16 bit handling,
// the specified fp32 exp2, and wave64 reductions whose summation order is the
// pairwise tree (adjacent pairs first) used throughout the selection path.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace kvc {

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// log2(e) rounded to fp32.
#define KVC_LOG2E 0x1.715476p+0f

// Maximum of two non-NaN floats in one instruction (v_maximum3_f32).  It
// equals fmaxf except that +0 ranks above -0; every caller subtracts the
// maximum or compares against it, where the sign of a zero changes nothing.
__device__ __forceinline__ float fmax_nn(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// 2^y for y <= 0 from the Taylor series of e^(f ln 2) truncated after the
// degree-7 term (coefficients ln2^k / k! rounded to fp32), evaluated by Horner
// with fused multiply-adds after the split y = n + f, n = rint(y), |f| <= 1/2.
// Below -125 the result is +0, so no result is subnormal.  Every operation is
// a correctly rounded IEEE fp32 operation, so the value is reproducible on any
// IEEE machine that evaluates the same sequence.
__device__ __forceinline__ float spec_exp2(float y) {
  // branch-free: evaluate at max(y, -125) and select
  const float yc = fmax_nn(y, -125.0f);
  const float n = __builtin_rintf(yc);
  const float f = yc - n;
  float p = 0x1.ffcbfcp-17f;
  p = __builtin_fmaf(p, f, 0x1.430912p-13f);
  p = __builtin_fmaf(p, f, 0x1.5d87fep-10f);
  p = __builtin_fmaf(p, f, 0x1.3b2ab6p-7f);
  p = __builtin_fmaf(p, f, 0x1.c6b08ep-5f);
  p = __builtin_fmaf(p, f, 0x1.ebfbe0p-3f);
  p = __builtin_fmaf(p, f, 0x1.62e430p-1f);
  p = __builtin_fmaf(p, f, 1.0f);
  const float r = __builtin_ldexpf(p, (int)n);
  return (y >= -125.0f) ? r : 0.0f;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Sum over `width` consecutive lanes (a power of two <= 64) in pairwise-tree
// order: lanes 2i and 2i+1 first, then pairs of pairs, ...  IEEE addition is
// commutative, so every lane of the group ends with the same bits.
__device__ __forceinline__ float tree_sum_lanes(float v, int width = 64) {
  for (int m = 1; m < width; m <<= 1) v = v + shfl_xor_f(v, m);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

// Cross-lane moves inside DPP rows of 16 lanes (controls: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror).  Every lane has a valid
// source under these controls; written as an update with bound_ctrl so that
// the compiler folds the move into the consuming add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Maximum and pairwise-tree sum over the 16 lanes of a DPP row (every lane
// gets the result): lane pairs, quads, 8-lane halves, then the two halves.
__device__ __forceinline__ float row16_max(float v) {
  v = fmax_nn(v, dpp_mov<0xB1>(v));
  v = fmax_nn(v, dpp_mov<0x4E>(v));
  v = fmax_nn(v, dpp_mov<0x141>(v));
  v = fmax_nn(v, dpp_mov<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_mov<0xB1>(v);
  v = v + dpp_mov<0x4E>(v);
  v = v + dpp_mov<0x141>(v);
  v = v + dpp_mov<0x140>(v);
  return v;
}

// Pairwise-tree sum over the 64 lanes of a full wave (every lane active),
// returned wave-uniform.  Same order as tree_sum_lanes: lane pairs, quads,
// 8-lane halves and 16-lane rows by DPP (after each step the lanes of a group
// agree, so a mirror reaches the partner group), then (r0 + r1) + (r2 + r3)
// over the four rows.
__device__ __forceinline__ float tree_sum64(float v) {
  v = row16_sum(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Maximum over the 64 lanes of a full wave, returned wave-uniform.
__device__ __forceinline__ float max64(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmax_nn(fmax_nn(r0, r1), fmax_nn(r2, r3));
}

// max64 and tree_sum64 of N independent values at once, each step applied
// to all of them before the next, so that the DPP moves of one value fill
// the wait states after another's (same operations and order per value).
template <int N>
__device__ __forceinline__ void max64_n(float* v) {
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = fmax_nn(v[j], dpp_mov<0xB1>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = fmax_nn(v[j], dpp_mov<0x4E>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = fmax_nn(v[j], dpp_mov<0x141>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = fmax_nn(v[j], dpp_mov<0x140>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 48));
    v[j] = fmax_nn(fmax_nn(r0, r1), fmax_nn(r2, r3));
  }
}
template <int N>
__device__ __forceinline__ void tree_sum64_n(float* v) {
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0xB1>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x4E>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x141>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x140>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[j]), 48));
    v[j] = (r0 + r1) + (r2 + r3);
  }
}

// Signed integer with the order of a non-NaN float (-0 below +0): the
// magnitude bits of a negative float are inverted.  The map is its own
// inverse.  Integer maxima fold into one DPP instruction per step, where a
// float maximum needs a move and a three-operand maximum.
__device__ __forceinline__ int32_t f_order_key(float x) {
  const int32_t i = __float_as_int(x);
  return i ^ (int32_t)((uint32_t)(i >> 31) >> 1);
}
__device__ __forceinline__ float f_order_key_inv(int32_t k) {
  return __int_as_float(k ^ (int32_t)((uint32_t)(k >> 31) >> 1));
}
template <int CTRL>
__device__ __forceinline__ int32_t dpp_mov_i(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// max64_n and tree_sum64_n with the last two steps done by the row
// broadcasts (lane 15 of each row into the next row, then lane 31 into rows
// 2 and 3): lane 63 ends with (r3 . r2) . (r1 . r0), the same tree as
// (r0 . r1) . (r2 . r3) since both operations commute.  Only lane 63 holds
// the result; the maxima are returned wave-uniform, the sums stay in lane 63.
template <int N>
__device__ __forceinline__ void max64_n_last(float* v) {
  int32_t k[N];
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = f_order_key(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = max(k[j], dpp_mov_i<0xB1>(k[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = max(k[j], dpp_mov_i<0x4E>(k[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = max(k[j], dpp_mov_i<0x141>(k[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = max(k[j], dpp_mov_i<0x140>(k[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = max(k[j], dpp_mov_i<0x142>(k[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) k[j] = max(k[j], dpp_mov_i<0x143>(k[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = f_order_key_inv(__builtin_amdgcn_readlane(k[j], 63));
}
template <int N>
__device__ __forceinline__ void tree_sum64_n_last(float* v) {
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0xB1>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x4E>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x141>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x140>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x142>(v[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = v[j] + dpp_mov<0x143>(v[j]);
}

// Inclusive sum over the 64 lanes: rows by row_shr, then the row broadcasts
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
  return x;
}

// Count of set bits of a 64-bit lane mask below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Packed bytes of one segment (layout in kvc.h).
__host__ __device__ __forceinline__ uint32_t seg_bytes(uint32_t T, uint32_t c, uint32_t S) {
  if (T == 0) return 0;
  const uint32_t mk = (c < 128) ? 16u * T : 0u;
  const uint32_t vals = 2u * T * c;
  const uint32_t idx = (T < S) ? ((2u * T + 15u) / 16u) * 16u : 0u;
  return 2u * mk + 2u * vals + idx;
}

}  // namespace kvc
