// kvc_rotate.hip -- gfx950 kernels of the SVD rotation applied before the
// per-vector channel selection (MosaicKV review page, Fig. 6 caption,
// Stage-1: the rotation matrix R of the K and of the V matrix from their
// SVD, the vectors rotated before the top-r elements of each are kept;
// Fig. 4: after the rotation the important elements sit in a few channels).
//
// One R per span and side (K, V): the region one call compresses is cut into
// spans of span_len tokens (one span when the caller asks for none):
//   gram          X^T X of each span, every entry one fma chain over the
//                 span's tokens in order (64 x 64 tiles, 4 x 4 per thread)
//   jacobi        cyclic Jacobi in fp32 with the round-robin (tournament)
//                 pair ordering of parallel Jacobi methods: 127 rounds of 64
//                 rotations on disjoint index pairs per sweep, each round's
//                 rotations computed from the matrix as it stands and applied
//                 to its rows, its columns and the eigenvector columns; R =
//                 eigenvectors ordered by eigenvalue (largest first, ties to
//                 the lower index)
//   rotate_vec    y = R^T x rounded to bf16 for every region vector, with the
//                 R of its span
// Every operation is a correctly rounded fp32 operation in a fixed order
// (division and square root correctly rounded, no contraction), so R and
// the rotated vectors are reproducible bit for bit.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

constexpr int JSWEEPS = 10;   // Jacobi sweeps
constexpr int APAD = D + 1;   // LDS row stride of the Jacobi matrices (conflict-free columns)

// grid (3 tiles * 2 sides, spans, streams), 256 threads.  Tile (bi, bj) of
// 64 x 64 entries with bi <= bj (the lower-left tile is the transpose of the
// upper-right one: fma(a, b, c) = fma(b, a, c), so the matrix is exactly
// symmetric); thread (ti, tj) = (tid / 16, tid % 16) owns rows bi*64 + 4ti ..
// +3 and columns bj*64 + 4tj .. +3 and runs their 16 fma chains over the
// span's tokens in order.
__global__ __launch_bounds__(256) void k_gram(RotatePlan p) {
  __shared__ float4 xs[64 * D / 4];  // 64 tokens x 128 channels, fp32
  const int tid = threadIdx.x;
  const int s = blockIdx.z, span = blockIdx.y;
  const int side = blockIdx.x / 3, tile = blockIdx.x - side * 3;
  const int bi = tile == 2 ? 1 : 0, bj = tile == 0 ? 0 : 1;
  const int ti = tid >> 4, tj = tid & 15;
  const int ri = bi * 64 + 4 * ti, rj = bj * 64 + 4 * tj;
  const uint16_t* X = (side ? p.V : p.K) + (uint64_t)s * p.kv_stride + (uint64_t)p.region_begin * D;
  const int t_lo = span * p.span_len, t_hi = t_lo + p.span_len;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int t0 = t_lo; t0 < t_hi; t0 += 64) {
    const int n = min(64, t_hi - t0);
    __syncthreads();  // the previous chunk's reads are done
    {
      // thread: token tid / 4, channels 32 * (tid % 4) .. +31
      const int tk = tid >> 2, part = tid & 3;
      if (tk < n) {
        const uint4* src = reinterpret_cast<const uint4*>(X + (uint64_t)(t0 + tk) * D + 32 * part);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 w = src[v];
          xs[tk * 32 + part * 8 + 2 * v] =
              make_float4(bf2f(w.x & 0xFFFFu), bf2f(w.x >> 16), bf2f(w.y & 0xFFFFu), bf2f(w.y >> 16));
          xs[tk * 32 + part * 8 + 2 * v + 1] =
              make_float4(bf2f(w.z & 0xFFFFu), bf2f(w.z >> 16), bf2f(w.w & 0xFFFFu), bf2f(w.w >> 16));
        }
      }
    }
    __syncthreads();
    for (int t = 0; t < n; ++t) {
      const float4 xi = xs[t * 32 + ri / 4];
      const float4 xj = xs[t * 32 + rj / 4];
      const float vi[4] = {xi.x, xi.y, xi.z, xi.w}, vj[4] = {xj.x, xj.y, xj.z, xj.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(vi[a], vj[b], acc[a][b]);
    }
  }
  float* out = p.gram + (((uint64_t)s * p.n_span + span) * 2 + side) * D * D;
#pragma unroll
  for (int a = 0; a < 4; ++a)
    *reinterpret_cast<float4*>(out + (ri + a) * D + rj) =
        make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
}

// Pair k of round r of the round-robin ordering of 128 indices: 127 meets r,
// and r + k meets r - k (mod 127) for k = 1..63; p < q.
__device__ __forceinline__ void jacobi_pair(int r, int k, int& p, int& q) {
  int a = r, b = 127;
  if (k > 0) {
    a = (r + k) % 127;
    b = (r - k + 127) % 127;
  }
  p = a < b ? a : b;
  q = a < b ? b : a;
}

// grid (2 sides, spans, streams), JT threads (16 waves, so that LDS latency
// is hidden inside the one workgroup a CU holds).  A and V live in LDS with
// rows of APAD floats, so that a column walk hits 32 different banks.
constexpr int JT = 1024;
__global__ __launch_bounds__(JT) void k_jacobi(RotatePlan p) {
  extern __shared__ float lds[];
  float* A = lds;                   // [128][APAD]
  float* V = lds + D * APAD;        // [128][APAD]
  float* cs = V + D * APAD;         // [64]
  float* sn = cs + 64;              // [64]
  int* P = reinterpret_cast<int*>(sn + 64);  // [64]
  int* Q = P + 64;                  // [64]
  int* rank = Q + 64;               // [128]
  const int tid = threadIdx.x;
  const int side = blockIdx.x, span = blockIdx.y, s = blockIdx.z;
  const uint64_t mat = ((uint64_t)s * p.n_span + span) * 2 + side;
  // A = the span's Gram matrix; the lower-left tile mirrors the upper-right
  const float* gp = p.gram + mat * D * D;
  for (int e = tid; e < D * D; e += JT) {
    const int i = e / D, j = e % D;
    const int src = (i >= 64 && j < 64) ? j * D + i : e;
    A[i * APAD + j] = gp[src];
    V[i * APAD + j] = i == j ? 1.0f : 0.0f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < JSWEEPS; ++sweep) {
    for (int r = 0; r < 127; ++r) {
      if (tid < 64) {
        int pp, qq;
        jacobi_pair(r, tid, pp, qq);
        const float app = A[pp * APAD + pp], aqq = A[qq * APAD + qq], apq = A[pp * APAD + qq];
        float c = 1.0f, sv = 0.0f;
        if (apq != 0.0f) {
          const float tau = (aqq - app) / (2.0f * apq);
          const float t = (tau >= 0.0f ? 1.0f : -1.0f) /
                          (fabsf(tau) + __builtin_sqrtf(__builtin_fmaf(tau, tau, 1.0f)));
          c = 1.0f / __builtin_sqrtf(__builtin_fmaf(t, t, 1.0f));
          sv = t * c;
        }
        cs[tid] = c;
        sn[tid] = sv;
        P[tid] = pp;
        Q[tid] = qq;
      }
      __syncthreads();
      // rows p and q of A (64 pairs x 128 columns)
      for (int e = tid; e < 64 * D; e += JT) {
        const int k = e / D, j = e % D;
        const float c = cs[k], sv = sn[k];
        float* rp = A + P[k] * APAD + j;
        float* rq = A + Q[k] * APAD + j;
        const float a = *rp, b = *rq;
        *rp = __builtin_fmaf(c, a, -(sv * b));
        *rq = __builtin_fmaf(sv, a, c * b);
      }
      __syncthreads();
      // columns p and q of A and of V
      for (int e = tid; e < 64 * D; e += JT) {
        const int k = e / D, i = e % D;
        const float c = cs[k], sv = sn[k];
        const int pp = P[k], qq = Q[k];
        {
          float* cp = A + i * APAD + pp;
          float* cq = A + i * APAD + qq;
          const float a = *cp, b = *cq;
          *cp = __builtin_fmaf(c, a, -(sv * b));
          *cq = __builtin_fmaf(sv, a, c * b);
        }
        {
          float* cp = V + i * APAD + pp;
          float* cq = V + i * APAD + qq;
          const float a = *cp, b = *cq;
          *cp = __builtin_fmaf(c, a, -(sv * b));
          *cq = __builtin_fmaf(sv, a, c * b);
        }
      }
      __syncthreads();
    }
  }
  // order of the eigenvalues: largest first, ties to the lower index
  if (tid < D) {
    const float d = A[tid * APAD + tid];
    int rk = 0;
    for (int j = 0; j < D; ++j) {
      const float dj = A[j * APAD + j];
      rk += (dj > d || (dj == d && j < tid)) ? 1 : 0;
    }
    rank[tid] = rk;
  }
  __syncthreads();
  float* R = p.rot + mat * D * D;
  for (int e = tid; e < D * D; e += JT) {
    const int i = e / D, o = e % D;
    R[i * D + rank[o]] = V[i * APAD + o];
  }
}

// grid (ceil(region_len / 64), 2 sides, streams), 128 threads: thread k
// holds column k of the R of the block's span in registers (a span is a
// multiple of 64 tokens, or the whole region) and writes channel k of every
// rotated vector of its 64 tokens; the tokens are staged in LDS as fp32 and
// read by all lanes at once.
__global__ __launch_bounds__(128) void k_rotate_vec(RotatePlan p) {
  __shared__ float4 xs[64 * D / 4];
  const int k = threadIdx.x;
  const int side = blockIdx.y, s = blockIdx.z;
  const int t0 = blockIdx.x * 64;
  const int n = min(64, p.region_len - t0);
  const uint16_t* X = (side ? p.V : p.K) + (uint64_t)s * p.kv_stride +
                      (uint64_t)(p.region_begin + t0) * D;
  {
    // two passes of 128 threads: token (k + 128 * pass) / 4, 32 channels each
    for (int pass = 0; pass < 2; ++pass) {
      const int e = k + 128 * pass;
      const int tk = e >> 2, part = e & 3;
      if (tk < n) {
        const uint4* src = reinterpret_cast<const uint4*>(X + (uint64_t)tk * D + 32 * part);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 w = src[v];
          xs[tk * 32 + part * 8 + 2 * v] =
              make_float4(bf2f(w.x & 0xFFFFu), bf2f(w.x >> 16), bf2f(w.y & 0xFFFFu), bf2f(w.y >> 16));
          xs[tk * 32 + part * 8 + 2 * v + 1] =
              make_float4(bf2f(w.z & 0xFFFFu), bf2f(w.z >> 16), bf2f(w.w & 0xFFFFu), bf2f(w.w >> 16));
        }
      }
    }
  }
  const int span = p.n_span > 1 ? t0 / p.span_len : 0;
  const float* R = p.rot + (((uint64_t)s * p.n_span + span) * 2 + side) * D * D;
  float rc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) rc[i] = R[i * D + k];
  __syncthreads();
  uint16_t* Y = (side ? p.YV : p.YK) + ((uint64_t)s * p.region_len + t0) * D;
  // two tokens per pass: independent chains (n is even: region_len % 16 == 0)
  for (int t = 0; t < n; t += 2) {
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i4 = 0; i4 < D / 4; ++i4) {
      const float4 x = xs[t * 32 + i4];
      const float4 y = xs[(t + 1) * 32 + i4];
      a0 = __builtin_fmaf(x.x, rc[4 * i4], a0);
      a1 = __builtin_fmaf(y.x, rc[4 * i4], a1);
      a0 = __builtin_fmaf(x.y, rc[4 * i4 + 1], a0);
      a1 = __builtin_fmaf(y.y, rc[4 * i4 + 1], a1);
      a0 = __builtin_fmaf(x.z, rc[4 * i4 + 2], a0);
      a1 = __builtin_fmaf(y.z, rc[4 * i4 + 2], a1);
      a0 = __builtin_fmaf(x.w, rc[4 * i4 + 3], a0);
      a1 = __builtin_fmaf(y.w, rc[4 * i4 + 3], a1);
    }
    Y[(uint64_t)t * D + k] = (uint16_t)f2bf(a0);
    Y[(uint64_t)(t + 1) * D + k] = (uint16_t)f2bf(a1);
  }
}

size_t jacobi_lds_bytes() { return (2 * D * APAD + 2 * 64) * sizeof(float) + (3 * 64 + D) * sizeof(int); }

hipError_t launch_rotate(const RotatePlan& p, hipStream_t st) {
  // the Jacobi matrices need more than the default 64 KB of dynamic LDS
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_jacobi),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)jacobi_lds_bytes()) != hipSuccess)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gram, dim3(3 * 2, p.n_span, p.streams), dim3(256), 0, st, p);
  hipLaunchKernelGGL(k_jacobi, dim3(2, p.n_span, p.streams), dim3(JT), jacobi_lds_bytes(), st, p);
  hipLaunchKernelGGL(k_rotate_vec, dim3((p.region_len + 63) / 64, 2, p.streams), dim3(128), 0, st,
                     p);
  return hipGetLastError();
}

}  // namespace kvc
