// kvc_measure.hip -- a plain HBM read stream, the achievable-bandwidth
// reference that decode attention's bytes per second are compared with.
// Not a step of the method: it reads a buffer once with 16-byte loads spread
// over every CU and keeps a running XOR so that no load can be dropped.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_internal.h"

namespace kvc {

typedef __attribute__((ext_vector_type(4))) uint32_t rs_u32x4;

#ifndef KVC_RS_BLOCKS_PER_CU
#define KVC_RS_BLOCKS_PER_CU 2
#endif
#ifndef KVC_RS_UNROLL
#define KVC_RS_UNROLL 3
#endif
constexpr int RS_THREADS = 256;
constexpr int RS_UNROLL = KVC_RS_UNROLL;
constexpr uint32_t RS_MAGIC = 0x9E3779B9u;

// grid-stride over n16 16-byte words; each thread keeps RS_UNROLL loads in
// flight per step
__global__ __launch_bounds__(RS_THREADS) void k_read_stream(const rs_u32x4* __restrict__ src,
                                                             uint64_t n16, uint32_t* sink) {
  const uint64_t stride = (uint64_t)gridDim.x * RS_THREADS;
  uint64_t i = (uint64_t)blockIdx.x * RS_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (RS_UNROLL - 1) * stride < n16; i += RS_UNROLL * stride) {
    rs_u32x4 v[RS_UNROLL];
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const rs_u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == RS_MAGIC) sink[0] = acc;
}

hipError_t launch_read_stream(const void* src, uint64_t bytes, uint32_t* sink, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const uint64_t n16 = bytes / 16;
  const uint64_t want = (n16 + RS_THREADS - 1) / RS_THREADS;
  const uint64_t cap = (uint64_t)cus * KVC_RS_BLOCKS_PER_CU;
  const unsigned blocks = (unsigned)(want < cap ? want : cap);
  hipLaunchKernelGGL(k_read_stream, dim3(blocks), dim3(RS_THREADS), 0, st,
                     static_cast<const rs_u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace kvc
