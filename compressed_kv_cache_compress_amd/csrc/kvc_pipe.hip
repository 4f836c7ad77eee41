// kvc_pipe.hip -- gfx950 kernels of the incremental compression pipeline:
// appending tokens to dense pages, and the switch that replaces a page with
// its final compressed segment (MosaicKV review page, Fig. 5 caption: the
// temporary form of a segment is replaced by the final one without blocking
// decode).  All three are small copies; they run on the decode stream, so
// the decode launches before and after them see the list before and after.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_internal.h"

namespace kvc {

// grid (n_new, streams), 64 threads: one token of one stream per wave.  Lanes
// 0..31 copy its K row (8 bytes each), lanes 32..63 its V row.  The wave of
// the last token also writes the page's descriptor.
__global__ __launch_bounds__(64) void k_append(AppendPlan p) {
  const int t = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int half = lane >> 5, l = lane & 31;
  const uint16_t* src = (half ? p.v : p.k) + (uint64_t)s * p.src_stride + (uint64_t)t * D;
  const uint64_t page = p.page_offset + (uint64_t)s * p.pstride;
  uint8_t* dst = p.packed + page + (uint64_t)half * p.capacity * (2 * D) +
                 (uint64_t)(p.fill + t) * (2 * D);
  reinterpret_cast<uint2*>(dst)[l] = reinterpret_cast<const uint2*>(src)[l];
  if (t == p.n_new - 1 && lane == 0) {
    kvc_seg_desc d;
    d.offset = page;
    d.n_tok = (uint16_t)(p.fill + p.n_new);
    d.n_ch = (uint16_t)D;
    d.strategy = 0;
    d.flags = (uint8_t)(0x01u | 0x02u | KVC_DESC_PAGED);
    d.seg_tokens = (uint16_t)p.capacity;
    p.desc[(uint64_t)s * p.dstride] = d;
  }
}

// grid (ceil(streams / 256)): per stream, the staged final descriptor goes
// to its event slot and the page slot is emptied, in that one kernel.
__global__ __launch_bounds__(256) void k_switch(SwitchPlan p) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= p.streams) return;
  kvc_seg_desc* row = p.list + (uint64_t)s * p.dstride;
  if (p.final_slot >= 0) row[p.final_slot] = p.staged[s];
  if (p.clear_slot >= 0) {
    kvc_seg_desc z;
    z.offset = 0;
    z.n_tok = 0;
    z.n_ch = 0;
    z.strategy = 0;
    z.flags = 0;
    z.seg_tokens = 0;
    row[p.clear_slot] = z;
  }
}

// grid (streams), 64 threads: empties list slots first .. first + count - 1.
__global__ __launch_bounds__(64) void k_clear(ClearPlan p) {
  const int s = blockIdx.x;
  uint4* row = reinterpret_cast<uint4*>(p.list + (uint64_t)s * p.dstride + p.first);
  for (int i = threadIdx.x; i < p.count; i += 64) row[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_append(const AppendPlan& p, hipStream_t st) {
  hipLaunchKernelGGL(k_append, dim3(p.n_new, p.streams), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_switch(const SwitchPlan& p, hipStream_t st) {
  hipLaunchKernelGGL(k_switch, dim3((p.streams + 255) / 256), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_clear(const ClearPlan& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_clear, dim3(p.streams), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace kvc
