// kvc_internal.h -- launch interface between the host planner (kvc_host.cpp)
// and the gfx950 kernels (kvc_compress.hip, kvc_decode.hip).  Not installed.
#pragma once
#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

#include "../../include/kvc.h"

namespace kvc {

constexpr int D = KVC_HEAD_DIM;
constexpr int BLK = 64;        // tokens per normalisation partial block
constexpr int MAX_NC = 8;      // distinct channel counts below 128 per table

// Everything the compress kernels need, resolved on the host.
struct CompressPlan {
  // shapes
  int batch, hq, hkv, G, n_ctx, region_begin, region_len, S, W, nq, nblk, n_seg, streams;
  float scale;
  uint64_t kv_stride, qw_stride, pstride, pbase;
  uint32_t dstride;
  // strategy table
  int n_strat;
  int sT[KVC_MAX_STRATEGIES], sc[KVC_MAX_STRATEGIES], su[KVC_MAX_STRATEGIES];
  uint32_t feasible_mask;
  int nc;                 // distinct channel counts < 128
  int cvals[MAX_NC];
  int t2c_alpha, t2c_gamma;
  bool scoring;           // run the window-scoring kernels
  uint32_t max_waves;     // cap on the waves of each scoring / selection kernel (0: none)
  // inputs / outputs
  const uint16_t *K, *V, *Qw;
  const uint8_t* forced;
  uint8_t* packed;
  kvc_seg_desc* desc;
  uint64_t* used;
  float* scores_out;
  float* objective;
  // workspace carve-up (device pointers)
  float *part_m, *part_z, *norm_m, *norm_iz, *scores, *rho;
  float* qf;              // window queries in fp32, [streams][G * W][128]
  float* logits;          // store_logits: [streams][G * W][n_ctx] fp32, else null
  uint32_t* masks;        // [streams][region_len][nc][2][4]
  uint32_t* keep;         // [streams][n_seg][S/32]
  // per-stream budget (budget_scope == KVC_BUDGET_STREAM)
  bool stream_budget;
  uint64_t stream_bytes;  // n_seg * budget_bytes
  uint32_t seg_bytes[KVC_MAX_STRATEGIES];
  uint32_t* keep_all;     // [streams][n_seg][n_strat][S/32]
  float* J_all;           // [streams][n_seg][n_strat]
  // SVD rotation before channel selection (kvc_rotate.hip)
  bool rotate;
  int n_span, span_len;   // rotation spans of the region (1 span: the whole region)
  float* rot;             // [streams][n_span][2][128][128] output: R_K, R_V
  float* gram;            // [streams][n_span][2][128][128] Gram matrices
  uint16_t *YK, *YV;      // [streams][region_len][128] rotated region vectors
};

struct RotatePlan {
  const uint16_t *K, *V;
  uint64_t kv_stride;
  int region_begin, region_len, streams;
  int n_span, span_len;
  float* gram;
  float* rot;
  uint16_t *YK, *YV;
};

struct DecodePlan {
  int batch, hq, hkv, G, streams, maxd, splits;
  float scale;
  const uint16_t* q;
  const uint8_t* packed;
  const kvc_seg_desc* desc;
  const uint32_t* n_desc;
  uint16_t* out;
  float* lse;
  float *part_ml, *part_acc;
  // rotated cache (null when not rotated): R_K, R_V per stream and span
  // ([streams][n_span][2][128][128]) and, in the workspace, the rotated
  // queries' bf16 parts ([batch * hq][n_span][128]) and each span's share of
  // the output; descriptor i of a stream is in span i / span_desc, and split
  // sp covers descriptors of span sp / spl
  const float* rot;
  uint16_t *qhi, *qlo;
  float* span_out;  // [batch * hq][n_span][128]: each span's rotated-back share
  int n_span, span_desc, spl;
};

// Query-aware segment selection (kvc_select.hip).
constexpr int SEL_MAXD = 8192;  // descriptors per stream the selection holds in LDS
struct SummaryPlan {
  int streams, maxd;
  const uint8_t* packed;
  const kvc_seg_desc* desc;
  const uint32_t* n_desc;
  uint16_t* summary;      // [streams][maxd][2][128]
};

struct SelectPlan {
  int streams, hkv, hq, G, maxd, keep;
  const uint16_t* q;
  const uint16_t* summary;
  const kvc_seg_desc* desc;
  const uint32_t* n_desc;
  kvc_seg_desc* out_desc;  // [streams][keep]
  uint32_t* out_n;         // [streams]
  float* score;            // [streams][maxd]
};

// Dense pages and the descriptor switch of the compression pipeline
// (kvc_pipe.hip).
struct AppendPlan {
  int streams, n_new, fill, capacity;
  uint64_t src_stride;     // elements between streams of k_new / v_new
  uint64_t page_offset;    // stream 0's page, bytes from packed
  uint64_t pstride;        // bytes between streams' pages
  uint32_t dstride;        // descriptors between streams
  const uint16_t *k, *v;
  uint8_t* packed;
  kvc_seg_desc* desc;
};

struct SwitchPlan {
  int streams;
  uint32_t dstride;        // descriptors between streams in the list
  int final_slot;          // list index that receives the staged descriptor (-1: none)
  int clear_slot;          // list index emptied (the page), -1: none
  const kvc_seg_desc* staged;  // [streams]
  kvc_seg_desc* list;
};

struct ClearPlan {
  int streams, first, count;   // empties list slots first .. first + count - 1
  uint32_t dstride;
  kvc_seg_desc* list;
};

hipError_t launch_compress(const CompressPlan& p, hipStream_t st);
hipError_t launch_rotate(const RotatePlan& p, hipStream_t st);
hipError_t launch_append(const AppendPlan& p, hipStream_t st);
hipError_t launch_switch(const SwitchPlan& p, hipStream_t st);
hipError_t launch_clear(const ClearPlan& p, hipStream_t st);
hipError_t launch_summarize(const SummaryPlan& p, hipStream_t st);
hipError_t launch_read_stream(const void* src, uint64_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_select(const SelectPlan& p, hipStream_t st);
hipError_t launch_decode(const DecodePlan& p, hipStream_t st);
// Device address of the fixed decode scratch on the current device (looked
// up once per device).
hipError_t noalloc_scratch(void** ptr);

}  // namespace kvc
