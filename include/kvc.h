/*
 * kvc.h -- C ABI of libkvc: segment-wise two-dimensional KV-cache compression
 * and decode attention over the compressed cache, for AMD Instinct MI355X
 * (gfx950).
 *
 * Method sources (review pages):
 *  - "MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache
 *    Compression" (arXiv 2607.00760): abstract (important elements of each KV
 *    vector; a compression strategy chosen per KV segment), Fig. 5 caption
 *    (segments and strategy generation), Fig. 6 caption (Stage-1 per-vector
 *    top-r elements, packed KV format, flexible KV encoding, PackedAttention).
 *  - "KARA: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
 *    Compression" (arXiv 2607.01237): "What carries the argument" (keys of a
 *    recent window scored by the attention all window queries give them;
 *    Token2Chunk), Fig. 3 caption (bidirectional: every query/key pair),
 *    free-parameter ledger (retention, window, chunk budget alpha, max chunk
 *    length gamma).
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers (HIP global memory), 16-byte
 *    aligned, owned by the caller.  bf16 tensors are uint16_t bit patterns.
 *  - Work is enqueued on the caller's `stream`; nothing is synchronised and
 *    the library never allocates or frees device memory.  All scratch space
 *    comes from the caller's workspace `ws` (size from kv_layout_query),
 *    except for kv_attend_decode_noalloc, which uses a fixed array the
 *    library holds on each device.
 *  - Arguments are validated on the host first; on any error nothing is
 *    enqueued and the call returns a negative kvc_status.  Device faults
 *    surface at the caller's next synchronisation.
 *  - Inputs must be finite; results for NaN/Inf inputs are undefined (a
 *    segment whose tokens are all dropped is never read, so its bytes may
 *    hold anything).
 *  - Calls on distinct streams with distinct buffers may run concurrently.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 1
#define KVC_HEAD_DIM 128
#define KVC_MAX_STRATEGIES 32
#define KVC_DESC_CHOOSE 0xFF      /* forced_strategy entry: let the library choose */

typedef enum {
  KVC_OK = 0,
  KVC_E_INVALID = -1,     /* malformed parameters */
  KVC_E_UNSUPPORTED = -2, /* valid but not supported (head_dim != 128, ...) */
  KVC_E_BUDGET = -3,      /* no strategy fits the per-segment byte budget */
  KVC_E_WORKSPACE = -4,   /* workspace too small */
  KVC_E_ALIGN = -5,       /* a pointer is not 16-byte aligned */
  KVC_E_HIP = -6          /* a HIP launch failed */
} kvc_status;

/* One compression strategy: keep n_tok of the segment's S tokens and, of each
 * kept K and V vector, its n_ch largest-magnitude channels.  n_tok in [0, S];
 * n_ch in {8, 16, ..., 128} when n_tok > 0 (ignored when n_tok == 0). */
typedef struct {
  uint16_t n_tok;
  uint16_t n_ch;
} kvc_strategy;

/* Shapes and knobs shared by every entry point.  Zero-initialise, set
 * struct_size = sizeof(kvc_params), then fill what the call uses.
 *
 * Streams: one stream = one (batch entry b, kv head h), index b*n_kv_heads+h.
 * K, V:  [batch][n_kv_heads][n_ctx][128] bf16 (stream stride kv_stream_stride
 *        elements).  Qwin: [batch][n_q_heads][n_win][128] bf16 (row stride
 *        qw_head_stride elements).  q heads h*G .. h*G+G-1 (G = n_q_heads /
 *        n_kv_heads) belong to kv head h.
 */
typedef struct {
  uint32_t struct_size;      /* == sizeof(kvc_params) (ABI guard) */
  uint32_t batch;
  uint32_t n_q_heads;
  uint32_t n_kv_heads;       /* divides n_q_heads; G <= 16 */
  uint32_t head_dim;         /* must be 128 */
  /* --- compression (kv_compress) --- */
  uint32_t n_ctx;            /* tokens per stream in the scoring domain; multiple of 64 */
  uint32_t region_begin;     /* first token to compress (domain position) */
  uint32_t region_len;       /* tokens to compress; multiple of seg_tokens */
  uint32_t seg_tokens;       /* S: power of two in [16, 256] */
  uint32_t n_win;            /* W: window queries per q head (>= 1) */
  const kvc_strategy* strategies; /* HOST array; index order is the tie-break order */
  uint32_t n_strategies;     /* 1 .. KVC_MAX_STRATEGIES */
  uint32_t budget_bytes;     /* per-segment cap on packed bytes */
  uint32_t t2c_alpha;        /* Token2Chunk budget (0 = plain top-T) */
  uint32_t t2c_gamma;        /* Token2Chunk max chunk length (>= 2 when alpha > 0) */
  float scale;               /* logit scale; 0 => (float)(1/sqrt(head_dim)) */
  uint64_t kv_stream_stride; /* elements between streams of K and V; 0 => n_ctx*128 */
  uint64_t qw_head_stride;   /* elements between q-head rows of Qwin; 0 => n_win*128 */
  uint64_t packed_stream_stride; /* bytes between streams' packed slots; 0 => layout.stream_capacity */
  uint64_t packed_base_offset;   /* added to every descriptor offset written */
  uint32_t desc_stream_stride;   /* descriptors between streams; 0 => region_len/seg_tokens */
  /* --- decode (kv_attend_decode) --- */
  uint32_t max_desc_per_stream;  /* descriptor stride per stream for decode; 0 => region_len/seg_tokens */
  uint32_t decode_splits;        /* split-K factor, 1 .. 65536; 0 => library choice */
  /* --- compression, continued --- */
  uint32_t budget_scope;         /* KVC_BUDGET_SEGMENT (0) or KVC_BUDGET_STREAM (1) */
  uint32_t compress_max_waves;   /* 0, or a cap on the waves each scoring and channel-
                                    selection kernel of kv_compress keeps in flight (each
                                    workgroup then walks several work units): keeps a
                                    compression that runs beside decode to a share of the
                                    GPU; results do not depend on it */
  uint32_t rotate;               /* 1: SVD rotation before channel selection (calls
                                    kv_compress_rotated / kv_attend_decode_rotated; sizes
                                    their workspaces); 0: none */
  uint32_t store_logits;         /* 1: the first scoring pass keeps every window-query
                                    logit of the domain in the compress workspace
                                    (streams x G*n_win x n_ctx fp32) and the later
                                    passes read them back instead of recomputing them;
                                    0: they recompute them.  Same results. */
  uint32_t rot_span;             /* rotate = 1: tokens per rotation span; every span of
                                    the region has its own R_K, R_V.  0 => the whole
                                    region (one R per stream).  Otherwise a multiple of
                                    seg_tokens and of 64 that divides region_len. */
} kvc_params;

/* budget_scope values.
 * KVC_BUDGET_SEGMENT: every segment's packed bytes <= budget_bytes; each
 *   segment takes its best feasible strategy.
 * KVC_BUDGET_STREAM: a stream's segments together <= n_seg * budget_bytes
 *   (MosaicKV abstract: strategies chosen per segment under the memory
 *   target; Fig. 5 caption: strategy generation).  Multiple-choice knapsack
 *   by Lagrangian relaxation: every segment takes argmax_i fl(J_i -
 *   fl(lambda * seg_bytes_i)) (ties to the lower index) for the smallest fp32
 *   lambda, by binary search over its bit patterns 0 .. 2^97, whose total
 *   fits; optimal among all assignments that use at most the bytes it uses.
 *   forced_strategy must be NULL. */
#define KVC_BUDGET_SEGMENT 0u
#define KVC_BUDGET_STREAM 1u

/* Segment descriptor (16 bytes), one per compressed segment.
 * offset: byte offset of the segment's data from the packed base pointer.
 * flags: bit0 = all S tokens kept (no index list), bit1 = all 128 channels
 * kept (no masks), bit2 = paged (KVC_DESC_PAGED: the parts below are laid out
 * for seg_tokens tokens, a power of two >= n_tok, of which the first n_tok
 * are filled, so tokens are appended in place; written by kv_append), bit7 =
 * a forced strategy was rejected (out of range or over budget) and the
 * library chose instead. */
#define KVC_DESC_PAGED 0x04u
typedef struct {
  uint64_t offset;
  uint16_t n_tok;
  uint16_t n_ch;
  uint8_t strategy;
  uint8_t flags;
  uint16_t seg_tokens;
} kvc_seg_desc;

/* Packed segment layout (MosaicKV Fig. 6 caption: packed KV format, a
 * bitmask and the kept values of every vector), parts in this order, each
 * starting 16-byte aligned:
 *   K masks  [n_tok] x 16 B   (only if n_ch < 128; channel c = byte c/8, bit c%8)
 *   K values [n_tok][n_ch] bf16, kept channels in ascending order
 *   V masks  16 * n_tok B     (only if n_ch < 128)
 *   V values 2 * n_tok * n_ch B
 *   indices  [n_tok] u16 ascending, position in the segment (only if n_tok < S),
 *            zero-padded to a multiple of 16 bytes.
 * V with n_ch < 128 is stored transposed in blocks of 8 tokens: block b
 * holds tokens 8b .. 8b+nb-1 (nb = min(8, n_tok - 8b)); its mask bits fill
 * bytes [128 b, 128 b + 16 nb) of the V masks, bit nb*(2l + h) + t (LSB
 * first) set iff token 8b+t keeps channel 64h + l (l = 0..63, h = 0, 1),
 * and its kept values fill bytes [16 n_ch b, 16 n_ch b + 2 n_ch nb) of the
 * V values in (l, h, t) order.  Same bytes as a per-token layout; decode
 * expands a channel's tokens straight into its p.v operand.  Dense V
 * (n_ch = 128) is [n_tok][128].  Decode never reads the index list. */

typedef struct {
  uint32_t seg_bytes[KVC_MAX_STRATEGIES]; /* packed bytes of one segment per strategy */
  uint32_t feasible_mask;     /* bit i: strategy i can be chosen (fits budget_bytes;
                                 stream scope: fits n_seg * budget_bytes) */
  uint32_t n_seg;             /* segments per stream in the region */
  uint64_t max_seg_bytes;     /* largest feasible seg_bytes */
  uint64_t stream_capacity;   /* bytes one stream may write, rounded up to 256:
                                 n_seg * max_seg_bytes (stream scope: at most
                                 n_seg * budget_bytes) */
  uint64_t packed_bytes_max;  /* streams * stream_capacity */
  uint64_t n_desc;            /* streams * n_seg */
  uint64_t compress_ws_bytes; /* workspace for kv_compress */
  uint64_t decode_ws_bytes;   /* workspace for kv_attend_decode */
  uint32_t decode_splits;     /* split-K factor kv_attend_decode will use */
  uint32_t needs_scoring;     /* 1 if kv_compress runs the window-scoring kernels */
} kvc_layout;

/* Host only (no device call).  Validates p and reports byte costs, feasible
 * strategies, buffer and workspace sizes: the packed bytes of one segment
 * under each strategy of the table (MosaicKV review page, Fig. 6 caption:
 * packed KV format, bitmask plus the kept bf16 elements of each vector;
 * abstract and Fig. 5 caption: a strategy per segment under the memory
 * target), which strategies fit the budget, and the split-K factor decode
 * will use.  Returns KVC_E_BUDGET when no strategy fits budget_bytes (the
 * layout is still filled), KVC_E_INVALID for malformed parameters,
 * including a decode_splits above 65536 or one that makes streams x splits
 * exceed INT_MAX (or, for a rotated decode over spans, that is no multiple of
 * the span count). */
kvc_status kv_layout_query(const kvc_params* p, kvc_layout* out);

/* Compress the region of every stream (MosaicKV: dynamic two-D compression;
 * Kara: a sliding window with Token2Chunk when t2c_alpha > 0).
 *  1. Window scores: each of the G*n_win window queries of a stream attends
 *     to all n_ctx keys (no mask); a region token's score is the sum of the
 *     probabilities it receives.  (KARA, "What carries the argument";
 *     Fig. 3 caption.)
 *  2. Per K and V vector and per channel count used by the table: the top
 *     n_ch channels by bf16 magnitude (ties to the lower channel) and the
 *     share of the vector's energy they hold.  (MosaicKV Fig. 6, Stage-1.)
 *  3. Per segment and strategy: top n_tok tokens by score (ties to the lower
 *     position) or Token2Chunk; objective = kept score mass weighted by the
 *     mean kept energy share; the best strategy within budget_bytes (ties to
 *     the lower index), unless forced.  (MosaicKV abstract, Fig. 5 caption.)
 *  4. Offsets (per-stream scan) and packing into the layout above.
 * Arguments:
 *  K, V              device, layout above.
 *  Qwin              device [batch][n_q_heads][n_win][128]; may be NULL when
 *                    layout.needs_scoring == 0 and neither scores nor
 *                    objective is requested (scoring needs n_win >= 1).
 *  forced_strategy   device [streams][n_seg] u8 or NULL; entry < n_strategies
 *                    forces that strategy if it fits the budget (else flag
 *                    bit7 and choose); KVC_DESC_CHOOSE lets the library choose.
 *  packed            device, stream s writes at packed + s*packed_stream_stride.
 *  desc              device [streams][desc_stream_stride] descriptors.
 *  used_bytes        device [streams] u64: packed bytes written per stream; may be NULL.
 *  scores            device [streams][region_len] fp32 or NULL.
 *  objective         device [streams][n_seg][n_strategies] fp32 or NULL.
 *  ws, ws_bytes      device workspace, >= layout.compress_ws_bytes.
 * Every selection output (desc, masks, index lists, packed bytes) is a
 * deterministic function of the inputs. */
kvc_status kv_compress(const kvc_params* p, const uint16_t* K, const uint16_t* V,
                       const uint16_t* Qwin, const uint8_t* forced_strategy, void* packed,
                       kvc_seg_desc* desc, uint64_t* used_bytes, float* scores, float* objective,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Compression with an SVD rotation before the channel selection (MosaicKV
 * review page: Fig. 6 caption, Stage-1 -- the rotation matrix R of the
 * current segment's K and of its V matrix from their SVD, the vectors rotated
 * before the top-r elements of each are kept; Fig. 4 -- after the rotation
 * the important elements concentrate in a few channels).  As kv_compress
 * (p->rotate = 1), and per stream and span of p->rot_span tokens (the whole
 * region when rot_span = 0):
 *  1. R_K, R_V: eigenvectors of the Gram matrices X^T X of the span's K and
 *     V vectors, ordered by eigenvalue (largest first, ties to the lower
 *     index).  Every Gram entry is one fp32 fma chain over the span's tokens
 *     in order; the eigenvectors come from 10 sweeps of cyclic Jacobi in
 *     fp32 with the round-robin pair ordering of parallel Jacobi methods
 *     (each round's 64 rotations act on disjoint index pairs, are computed
 *     from the matrix as it stands and applied to its rows, its columns and
 *     the eigenvector columns), so R is reproducible bit for bit.
 *  2. Every region vector x becomes y = R^T x with the R of its span (fp32
 *     fma chain over input channels, rounded to bf16); channel selection,
 *     the objective and the packed values use y.  Window scoring uses the
 *     original keys.
 *  rot   device [streams][n_span][2][128][128] fp32, written: R_K then R_V
 *        of each span (row i, column k = component i of the k-th
 *        eigenvector); n_span = region_len / rot_span (1 when rot_span = 0).
 * The rotations are part of what a cache stores: 128 KB per span and
 * stream in fp32, beside the packed bytes (a span of one 128-token segment
 * would need more for its two matrices than its compressed vectors may
 * occupy).  Decode the result with kv_attend_decode_rotated. */
kvc_status kv_compress_rotated(const kvc_params* p, const uint16_t* K, const uint16_t* V,
                               const uint16_t* Qwin, const uint8_t* forced_strategy, void* packed,
                               kvc_seg_desc* desc, uint64_t* used_bytes, float* scores,
                               float* objective, float* rot, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Decode attention of one query per q head over every stream's compressed
 * segments (MosaicKV Fig. 6 caption, PackedAttention): softmax over all kept
 * tokens of the stream's descriptors; a dropped channel contributes 0 to
 * q.k and to the output; fp32 accumulation.  Split-K over each stream's
 * chunks of kept tokens (the splits of a stream take equal shares of its
 * chunks to within one, a share may start and end inside a segment; lists
 * of more than 1024 descriptors are split by descriptor count), then a
 * log-sum-exp merge (when the split count is a multiple of 4, the four
 * splits of a workgroup are merged first, in the split kernel).
 *  q                 device [batch][n_q_heads][128] bf16.
 *  packed            device base that descriptor offsets index.
 *  desc              device [streams][max_desc_per_stream]; entries past a
 *                    stream's n_desc may be read but are never used.
 *  n_desc_per_stream device [streams] u32 or NULL (= max_desc_per_stream each).
 *  out               device [batch][n_q_heads][128] bf16 (RNE), overwritten;
 *                    zero for a stream with no kept token.
 *  lse               device [batch][n_q_heads] fp32 or NULL: natural-log
 *                    softmax denominator including the max (-inf if empty).
 *  ws, ws_bytes      device workspace, >= layout.decode_ws_bytes.
 * Uses batch, n_q_heads, n_kv_heads, head_dim, scale, max_desc_per_stream
 * and decode_splits of p. */
kvc_status kv_attend_decode(const kvc_params* p, const uint16_t* q, const void* packed,
                            const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                            uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): kv_attend_decode without
 * a workspace argument.  The split partials go to a fixed device array of
 * KVC_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends); the call allocates nothing.  Same kernels and results as
 * kv_attend_decode with the same p.  Returns KVC_E_WORKSPACE when the
 * workspace kv_layout_query reports for p (decode_ws_bytes) exceeds
 * KVC_NOALLOC_SCRATCH_BYTES, KVC_E_HIP when the array cannot be located on
 * the current device.  Every call on one GPU uses the same array: calls that
 * overlap on one GPU (on different streams or host threads) race and must
 * be ordered by the caller. */
#define KVC_NOALLOC_SCRATCH_BYTES (16u << 20)
kvc_status kv_attend_decode_noalloc(const kvc_params* p, const uint16_t* q, const void* packed,
                                    const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                                    uint16_t* out, float* lse, hipStream_t stream);

/* Decode over a cache compressed by kv_compress_rotated (p->rotate = 1):
 * descriptor i of a stream holds vectors rotated by the R of span
 * i / (rot_span / seg_tokens) (one span when rot_span = 0).  Each query
 * becomes q' = R_K^T q per span (fp32, passed to the score product as its
 * bf16 rounding plus the bf16 rounding of the remainder, so about 16 bits of
 * it survive), attention runs as in kv_attend_decode with the logits of a
 * token taken against its span's q', and the output is the sum over spans of
 * R_V times the span's share of the merged rotated output, in fp32, before
 * its bf16 rounding.  Every split covers descriptors of one span, so the
 * split count is a multiple of the span count (decode_splits, when given,
 * must be).  rot as written by kv_compress_rotated; lse as for
 * kv_attend_decode (the rotation does not change the logits).  Uses
 * seg_tokens and rot_span besides the fields kv_attend_decode uses;
 * workspace from kv_layout_query with p->rotate = 1. */
kvc_status kv_attend_decode_rotated(const kvc_params* p, const uint16_t* q, const void* packed,
                                    const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                                    const float* rot, uint16_t* out, float* lse, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/* Query-aware segment selection before decode attention (MosaicKV review
 * page: Fig. 6 caption, stage 2 runs during the decode stage before each
 * attention layer; Sec. 5.3, PackedAttention performs sequence compression in
 * each decode attention layer; Fig. 8, token selection rates 6.25 % and
 * 12.5 %).  Two calls: kv_summarize once per compressed cache, then
 * kv_select_segments per decode step, whose output descriptor list feeds
 * kv_attend_decode (max_desc_per_stream = keep, n_desc_per_stream = out_n).
 *
 * kv_summarize: for every descriptor, the channel-wise maximum and minimum of
 * its decoded K vectors (a dropped channel counts as 0, -0 as +0).
 *  packed, desc, n_desc_per_stream   as for kv_attend_decode.
 *  summary   device [streams][max_desc_per_stream][2][128] bf16: kmax then
 *            kmin; zeros for an empty descriptor or one past n_desc.
 * Uses batch, n_q_heads, n_kv_heads, head_dim and max_desc_per_stream of p
 * (max_desc_per_stream <= 65535).  Errors as for every entry point. */
kvc_status kv_summarize(const kvc_params* p, const void* packed, const kvc_seg_desc* desc,
                        const uint32_t* n_desc_per_stream, uint16_t* summary, hipStream_t stream);

/* kv_select_segments: for each stream, every non-empty descriptor d below
 * n_desc gets score(d) = max over the group's q heads g of the pairwise-tree
 * fp32 sum over channels 0..127 (the same tree as every selection sum) of
 * max(q_g kmax, q_g kmin) + 0 (exact bf16 products; -0 taken
 * as +0), an upper bound of q_g . k over the descriptor's kept keys (scale
 * omitted: it does not change the order).  The keep best by (score desc, index asc)
 * are written to out_desc in index order.
 *  q         device [batch][n_q_heads][128] bf16 (the decode query).
 *  summary   from kv_summarize.
 *  keep      descriptors to keep per stream, >= 1 (capped at max_desc).
 *  out_desc  device [streams][keep]; entries past out_n are left untouched.
 *  out_n     device [streams] u32: min(keep, non-empty descriptors).
 *  score     device [streams][max_desc_per_stream] fp32: each descriptor's
 *            score, -inf for an empty one or one past n_desc.
 * max_desc_per_stream <= 8192 (else KVC_E_UNSUPPORTED).  No workspace. */
kvc_status kv_select_segments(const kvc_params* p, const uint16_t* q, const uint16_t* summary,
                              const kvc_seg_desc* desc, const uint32_t* n_desc_per_stream,
                              uint32_t keep, kvc_seg_desc* out_desc, uint32_t* out_n, float* score,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Incremental, asynchronous compression (MosaicKV review page: Fig. 1 and
 * Fig. 5 captions -- compression runs asynchronously and, once a new segment
 * is complete and compressed, a switch replaces its temporary form with the
 * final one without blocking decode; Fig. 7 caption -- double compression
 * buffering.  KARA review page, free-parameter ledger -- compression period
 * delta and protected buffer U).
 *
 * Newly generated tokens are appended to dense pages (the temporary form of
 * a segment: every token, all 128 channels).  When a page completes and
 * `protect` more tokens follow it, that page is compressed by kv_compress on
 * a second stream; decode keeps reading the page until the switch writes the
 * final descriptor into its event slot and empties the page's slot, in one
 * kernel on the decode stream.
 * ------------------------------------------------------------------------ */

/* Append n_new tokens per stream to dense paged segments.
 *  k_new, v_new  device [streams][n_new][128] bf16, stream stride
 *                p->kv_stream_stride elements (0 => n_new * 128).
 *  fill          tokens already in each page; fill + n_new <= capacity.
 *  capacity      tokens a page holds: a power of two in [1, 32768].
 *  page_offset   byte offset of stream 0's page from `packed`; stream s's
 *                page is at packed + page_offset + s * p->packed_stream_stride
 *                (stride required, >= 512 * capacity, multiple of 16).
 *  page_desc     device; stream s's descriptor at page_desc[s *
 *                p->desc_stream_stride] (0 => 1) is overwritten with
 *                {page offset, n_tok = fill + n_new, n_ch = 128, strategy 0,
 *                flags = bit0 | bit1 | KVC_DESC_PAGED, seg_tokens = capacity}.
 * Page layout: K rows [capacity][128] bf16, then V rows [capacity][128] bf16;
 * token fill + i goes to row fill + i of both.  Uses batch, n_q_heads,
 * n_kv_heads, head_dim and the strides of p.  Pure copy: bit-exact. */
kvc_status kv_append(const kvc_params* p, const uint16_t* k_new, const uint16_t* v_new,
                     uint32_t n_new, uint32_t fill, uint32_t capacity, uint64_t page_offset,
                     void* packed, kvc_seg_desc* page_desc, hipStream_t stream);

/* When a finished event's final segment replaces its page. */
#define KVC_PIPE_ASYNC 0u /* at the first step after the host sees the event done (no wait) */
#define KVC_PIPE_SYNC 1u  /* compress on the decode stream inside the step that fires it,
                             switched before that step's decode: the blocking baseline */
#define KVC_PIPE_LAG 2u   /* exactly switch_lag steps after the step that fires it (the
                             decode stream waits for the event on the device if needed):
                             deterministic, for tests */

typedef struct {
  uint32_t struct_size;   /* == sizeof(kvc_pipe_config) */
  uint32_t mode;          /* KVC_PIPE_ASYNC, KVC_PIPE_SYNC or KVC_PIPE_LAG */
  uint32_t switch_lag;    /* KVC_PIPE_LAG: steps from firing to switch, 0 .. slack
                             (slack = (pages - protect/period - 1) * period) */
  uint32_t pages;         /* dense pages per stream, >= protect/period + 2 */
  uint32_t max_events;    /* event slots per stream (events beyond them: KVC_E_INVALID) */
  uint32_t prefix_desc;   /* the caller's descriptors at the head of every stream's list */
  uint32_t protect;       /* tokens that stay dense after the region: a multiple of period */
  uint32_t reserved0;
  uint64_t events_offset; /* byte offset of event slot 0 in a stream's packed slot */
  uint64_t pages_offset;  /* byte offset of page 0 in a stream's packed slot */
  uint64_t reserved[2];
} kvc_pipe_config;

typedef struct {
  uint32_t desc_per_stream;  /* prefix_desc + max_events + pages: the decode list stride */
  uint32_t period;           /* tokens per page = region tokens per event = seg_tokens */
  uint64_t event_bytes;      /* bytes of one event slot (largest feasible segment) */
  uint64_t page_bytes;       /* bytes of one page: 512 * period */
  uint64_t stream_bytes_min; /* smallest packed_stream_stride that holds both areas */
  uint64_t ws_bytes;         /* workspace: event compress + staged descriptors + decode */
  uint32_t decode_splits;    /* split-K factor of the pipeline's decode */
  uint32_t reserved;
} kvc_pipe_layout;

typedef struct {
  uint64_t steps, tokens;     /* kv_pipe_step calls; tokens appended */
  uint64_t events_fired;      /* event compressions launched */
  uint64_t events_switched;   /* of which switched into the decode list */
  uint64_t host_waits;        /* KVC_PIPE_ASYNC: a page was needed before its event was seen
                                 done, so the host waited */
  uint32_t pending;           /* fired events not yet switched */
  uint32_t reserved;
} kvc_pipe_stats;

typedef struct kvc_pipe kvc_pipe; /* opaque pipeline state (host memory) */

/* Host only.  p describes one event's compression: n_ctx = window positions
 * scored, region_begin = n_ctx - protect - seg_tokens, region_len =
 * seg_tokens, n_win, strategies, budget_bytes, t2c_*, scale as for
 * kv_compress; kv_stream_stride / qw_head_stride describe the caller's window
 * arrays; packed_stream_stride is the stride of the whole packed buffer;
 * desc_stream_stride is 0 or desc_per_stream; decode_splits as for decode. */
kvc_status kv_pipe_layout(const kvc_params* p, const kvc_pipe_config* cfg, kvc_pipe_layout* out);

/* Creates the pipeline (host state, one non-blocking stream of default
 * priority and its events) and enqueues on `stream` the clearing of every
 * stream's event and page slots in desc [streams][desc_per_stream].  The
 * caller owns packed, desc and ws (>= ws_bytes) and keeps them alive until
 * kv_pipe_destroy; the prefix descriptors are the caller's.  Every later call
 * on this pipeline passes the same `stream`. */
kvc_status kv_pipe_create(const kvc_params* p, const kvc_pipe_config* cfg, void* packed,
                          kvc_seg_desc* desc, void* ws, size_t ws_bytes, hipStream_t stream,
                          kvc_pipe** out);

/* One step: switch the events that are due, append n_new tokens per stream
 * to the current page (a step's tokens stay within one page), fire an event
 * when the pipeline's token count g reaches a multiple of period with g >=
 * protect + period (its region: tokens g - protect - period .. g - protect -
 * 1, one page), then decode q over the list (skipped when out is NULL).
 *  k_new, v_new       device [streams][n_new][128] bf16, stream stride new_stride
 *                     elements (0 => n_new * 128).
 *  win_K, win_V       device: position 0 of the scoring window (the last
 *                     p->n_ctx positions, this step's tokens included) of
 *                     every stream, stream stride p->kv_stream_stride;
 *  win_Q              device: the window's queries, [streams * G] rows of
 *                     stride p->qw_head_stride, the last n_win positions;
 *                     all three only read when an event fires (else may be
 *                     NULL) and must stay unchanged until it is switched.
 *  q, out, lse        as for kv_attend_decode over the pipeline's list.
 * Events whose region would start before the pipeline's first token are not
 * fired.  Returns KVC_E_INVALID when an event is due and the window is
 * missing or the event slots are used up; every such error leaves the
 * pipeline unchanged, with nothing enqueued.  KVC_E_HIP (a failed HIP call
 * after part of the step was enqueued) leaves it unusable: every later call
 * but kv_pipe_destroy returns KVC_E_HIP. */
kvc_status kv_pipe_step(kvc_pipe* pipe, const uint16_t* k_new, const uint16_t* v_new,
                        uint32_t n_new, uint64_t new_stride, const uint16_t* win_K,
                        const uint16_t* win_V, const uint16_t* win_Q, const uint16_t* q,
                        uint16_t* out, float* lse, hipStream_t stream);

/* Switches every fired event (the decode stream waits for each on the
 * device; the host does not block).  Afterwards the list holds every final
 * segment and only the pages that no event covers. */
kvc_status kv_pipe_drain(kvc_pipe* pipe, hipStream_t stream);

kvc_status kv_pipe_get_stats(const kvc_pipe* pipe, kvc_pipe_stats* out);

/* Waits for the pipeline's own stream, then releases its stream, events and
 * host state.  NULL is accepted. */
kvc_status kv_pipe_destroy(kvc_pipe* pipe);

/* Measurement reference, not a step of the method: reads `bytes` bytes of
 * device memory at `src` once with 16-byte loads spread over every CU.  It
 * writes nothing unless the XOR of all words read equals a fixed constant;
 * then it writes that word to *sink.  Timing it on a buffer the size of a
 * decode's reads gives the achievable HBM read bandwidth of the same box.
 * src and sink 16-byte aligned device pointers; bytes a multiple of 16,
 * > 0 (else KVC_E_INVALID / KVC_E_ALIGN). */
kvc_status kv_read_stream(const void* src, uint64_t bytes, uint32_t* sink, hipStream_t stream);

/* Static description of a status code. */
const char* kvc_status_str(kvc_status s);

/* KVC_ABI_VERSION of the loaded library. */
int kvc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
