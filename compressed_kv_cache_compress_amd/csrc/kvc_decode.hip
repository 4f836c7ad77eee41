// kvc_decode.hip -- gfx950 decode attention over compressed KV segments
// (MosaicKV review page, Fig. 6 caption: PackedAttention over the packed KV
// format).
//
// Work split: one wave per (stream, split); a split is a contiguous range of
// the stream's descriptors.  Four independent waves share a workgroup only to
// share one LDS table.  Each wave walks its descriptors in chunks of up to 16
// kept tokens (8 for masked rows wider than 88 channels, 12 for dense rows):
//   * the next chunk's K and V bytes (masks + compact values) are loaded into
//     registers while the current chunk is computed, then written to LDS;
//   * every kept K vector is expanded from (bitmask, compact bf16 values) to
//     a dense 128-channel row, one mask byte (8 channels) per lane and step,
//     one nibble (4 channels) at a time: the nibble's candidate values are
//     the 4 compact elements starting at its rank (an 8-byte window, shifted
//     by one element when the rank is odd), and one v_perm_b32 per output
//     dword places them (or zero) using a 16-entry selector table indexed by
//     the nibble; staged K rows are padded by 16 bytes so that the 16 tokens
//     of a chunk start on different LDS banks;
//   * the V side of a masked segment is stored in transposed blocks of 8
//     tokens (per channel, the tokens that keep it), so the same nibble
//     expansion over a channel's token mask yields 4 tokens of one channel:
//     exactly the B operand the p.v product takes, with no dense V tile in
//     between;
//   * q.k of the 16 tokens and p.v run on MFMA (bf16 inputs, fp32
//     accumulation); the softmax is online, in base 2, with DPP row
//     reductions.
// A second kernel merges the splits (log-sum-exp) and rounds to bf16.
//
// MFMA row mapping of q.k: q head h of the group is A-row 4*(h & 3) + (h >> 2),
// so in the 16x16 accumulator layout (lane l, item j <-> row 4*(l>>4)+j,
// column l&15) lane l's item j belongs to head 4*j+(l>>4) and to token l&15.
// p.v uses the 16-block 4x4x4 MFMA (block b = lanes 4b..4b+3; A[i][k] at lane
// 4b+i item k, B[k][j] at lane 4b+j item k, D[i][j] at lane 4b+j item i):
// head 4 jg + i x channel (64*half + lane) accumulates over 4 tokens per
// instruction, so a group of 4 heads needs 8 output registers.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <mutex>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) const uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) const uint16_t lds_u16_t;
typedef __attribute__((address_space(1))) const u32x4_t glb_u32x4_t;

// LDS byte offset of a pointer into shared memory, and back.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u32_t*)p;
}
__device__ __forceinline__ const lds_u32_t* lds_ptr(uint32_t off) {
  return (const lds_u32_t*)(uintptr_t)off;
}

constexpr int CT = 16;  // MFMA columns: at most this many kept tokens per chunk
constexpr int VB = 8;   // tokens per transposed V block of a masked segment
#ifndef KVC_DECODE_SLOTS
#define KVC_DECODE_SLOTS 3
#endif
// uint4 prefetch slots per lane and side: a chunk side (masks + values) is at
// most 64 * NPF slots of 16 bytes.
constexpr int NPF = KVC_DECODE_SLOTS;
constexpr int slots_per_token(int c) { return (c < D ? 1 : 0) + c / 8; }
// Tokens per chunk for c kept channels.  Masked rows: two V blocks (16
// tokens) while the prefetch slots hold them (c <= 88), else one (8); a
// chunk of a masked segment therefore always starts on a V block.  Dense
// rows: 12.
constexpr int chunk_tokens(int c) {
  return c >= D ? 12 : (2 * VB * slots_per_token(c) <= 64 * NPF ? 2 * VB : VB);
}
constexpr int cmax(int x, int y) { return x > y ? x : y; }
// Staging of one chunk side.  K: [masks 16 nt][rows (2c + 16) nt] (each row
// padded by 16 bytes); dense V likewise (the rows are the tile the
// transposing reads take, whole 4-token groups of them); masked V: [masks
// 16 nt][values 2 c nt] as stored.  + pad: a window may read 12 bytes past
// the last element, and an absent second V block is addressed 16 c bytes
// past the first.
constexpr int VR_STRIDE = 136;  // u16 per staged dense row (2 * 128 + 16 bytes)
constexpr int kstage_bytes() {
  int m = 0;
  for (int c = 8; c <= D; c += 8)
    m = cmax(m, chunk_tokens(c) * ((c < D ? 16 : 0) + 2 * c + 16));
  return m + 32;
}
constexpr int vstage_bytes() {
  int m = 4 * ((chunk_tokens(D) + 3) / 4) * 2 * VR_STRIDE;
  for (int c = 8; c < D; c += 8) {
    const int nt = chunk_tokens(c);
    m = cmax(m, nt * (16 + 2 * c) + 32);
    m = cmax(m, 16 * nt + 2 * c * VB + 32);
  }
  return m;
}
constexpr int KSTAGE = (kstage_bytes() + 15) / 16 * 16;
constexpr int VSTAGE = (vstage_bytes() + 15) / 16 * 16;
constexpr float RESCALE_SLACK = 8.0f;             // log2 units the running max may lag
constexpr int WAVES = 4;
constexpr int XCDS = 8;  // accelerator complex dies of the chip, one L2 each
#ifndef KVC_DECODE_MIN_BLOCKS
#define KVC_DECODE_MIN_BLOCKS 2  // workgroups per CU the register budget is sized for
#endif

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* q_lo;  // QLO: low bf16 parts of the queries (q + q_lo ~ the fp32 query)
  const uint8_t* packed;
  const kvc_seg_desc* desc;
  const uint32_t* n_desc;
  float* part_ml;
  float* part_acc;
  int hkv, hq, G, maxd, splits, items;
  // rotation spans (QLO only): descriptor i is in span i / span_desc, split
  // sp covers span sp / spl, and the queries are [row][n_span][128]
  int n_span, span_desc, spl;
  // the four waves of a workgroup hold consecutive splits of one stream
  // (splits a multiple of 4, no rotation): they merge their states and the
  // workgroup writes one partial, split index sp / 4 of splits / 4
  int wg_merge;
  float sl2;  // scale * log2(e)
};

// Per-wave LDS.  The loop is software-pipelined: while the K side of chunk
// i+1 is computed, the V side of chunk i is, so V stages and probabilities
// are double-buffered.
union VStage {
  u32x4_t v[VSTAGE / 16];
  uint16_t vt[VSTAGE / 2];
};
template <int JG>
struct WaveLds {
  u32x4_t k[KSTAGE / 16];
  VStage vs[2];                   // chunk i's V side and chunk i+1's, alternating
  uint16_t pl[2][4 * JG * CT];    // probabilities, [head][token], alternating
};

static_assert(chunk_tokens(64) == CT && chunk_tokens(88) == CT && chunk_tokens(96) == VB &&
              chunk_tokens(D) == 12, "chunk sizing");
static_assert(64 * NPF >= 12 * slots_per_token(D), "dense chunks fit the prefetch slots");


// Ordering of a wave's LDS accesses, and why the chunk loop needs no fence:
// LDS executes a wave's DS instructions in issue order, so a later read sees
// an earlier write (also from another lane) and a later write cannot overtake
// an earlier read; the compiler keeps accesses that may overlap in program
// order (the library is built with -fno-strict-aliasing because the staging
// buffers are read and written through different types).

// Selectors for a mask nibble n (channels 0..3 of the nibble): dword d holds
// the v_perm_b32 selectors of channels 2d and 2d+1, i.e. bytes (2e, 2e+1) of
// an 8-byte window of compact elements where e = kept channels of the nibble
// before this one, or 0x0C (zero byte) when the channel is dropped.
__device__ void build_lut_entry(uint32_t n, uint32_t* e) {
  for (int d = 0; d < 2; ++d) {
    uint32_t sel = 0;
    for (int h = 0; h < 2; ++h) {
      const int ch = 2 * d + h;
      uint32_t pair = 0x0C0Cu;
      if ((n >> ch) & 1u) {
        const uint32_t el = __popc(n & ((1u << ch) - 1u));
        pair = (2 * el) | ((2 * el + 1) << 8);
      }
      sel |= pair << (16 * h);
    }
    e[d] = sel;
  }
}

// Expansion of one staged token (this lane's `col`) to the dense channels
// 8*(4*kk + grp) .. +7 for kk = 0..3 (mask byte 4*kk + grp; the MFMA
// contraction order over channels is the same permutation for q, so any
// assignment of channels to k-slots works).  Two phases so that every LDS
// read of a token side is in flight at once: issue() reads the mask, the
// two 12-byte windows (low and high nibble) per byte and the two selector
// entries; finish() aligns each window to its first element and places the
// values with one v_perm_b32 per output dword.  A window is read from the
// dword holding its first element; v_alignbyte_b32 takes the element's byte
// address itself as the shift (bits 1:0, 0 or 2 since rows start on 16-byte
// boundaries).  MASKED: rows carry a 16-byte mask (c < 128); otherwise every
// channel is kept.  Tokens past the chunk read the zero mask `zrow` (every
// output zero) and row 0, so every read stays inside the staging buffer.
struct Expand {
  uint32_t a[4][3], b[4][3];  // windows of the low / high nibble
  uint32_t sa[4], sb[4];      // byte address of the first element (bits 1:0 used)
  uint2 tl[4], th[4];         // selectors of the low / high nibble
};

template <bool MASKED>
__device__ __forceinline__ void expand_issue(const uint8_t* st, int col, int grp, int nt, int c,
                                             const uint2* lut, const u32x4_t* zrow, Expand& e) {
  const bool live = col < nt;
  const int rc = live ? col : 0;
  u32x4_t ml = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  if (MASKED) ml = *(live ? reinterpret_cast<const u32x4_t*>(st + 16 * col) : zrow);
  const uint32_t row = lds_off(st) + (MASKED ? 16 * nt : 0) + (2 * c + 16) * rc;
  uint32_t pre = 0;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t mw = ml[kk];
    const uint32_t mb = (MASKED || live) ? (mw >> (8 * grp)) & 0xFFu : 0u;
    const uint32_t ra = pre + __popc(mw & ((1u << (8 * grp)) - 1u));
    const uint32_t rb = ra + __popc(mb & 0xFu);
    pre += __popc(mw);
    const uint32_t ba = row + 2 * ra, bb = row + 2 * rb;
    const lds_u32_t* wa = lds_ptr(ba & ~3u);
    const lds_u32_t* wb = lds_ptr(bb & ~3u);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      e.a[kk][i] = wa[i];
      e.b[kk][i] = wb[i];
    }
    e.sa[kk] = ba;
    e.sb[kk] = bb;
    // lut[2 n] is the selector entry of nibble n (16-byte entries)
    e.tl[kk] = lut[2 * (mb & 0xFu)];
    e.th[kk] = lut[2 * (mb >> 4)];
  }
}

__device__ __forceinline__ u32x4_t expand_finish(const Expand& e, int kk) {
  const uint32_t xa0 = __builtin_amdgcn_alignbyte(e.a[kk][1], e.a[kk][0], e.sa[kk]);
  const uint32_t xa1 = __builtin_amdgcn_alignbyte(e.a[kk][2], e.a[kk][1], e.sa[kk]);
  const uint32_t xb0 = __builtin_amdgcn_alignbyte(e.b[kk][1], e.b[kk][0], e.sb[kk]);
  const uint32_t xb1 = __builtin_amdgcn_alignbyte(e.b[kk][2], e.b[kk][1], e.sb[kk]);
  u32x4_t o;
  o[0] = __builtin_amdgcn_perm(xa1, xa0, e.tl[kk].x);
  o[1] = __builtin_amdgcn_perm(xa1, xa0, e.tl[kk].y);
  o[2] = __builtin_amdgcn_perm(xb1, xb0, e.th[kk].x);
  o[3] = __builtin_amdgcn_perm(xb1, xb0, e.th[kk].y);
  return o;
}

// The 4 x 8 dense channels of this lane's token (zero past the chunk).
template <bool MASKED>
__device__ __forceinline__ void expand_side(const uint8_t* st, int col, int grp, int nt, int c,
                                            const uint2* lut, const u32x4_t* zrow, u32x4_t* o) {
  Expand e;
  expand_issue<MASKED>(st, col, grp, nt, c, lut, zrow, e);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) o[kk] = expand_finish(e, kk);
}

// V side of a masked chunk, staged as [masks 16 nt][values 2 c nt] in
// transposed blocks of VB tokens (block bk = tokens 8 bk .. of the chunk,
// mask bytes at 128 bk, values at 16 c bk; in a block of nb tokens, bit
// nb (2 l + h) + t says token t keeps channel 64 h + l, and the values run
// in (l, h, t) order).  Lane l takes channels l (h = 0) and 64 + l (h = 1):
// its 2 nb bits of each block, an exclusive prefix of the lanes' counts for
// the rank of its first value, and per nibble of a channel's block mask (4
// tokens) one window and one v_perm_b32 per output dword -- the 4 tokens'
// elements of the channel, which is the B operand of the 4x4x4 p.v product
// for that token group as it stands.  Two phases like Expand.
struct VExpand {
  uint32_t w[4][2][3];  // [token group sg = 2 bk + n][h] windows
  uint32_t sa[4][2];    // byte address of the first element (bits 1:0 used)
  uint2 sel[4][2];
};

__device__ __forceinline__ void vexpand_issue(const uint8_t* st, int lane, int nt, int c,
                                              const uint2* lut, VExpand& e) {
  const uint32_t base = lds_off(st);
  uint32_t chm[2][2];
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const int nb = min(max(nt - VB * bk, 0), VB);  // wave-uniform
    if (nb == VB) {
      // a whole block: the lane's two channel masks are byte 0 and 1 of
      // halfword l
      const uint32_t x = *reinterpret_cast<const lds_u16_t*>(
          (uintptr_t)(base + 128u * bk + 2u * (uint32_t)lane));
      chm[bk][0] = x & 0xFFu;
      chm[bk][1] = x >> 8;
    } else {
      uint32_t x = 0u;
      if (nb > 0) {
        const uint32_t bit = 2u * (uint32_t)nb * (uint32_t)lane;
        const lds_u32_t* m = lds_ptr(base + 128u * bk + 4u * (bit >> 5));
        x = __builtin_amdgcn_alignbit(m[1], m[0], bit & 31u);
      }
      chm[bk][0] = __builtin_amdgcn_ubfe(x, 0u, (uint32_t)nb);
      chm[bk][1] = __builtin_amdgcn_ubfe(x, (uint32_t)nb, (uint32_t)nb);
    }
  }
  const uint32_t p00 = __popc(chm[0][0]), p10 = __popc(chm[1][0]);
  const uint32_t cnt = (p00 + __popc(chm[0][1])) | ((p10 + __popc(chm[1][1])) << 16);
  const uint32_t ex = wave_incl_scan_u32(cnt) - cnt;  // two 16-bit prefixes
  const uint32_t vb = base + 16u * (uint32_t)nt;
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const uint32_t r0 = bk ? ex >> 16 : ex & 0xFFFFu;
    const uint32_t blk = vb + 16u * (uint32_t)c * bk;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t m = chm[bk][h];
      const uint32_t ra = r0 + (h ? (bk ? p10 : p00) : 0u);
      const uint32_t rb = ra + __popc(m & 0xFu);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int sg = 2 * bk + n;
        const uint32_t ba = blk + 2u * (n ? rb : ra);
        const lds_u32_t* w = lds_ptr(ba & ~3u);
#pragma unroll
        for (int i = 0; i < 3; ++i) e.w[sg][h][i] = w[i];
        e.sa[sg][h] = ba;
        e.sel[sg][h] = lut[2 * (n ? m >> 4 : m & 0xFu)];
      }
    }
  }
}

__device__ __forceinline__ s16x4_t vexpand_finish(const VExpand& e, int sg, int h) {
  const uint32_t x0 = __builtin_amdgcn_alignbyte(e.w[sg][h][1], e.w[sg][h][0], e.sa[sg][h]);
  const uint32_t x1 = __builtin_amdgcn_alignbyte(e.w[sg][h][2], e.w[sg][h][1], e.sa[sg][h]);
  u32x2_t o;
  o[0] = __builtin_amdgcn_perm(x1, x0, e.sel[sg][h].x);
  o[1] = __builtin_amdgcn_perm(x1, x0, e.sel[sg][h].y);
  return __builtin_bit_cast(s16x4_t, o);
}

// One chunk to stream: K part and V part each = [masks 16*nt][values 2*c*nt]
// in global memory.  Uniform bases: the value stream of a side is addressed
// as val + 16*j for stream slot j >= nm (val already offset by -16*nm).
struct Chunk {
  const uint8_t* kmask;
  const uint8_t* kval;
  const uint8_t* vmask;
  const uint8_t* vval;
  int nt, c, nm, n16;
  uint32_t delta;  // kval - kmask = vval - vmask
  uint32_t magic;  // ceil(2^20 / (c/8)): value slot -> row by multiply-shift
  bool valid;
};

// The next chunk's bytes, one uint4 of K and one of V per slot and lane.
struct Regs {
  u32x4_t k[NPF], v[NPF];
};

template <int I>
__device__ __forceinline__ void prefetch_slot(const Chunk& ch, int lane, Regs& r) {
  // Lanes past the chunk load its last slot again, so no branch surrounds
  // the loads (a branch there makes the compiler wait for every load in
  // flight before the next one); commit skips those lanes.  The packed
  // buffer is device (global) memory: each load takes a scalar base and an
  // unsigned 32-bit lane offset, its native addressing form; in slot 0 the
  // value slots sit delta bytes past the masks.
  const int j = min(lane + 64 * I, ch.n16 - 1);
  if (I == 0) {
    const uint32_t off = 16u * (uint32_t)j + (j < ch.nm ? 0u : ch.delta);
    r.k[I] = *(glb_u32x4_t*)(ch.kmask + off);
    r.v[I] = *(glb_u32x4_t*)(ch.vmask + off);
  } else {
    const uint32_t off = 16u * (uint32_t)j;
    r.k[I] = *(glb_u32x4_t*)(ch.kval + off);
    r.v[I] = *(glb_u32x4_t*)(ch.vval + off);
  }
}

__device__ __forceinline__ void prefetch(const Chunk& ch, int lane, Regs& r) {
  if (!ch.valid) return;
  prefetch_slot<0>(ch, lane, r);
  prefetch_slot<1>(ch, lane, r);
  prefetch_slot<2>(ch, lane, r);
  if constexpr (NPF > 3) prefetch_slot<3>(ch, lane, r);
}

// Slot j of the [masks | values] stream of the K side goes to LDS slot j
// (masks) or, for value slot v = j - nm, to nm + v + v / (c/8): one 16-byte
// pad per row.  The V side of a masked chunk is staged as stored (slot j);
// dense V rows are padded like K rows.
template <int I>
__device__ __forceinline__ void commit_slot(const Chunk& ch, int lane, const Regs& r, u32x4_t* sk,
                                            u32x4_t* sv) {
  const int j = lane + 64 * I;
  if (j < ch.n16) {
    const uint32_t v = (uint32_t)(j - ch.nm);
    const int dst = (I == 0 && j < ch.nm) ? j : j + (int)(__umul24(v, ch.magic) >> 20);
    sk[dst] = r.k[I];
    sv[ch.nm ? j : dst] = r.v[I];
  }
}

__device__ __forceinline__ void commit(const Chunk& ch, int lane, const Regs& r, u32x4_t* sk,
                                       u32x4_t* sv) {
  commit_slot<0>(ch, lane, r, sk, sv);
  commit_slot<1>(ch, lane, r, sk, sv);
  commit_slot<2>(ch, lane, r, sk, sv);
  if constexpr (NPF > 3) commit_slot<3>(ch, lane, r, sk, sv);
}

// Descriptor cursor of one wave.  Descriptors are fetched 64 at a time, one
// per lane, and read back wave-uniformly with readlane, so walking them costs
// no memory round trip per segment.  The current segment's geometry is kept
// in (scalar) registers so that chunks after the first of a segment only
// advance offsets.
struct Cursor {
  const kvc_seg_desc* dl;
  const uint8_t* packed;
  int di, d1, base;         // next descriptor, end, first descriptor held in the lanes
  // a split may start and end inside a segment: descriptor dfirst is walked
  // from token tfirst, descriptor dlast up to token tlast (-1: none)
  int dfirst, tfirst, dlast, tlast;
  uint32_t w0, w1, w2;      // this lane's descriptor (base + lane): offset lo/hi, n_tok|n_ch<<16
  uint32_t w3;              // its chunk geometry: tokens per chunk | row magic << 5 | page << 26
  // current segment
  const uint8_t *kmask, *kval, *vmask, *vval;  // at token 0
  int T, c, t0, ct;
  uint32_t magic;
};

// ceil(2^20 / k): value slot v of a stage with k slots per row is in row
// (v * magic) >> 20 for v < 16 * k.
constexpr uint32_t row_magic(int k) { return (1048576u + (uint32_t)k - 1u) / (uint32_t)k; }
// The fields of the packed chunk geometry hold every value they take: tokens
// per chunk in 5 bits (a chunk of 0 tokens would never advance and would
// address slot -1), the row magic in 21, log2(seg_tokens) + 1 <= 17 in 6.
constexpr bool geo_fields_fit() {
  for (int c = 8; c <= D; c += 8)
    if (chunk_tokens(c) < 1 || chunk_tokens(c) > 31 || row_magic(c >> 3) > 0x1FFFFFu) return false;
  return true;
}
static_assert(geo_fields_fit(), "chunk geometry fields");

// Chunk geometry of a descriptor (words 2 and 3), computed once per 64
// descriptors so that the chunk loop reads it with readlane instead of a
// memory lookup; a paged descriptor (flags bit2) also carries
// log2(seg_tokens) + 1, the token count its parts are laid out for.
__device__ __forceinline__ uint32_t desc_geometry(uint32_t d2, uint32_t d3) {
  const int c = (int)(d2 >> 16) & ~7;
  const int cc = c < 8 ? 8 : (c > D ? D : c);
  const uint32_t cap = d3 >> 16;
  const uint32_t page = ((d3 >> 8) & KVC_DESC_PAGED) && cap ? 32u - __clz(cap) : 0u;
  return (uint32_t)chunk_tokens(cc) | (row_magic(cc >> 3) << 5) | (page << 26);
}

__device__ __forceinline__ void fetch_descs(Cursor& cu, int lane) {
  cu.base = cu.di;
  const int i = min(cu.di + lane, cu.d1 - 1);
  const u32x4_t d = *reinterpret_cast<const u32x4_t*>(cu.dl + i);
  cu.w0 = d[0];
  cu.w1 = d[1];
  cu.w2 = d[2];
  cu.w3 = desc_geometry(d[2], d[3]);
}

// Chunks of descriptor i of a stream's list (0 past nd): ceil(T / ct) with
// ct = 8, 12 or 16 tokens per chunk.  T / ct is a multiple of 1/ct >= 1/16 apart
// from the next integer, so adding 31/32 to the product with the approximate
// reciprocal and truncating gives the exact ceiling.  (The count only
// balances the splits; any count gives the same results.)
// Chunks of a descriptor from its word 2 (n_tok | n_ch << 16), and its
// tokens per chunk.
__device__ __forceinline__ uint32_t desc_chunks(uint32_t tc, uint32_t& ct) {
  const uint32_t T = tc & 0xFFFFu;
  const int c = (int)(tc >> 16) & ~7;
  ct = (uint32_t)chunk_tokens(c < 8 ? 8 : (c > D ? D : c));
  return (uint32_t)((float)T * __builtin_amdgcn_rcpf((float)ct) + 0.96875f);
}

// Chunk range of split sp of a stream with nd descriptors: with W the
// stream's chunks, chunks floor(sp W / splits) .. floor((sp + 1) W / splits)
// - 1 in walking order, so that every split of a stream takes the same
// number of chunks to within one, starting and ending inside a segment
// where the share falls there.  A segment is 2 to 22 chunks here; whole
// segments per split left the busiest of 24 waves 20 % (1024 segments of 2
// and 4 chunks) to 25 % (128 such segments) above the mean.  Lane l holds
// word 2 of descriptors per l .. per l + per - 1 (tc[k]; per <= PER), one
// wave scan gives each lane the chunks before its first, and the lanes that
// hold the first and the last chunk of the share are found by ballot.
template <int PER>
__device__ __forceinline__ void balanced_core(const uint32_t (&tc)[PER], int per, int nd,
                                              int splits, int sp, int lane, Cursor& cu) {
  uint32_t w[PER], ct[PER], tot = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const uint32_t x = desc_chunks(tc[k], ct[k]);
    w[k] = k < per && lane * per + k < nd ? x : 0u;
    tot += w[k];
  }
  const uint32_t inc = wave_incl_scan_u32(tot);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  const uint32_t c0 = (uint32_t)(((uint64_t)sp * total) / (uint32_t)splits);
  const uint32_t c1 = (uint32_t)(((uint64_t)(sp + 1) * total) / (uint32_t)splits);
  cu.di = cu.d1 = 0;
  if (c0 >= c1) return;  // no chunks for this split
  // the descriptors holding chunk c0 and chunk c1 - 1 (each non-empty, so
  // one lane and slot each), and the tokens before / through them
  uint32_t e = inc - tot;
  int f0 = -1, f1 = -1;
  uint32_t t0 = 0, t1 = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = lane * per + k;
    const bool in0 = w[k] > 0u && e <= c0 && c0 < e + w[k];
    const bool in1 = w[k] > 0u && e < c1 && c1 <= e + w[k];
    if (in0) {
      f0 = i;
      t0 = (c0 - e) * ct[k];
    }
    if (in1) {
      f1 = i;
      t1 = (c1 - e) * ct[k];
    }
    e += w[k];
  }
  const uint64_t b0 = __ballot(f0 >= 0), b1 = __ballot(f1 >= 0);
  if (b0 == 0u || b1 == 0u) return;
  const int l0 = (int)__builtin_ctzll(b0), l1 = (int)__builtin_ctzll(b1);
  cu.di = __builtin_amdgcn_readlane(f0, l0);
  cu.tfirst = __builtin_amdgcn_readlane((int)t0, l0);
  cu.dlast = __builtin_amdgcn_readlane(f1, l1);
  cu.tlast = __builtin_amdgcn_readlane((int)t1, l1);
  cu.dfirst = cu.di;
  cu.d1 = cu.dlast + 1;
}

// Descriptor range of split sp, with the cursor's first 64 descriptors in
// place when it returns true.  Lists of at most 256 descriptors (by capacity
// maxd): every lane loads its up to four whole descriptors in the round trip
// that also brings the query and the list length (the layout follows maxd,
// not nd, so the loads wait for nothing), the chunk share is taken from
// their word 2, and lane j then takes descriptor di + j from the lane that
// holds it by cross-lane permutes -- one memory round trip where counting,
// then fetching took two more.  Up to 1024 descriptors: word 2 of each is
// loaded for the share and the cursor fetches its descriptors after.
// Longer lists take an equal share of the descriptors.
__device__ __forceinline__ bool split_range(int nd, int maxd, int splits, int sp, int lane,
                                            Cursor& cu) {
  cu.dfirst = cu.dlast = -1;
  cu.di = (int)(((int64_t)sp * nd) / splits);
  cu.d1 = (int)(((int64_t)(sp + 1) * nd) / splits);
  if (maxd <= 256) {
    constexpr int PER = 4;
    const int per = (maxd + 63) >> 6;
    u32x4_t dd[PER];
    uint32_t tc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      // unconditional loads of clamped indices go out together
      dd[k] = *reinterpret_cast<const u32x4_t*>(cu.dl + min(lane * per + k, maxd - 1));
      tc[k] = dd[k][2];
    }
    if (nd <= 0) return false;
    balanced_core<PER>(tc, per, nd, splits, sp, lane, cu);
    if (cu.di >= cu.d1) return false;
    // lane j takes descriptor i = di + j (clamped to the range), held by lane
    // i / per in slot i % per
    const int i = min(cu.di + lane, cu.d1 - 1);
    const int src = i / per, slot = i - src * per;
    uint32_t g[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < PER; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)dd[k][q]);
        g[q] = slot == k ? x : g[q];
      }
    cu.base = cu.di;
    cu.w0 = g[0];
    cu.w1 = g[1];
    cu.w2 = g[2];
    cu.w3 = desc_geometry(g[2], g[3]);
    return true;
  }
  if (nd <= 0 || nd > 1024) return false;
  constexpr int PER = 16;
  const int per = (nd + 63) >> 6;
  uint32_t tc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k)
    tc[k] = reinterpret_cast<const uint32_t*>(cu.dl + min(lane * per + k, nd - 1))[2];
  balanced_core<PER>(tc, per, nd, splits, sp, lane, cu);
  return false;
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Advances to the next non-empty chunk; returns its description.
__device__ __forceinline__ Chunk next_chunk(Cursor& cu, int lane) {
  Chunk ch;
  ch.valid = false;
  if (cu.t0 >= cu.T) {
    // next non-empty descriptor
    cu.T = 0;
    while (cu.di < cu.d1) {
      if (cu.di - cu.base >= 64) fetch_descs(cu, lane);
      const int sl = cu.di - cu.base;
      const uint32_t tc = __builtin_amdgcn_readlane(cu.w2, sl);
      const int T = (int)(tc & 0xFFFFu);
      // tokens [tb, te) of this segment belong to the split
      const int tb = cu.di == cu.dfirst ? cu.tfirst : 0;
      const int te = cu.di == cu.dlast ? min(T, cu.tlast) : T;
      ++cu.di;
      if (te > tb) {
        const uint32_t lo = __builtin_amdgcn_readlane(cu.w0, sl);
        const uint32_t hi = __builtin_amdgcn_readlane(cu.w1, sl);
        const uint32_t geo = __builtin_amdgcn_readlane(cu.w3, sl);
        const int c = (int)(tc >> 16);
        cu.ct = (int)(geo & 31u);
        cu.magic = (geo >> 5) & 0x1FFFFFu;
        const uint32_t page = geo >> 26;
        const uint32_t TL = page ? 1u << (page - 1u) : (uint32_t)T;  // tokens the parts are sized for
        const uint32_t mb = c < D ? 16u * TL : 0u;
        const uint8_t* base = cu.packed + (((uint64_t)hi << 32) | lo);
        cu.kmask = base;
        cu.kval = base + mb;
        cu.vmask = base + mb + 2u * TL * c;
        cu.vval = base + 2 * mb + 2u * TL * c;
        cu.T = te;
        cu.c = c;
        cu.t0 = tb;
        break;
      }
    }
    if (cu.T == 0) return ch;
  }
  const int c = cu.c, t0 = cu.t0, T = cu.T;
  const int ct = cu.ct;
  const int nt = min(ct, T - t0);
  const int nm = c < D ? nt : 0;
  // every field is wave-uniform; readfirstlane keeps them in scalar
  // registers, so loads take a scalar base and a 32-bit lane offset
  ch.kmask = uniform_ptr(cu.kmask + 16 * t0);
  ch.vmask = uniform_ptr(cu.vmask + 16 * t0);
  ch.kval = uniform_ptr(cu.kval + 2 * c * t0 - 16 * nm);
  ch.vval = uniform_ptr(cu.vval + 2 * c * t0 - 16 * nm);
  ch.delta = __builtin_amdgcn_readfirstlane((uint32_t)(ch.kval - ch.kmask));
  ch.nt = __builtin_amdgcn_readfirstlane(nt);
  ch.c = __builtin_amdgcn_readfirstlane(c);
  ch.nm = __builtin_amdgcn_readfirstlane(nm);
  ch.n16 = __builtin_amdgcn_readfirstlane(nm + (2 * c * nt) / 16);
  ch.magic = __builtin_amdgcn_readfirstlane(cu.magic);
  ch.valid = true;
  cu.t0 = t0 + ct;
  return ch;
}

// QLO: the queries come as two bf16 parts (a rotated query in fp32 split
// into its bf16 rounding and the rounded remainder); q.k is then the sum of
// two MFMA products, so the query keeps about 16 bits of precision.  For
// groups of up to 4 heads the low part of head h takes the otherwise empty
// A-row 4h + 1, so its product lands in accumulator item 1 of the lanes that
// hold head h in item 0: no extra MFMA and no extra registers.  Larger
// groups run a second set of MFMAs.
template <int JG, bool QLO>
__global__ __launch_bounds__(256, JG == 1 ? KVC_DECODE_MIN_BLOCKS : 2) void k_decode_split(DecodeArgs a) {
  // selector table, one 16-byte entry per nibble (its first 8 bytes used):
  // the entry of a high nibble is then at byte offset (mask byte & 0xF0)
  __shared__ uint4 lut4[16];
  const uint2* lut = reinterpret_cast<const uint2*>(lut4);
  __shared__ u32x4_t zrow[1];
  __shared__ WaveLds<JG> wl[WAVES];
  const int tid = threadIdx.x;
  static_assert(64 * WAVES == 256, "one selector entry per thread");
  if (tid < 16) {
    uint32_t lo[2];
    build_lut_entry((uint32_t)tid, lo);
    lut4[tid] = make_uint4(lo[0], lo[1], 0u, 0u);
    if (tid == 0) zrow[0] = u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6;
  // Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b mod
  // 8), and each XCD has an L2 of its own.  Renumbered so that consecutive
  // work items, the splits of one stream, run on one XCD: the stream's
  // query and descriptor list, read by every one of its splits, then come
  // from HBM once per stream rather than once per XCD.  A permutation of the
  // workgroups whenever their count is a multiple of 8 (else the identity).
  const int nb = (int)gridDim.x;
  const int bx = (nb % XCDS == 0) ? (int)(blockIdx.x % XCDS) * (nb / XCDS) + (int)(blockIdx.x / XCDS)
                                   : (int)blockIdx.x;
  // wave-uniform (the compiler cannot tell that tid >> 6 is), so the
  // descriptor walk and the chunk addresses live in scalar registers
  const int item = __builtin_amdgcn_readfirstlane(bx * WAVES + wv);
  if (item >= a.items) return;
  const int s = item / a.splits, sp = item - s * a.splits;
  const int grp = lane >> 4, col = lane & 15;
  const int b = s / a.hkv, h = s - b * a.hkv;
  // rotation span of this split (QLO with spans): its queries are rotated by
  // the span's R_K
  const int span = (QLO && a.span_desc) ? sp / a.spl : 0;
  const uint64_t qrow_mul = QLO ? (uint64_t)a.n_span : 1u;
  WaveLds<JG>& L = wl[wv];
  for (int i = lane; i < 2 * 4 * JG * CT; i += 64) (&L.pl[0][0])[i] = 0;

  // A operand of the score MFMA: row col holds head hh (zero if none); with
  // QLO and JG == 1, row 4h + 1 holds the low part of head h
  constexpr bool LO_ROWS = QLO && JG == 1;
  const bool lo_row = LO_ROWS && (col & 3) == 1 && (col >> 2) < a.G;
  const int hh = lo_row ? (col >> 2) : 4 * (col & 3) + (col >> 2);
  const bool hh_ok = lo_row || hh < a.G;
  const uint16_t* qh = (lo_row ? a.q_lo : a.q) +
                       ((uint64_t)(b * a.hq + h * a.G + (hh_ok ? hh : 0)) * qrow_mul + span) * D;
  bf16x8_t qa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (hh_ok) v = *reinterpret_cast<const u32x4_t*>(qh + 8 * (4 * kk + grp));
    qa[kk] = __builtin_bit_cast(bf16x8_t, v);
  }
  bf16x8_t qlo[QLO && !LO_ROWS ? 4 : 1];
  if constexpr (QLO && !LO_ROWS) {
    const uint16_t* ql =
        a.q_lo + ((uint64_t)(b * a.hq + h * a.G + (hh_ok ? hh : 0)) * qrow_mul + span) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (hh_ok) v = *reinterpret_cast<const u32x4_t*>(ql + 8 * (4 * kk + grp));
      qlo[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // O4[half][jg] item i = head 4 jg + i, channel 64 half + lane (4x4x4 MFMA)
  f32x4_t O4[2][JG];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int jg = 0; jg < JG; ++jg) O4[hf][jg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[JG], l_run[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
  }

  const int nd = a.n_desc ? min((int)a.n_desc[s], a.maxd) : a.maxd;
  Cursor cu;
  cu.dl = a.desc + (uint64_t)s * a.maxd;
  cu.packed = a.packed;
  bool placed = false;
  if (QLO && a.span_desc) {
    // a share of the span's chunks: the span's descriptors are a list of
    // their own (the cursor's base moves to its first)
    const int s0 = span * a.span_desc;
    const int n = max(0, min(nd, s0 + a.span_desc) - s0);
    const int cap = min(a.span_desc, a.maxd - s0);
    const int sub = sp - span * a.spl;
    cu.dl += s0;
    placed = split_range(n, cap, a.spl, sub, lane, cu);
  } else {
    placed = split_range(nd, a.maxd, a.splits, sp, lane, cu);
  }
  cu.T = 0;
  cu.c = 0;
  cu.t0 = 0;
  if (cu.di < cu.d1 && !placed) fetch_descs(cu, lane);

  const uint8_t* sk8 = reinterpret_cast<const uint8_t*>(L.k);

  // K side of a chunk staged in L.k: scores, online-softmax state, and the
  // probabilities into L.pl[pb].  The running max of a head moves only when
  // some score exceeds it by RESCALE_SLACK (so p <= 2^RESCALE_SLACK); the
  // accumulator rescale factor of each head is returned in alpha (1 = none)
  // and applied by the caller once the previous chunk's p.v is in.  Each lane
  // keeps its own part of the denominator; the parts are summed at the end.
  auto k_side = [&](const Chunk& ch, int pb, float* alpha) -> bool {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
    {
      u32x4_t kb[4];
      if (ch.c == D) {
        // dense rows need no expansion: 16 aligned bytes of the staged row
        // (stride 2*128 + 16 bytes) per MFMA step; tokens past the chunk are 0
        const bool live = col < ch.nt;
        const u32x4_t* r = reinterpret_cast<const u32x4_t*>(sk8 + (2 * D + 16) * (live ? col : 0));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4_t z = {0u, 0u, 0u, 0u};
          kb[kk] = live ? r[4 * kk + grp] : z;
        }
      } else {
        expand_side<true>(sk8, col, grp, ch.nt, ch.c, lut, zrow, kb);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8_t, kb[kk]),
                                                       sacc, 0, 0, 0);
      if constexpr (QLO && !LO_ROWS) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo[kk],
                                                         __builtin_bit_cast(bf16x8_t, kb[kk]), sacc,
                                                         0, 0, 0);
      }
    }
    bool resc = false;
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      const int hd = 4 * j + grp;
      const bool ok = col < ch.nt && hd < a.G;
      const float sj = LO_ROWS ? sacc[0] + sacc[1] : sacc[j];  // high + low query part
      const float x = ok ? sj * a.sl2 : -INFINITY;
      alpha[j] = 1.0f;
      if (__builtin_amdgcn_ballot_w64(x > m_run[j] + RESCALE_SLACK)) {
        const float cm = row16_max(x);
        const float mo = m_run[j];
        const float mn = (cm > mo + RESCALE_SLACK) ? cm : mo;
        alpha[j] = (mn == mo) ? 1.0f : __builtin_amdgcn_exp2f(mo - mn);
        l_run[j] *= alpha[j];
        m_run[j] = mn;
        resc = true;
      }
      const float p = (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x - m_run[j]);
      l_run[j] += p;
      if (hd < a.G) L.pl[pb][hd * CT + col] = __builtin_bit_cast(uint16_t, (__bf16)p);  // RNE
    }
    return resc;
  };
  // V side of a chunk staged in L.vs[vb]: O += P V with the probabilities
  // in L.pl[vb], one 4x4x4 product per token group of 4, channel half and
  // group of 4 heads.  Its B operand (4 tokens of the lane's channel) comes
  // from the transposed-block expansion (masked rows) or from the staged
  // dense rows through ds_read_b64_tr_b16: within each 16-lane group,
  // element r of lane i is element (i & 3) of the 8 bytes read by lane
  // 4r + (i >> 2), so lane l reads row 4 sg + ((l & 15) >> 2), channels
  // 64 half + 16 (l >> 4) + 4 (l & 3).  Token groups past the chunk are
  // skipped.
  auto v_side = [&](const Chunk& ch, int vb) {
    VStage& S = L.vs[vb];
    const int nsg = (ch.nt + 3) >> 2;
    s16x4_t bop[4][2];
    if (ch.c == D) {
      static_assert(2 * VR_STRIDE == 2 * D + 16, "dense staged rows are the tile rows");
      // rows nt .. 4 nsg - 1 may hold older data (their probabilities are 0,
      // but 0 * NaN is NaN)
      const int nz = (4 * nsg - ch.nt) * (VR_STRIDE / 8);
      for (int i = lane; i < nz; i += 64) {
        const u32x4_t z = {0u, 0u, 0u, 0u};
        S.v[ch.nt * (VR_STRIDE / 8) + i] = z;
      }
      const int trow = (lane & 15) >> 2, tcol = 16 * (lane >> 4) + 4 * (lane & 3);
#pragma unroll
      for (int sg = 0; sg < CT / 4; ++sg) {
        if (sg < nsg) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const uint16_t* src = S.vt + (4 * sg + trow) * VR_STRIDE + 64 * hf + tcol;
            bop[sg][hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)src);
          }
        }
      }
    } else {
      VExpand e;
      vexpand_issue(reinterpret_cast<const uint8_t*>(S.v), lane, ch.nt, ch.c, lut, e);
#pragma unroll
      for (int sg = 0; sg < CT / 4; ++sg)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) bop[sg][hf] = vexpand_finish(e, sg, hf);
    }
#pragma unroll
    for (int sg = 0; sg < CT / 4; ++sg) {
      if (sg < nsg) {
#pragma unroll
        for (int jg = 0; jg < JG; ++jg) {
          // A: head 4 jg + (lane & 3) x tokens 4sg..4sg+3
          const s16x4_t pa =
              *reinterpret_cast<const s16x4_t*>(L.pl[vb] + (4 * jg + (lane & 3)) * CT + 4 * sg);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            O4[hf][jg] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pa, bop[sg][hf], O4[hf][jg], 0, 0, 0);
        }
      }
    }
  };
  // alpha[j] of the lanes of row i (lane 16 i) belongs to head 4 j + i
  auto rescale = [&](const float* alpha) {
#pragma unroll
    for (int jg = 0; jg < JG; ++jg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[jg]), 16 * i));
        O4[0][jg][i] *= ai;
        O4[1][jg][i] *= ai;
      }
  };

  static_assert((NPF == 3 || NPF == 4) && CT == 16, "prefetch slots are unrolled by hand; masks fit slot 0");
  Regs rg;
  Chunk cur = next_chunk(cu, lane);
  if (cur.valid) {
    prefetch(cur, lane, rg);
    commit(cur, lane, rg, L.k, L.vs[0].v);
    Chunk nxt = next_chunk(cu, lane);
    prefetch(nxt, lane, rg);
    float alpha[JG];
    if (k_side(cur, 0, alpha)) rescale(alpha);
    int vb = 0;
    // iteration: stage chunk i+1, load chunk i+2, K side of i+1, V side of i.
    // Wave priorities order the work of the waves sharing a SIMD by how soon
    // other work waits for it: the commit first (its loads have landed, and
    // staging them frees the prefetch registers for the next loads), then the
    // walk and those loads, then the K side (its probabilities feed the next
    // V side), and the V side last, which only adds into this wave's
    // accumulators and may trail.  The arbiter then keeps the chunk chain of
    // each wave moving and fills the gaps with V work.
    constexpr int PRIO_COMMIT = 3, PRIO_LOAD = 2, PRIO_K = 1, PRIO_V = 0;
    while (nxt.valid) {
      __builtin_amdgcn_s_setprio(PRIO_COMMIT);
      commit(nxt, lane, rg, L.k, L.vs[vb ^ 1].v);
      __builtin_amdgcn_s_setprio(PRIO_LOAD);
      const Chunk far = next_chunk(cu, lane);
      prefetch(far, lane, rg);
      __builtin_amdgcn_s_setprio(PRIO_K);
      const bool resc = k_side(nxt, vb ^ 1, alpha);
      __builtin_amdgcn_s_setprio(PRIO_V);
      v_side(cur, vb);
      if (resc) rescale(alpha);
      cur = nxt;
      nxt = far;
      vb ^= 1;
    }
    v_side(cur, vb);
  }

  // partial state of this split
#pragma unroll
  for (int j = 0; j < JG; ++j) l_run[j] = row16_sum(l_run[j]);
  if (!QLO && a.wg_merge) {
    // Each wave writes its state into its own (now idle) staging, the
    // workgroup waits for all four, then wave wv merges the heads hd with
    // hd % 4 == wv over the four waves in order (log-sum-exp, base 2) and
    // writes them as one partial.  No wave of such a launch returned early:
    // its wave count is a multiple of 4.
    constexpr int NH = 4 * JG;  // head slots per wave
    float* mine = reinterpret_cast<float*>(&L);  // [NH][2] (m, l), then [NH][D] acc
#pragma unroll
    for (int j = 0; j < JG; ++j)
      if (col == 0) {
        mine[2 * (4 * j + grp)] = m_run[j];
        mine[2 * (4 * j + grp) + 1] = l_run[j];
      }
#pragma unroll
    for (int jg = 0; jg < JG; ++jg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mine[2 * NH + (4 * jg + i) * D + lane] = O4[0][jg][i];
        mine[2 * NH + (4 * jg + i) * D + 64 + lane] = O4[1][jg][i];
      }
    static_assert((2 + D) * NH * 4 <= sizeof(WaveLds<JG>), "wave states fit the staging");
    __syncthreads();
    const int splits4 = a.splits >> 2, sp4 = sp >> 2;
#pragma unroll
    for (int jg = 0; jg < JG; ++jg) {
      const int hd = 4 * jg + wv;
      if (hd >= a.G) continue;
      float mu[WAVES], M = -INFINITY;
#pragma unroll
      for (int u = 0; u < WAVES; ++u) {
        mu[u] = reinterpret_cast<const float*>(&wl[u])[2 * hd];
        M = fmaxf(M, mu[u]);
      }
      float Ls = 0.0f, a0 = 0.0f, a1 = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < WAVES; ++u) {
          const float* st = reinterpret_cast<const float*>(&wl[u]);
          const float w = mu[u] == -INFINITY ? 0.0f : exp2f(mu[u] - M);
          Ls += st[2 * hd + 1] * w;
          a0 += st[2 * NH + hd * D + lane] * w;
          a1 += st[2 * NH + hd * D + 64 + lane] * w;
        }
      }
      const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + hd) * splits4 + sp4;
      if (lane == 0) {
        a.part_ml[2 * pi] = M;
        a.part_ml[2 * pi + 1] = Ls;
      }
      a.part_acc[pi * D + lane] = a0;
      a.part_acc[pi * D + 64 + lane] = a1;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    const int hd = 4 * j + grp;
    if (hd < a.G && col == 0) {
      const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + hd) * a.splits + sp;
      a.part_ml[2 * pi] = m_run[j];
      a.part_ml[2 * pi + 1] = l_run[j];
    }
  }
#pragma unroll
  for (int jg = 0; jg < JG; ++jg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hd = 4 * jg + i;
      if (hd < a.G) {
        const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + hd) * a.splits + sp;
        a.part_acc[pi * D + lane] = O4[0][jg][i];
        a.part_acc[pi * D + 64 + lane] = O4[1][jg][i];
      }
    }
}

// Log-sum-exp merge of the splits of one (b, q head) row, for a slice of
// RC channels: thread (g, c) folds splits g, g + RG, ... of channel
// c0 + c into a group state (m, l, acc), then the RG group states are merged
// through LDS by the threads of group 0.  Many groups keep the per-thread
// chain of dependent loads short when there are many splits (RG 32 x RC 32
// above 32 splits, RG 8 x RC 128 above 8, one group of 128 threads
// otherwise, where idle threads would cost more than the short chains).  Returns acc / l for channel
// c0 + c and the row's log-sum-exp (base 2); false when every split was
// empty (the same answer on every thread of the block).
template <int RG, int RC>
__device__ __forceinline__ bool merge_splits(const float* __restrict__ ml,
                                             const float* __restrict__ acc_row, int splits,
                                             int c0, float* o, float* lse2) {
  __shared__ float gm[RG], gl[RG], gacc[RG][RC + 1];
  const int c = threadIdx.x % RC, g = threadIdx.x / RC;
  float M = -INFINITY;
  float L = 0.0f, acc = 0.0f;
  constexpr int NPT = RG == 1 ? 8 : 4;  // splits per thread loaded at once
  if (splits <= NPT * RG) {
    // every load of the thread in one round trip (clamped indices; a split
    // past the end weighs 0, which adds nothing to the sums)
    float mv[NPT], lv[NPT], av[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int sp = min(g + RG * k, splits - 1);
      mv[k] = ml[2 * sp];
      lv[k] = ml[2 * sp + 1];
      av[k] = acc_row[(uint64_t)sp * D + c0 + c];
    }
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      if (g + RG * k < splits) M = fmaxf(M, mv[k]);
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        if (g + RG * k < splits) {
          const float w = exp2f(mv[k] - M);
          L += lv[k] * w;
          acc += av[k] * w;
        }
      }
    }
  } else {
    for (int sp = g; sp < splits; sp += RG) M = fmaxf(M, ml[2 * sp]);
    if (M != -INFINITY) {
      for (int sp = g; sp < splits; sp += RG) {
        const float w = exp2f(ml[2 * sp] - M);
        L += ml[2 * sp + 1] * w;
        acc += acc_row[(uint64_t)sp * D + c0 + c] * w;
      }
    }
  }
  gacc[g][c] = acc;
  if (c == 0) {
    gm[g] = M;
    gl[g] = L;
  }
  __syncthreads();
  float Mt = -INFINITY;
#pragma unroll
  for (int k = 0; k < RG; ++k) Mt = fmaxf(Mt, gm[k]);
  if (Mt == -INFINITY) return false;
  float Lt = 0.0f, at = 0.0f;
  if (g == 0) {
#pragma unroll 8
    for (int k = 0; k < RG; ++k) {
      const float w = gm[k] == -INFINITY ? 0.0f : exp2f(gm[k] - Mt);
      Lt += gl[k] * w;
      at += gacc[k][c] * w;
    }
  }
  *o = at / Lt;
  *lse2 = Mt + log2f(Lt);
  return true;
}

// grid (batch*n_q_heads, 128 / RC), RG * RC threads; group 0 writes.
template <int RG, int RC>
__global__ __launch_bounds__(RG * RC) void k_decode_reduce(const float* __restrict__ part_ml,
                                                           const float* __restrict__ part_acc,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse, int splits) {
  const int r = blockIdx.x, c0 = blockIdx.y * RC, c = threadIdx.x % RC;
  float o, l2;
  const bool any = merge_splits<RG, RC>(part_ml + (uint64_t)r * splits * 2,
                                        part_acc + (uint64_t)r * splits * D, splits, c0, &o, &l2);
  if (threadIdx.x >= RC) return;
  out[(uint64_t)r * D + c0 + c] = any ? (uint16_t)f2bf(o) : (uint16_t)0;
  if (lse && blockIdx.y == 0 && c == 0) lse[r] = any ? l2 * 0.69314718055994530942f : -INFINITY;
}

// Rotated cache, first pass: per (stream, span), the span's share of the
// merged rotated output of every q head of the group, rotated back by the
// span's R_V:  y[g][c] = sum_k R_V[c][k] o1[g][k] with o1[g][k] = sum over
// the span's splits of acc[sp][k] exp2(m_sp - M_g), M_g the maximum over all
// splits of the row.  grid (streams, n_span, 4), 128 threads: workgroup z
// produces channels 32 z .. 32 z + 31 (a stream with one span still gets 4
// workgroups); thread t first merges channel t of o1, then four threads
// share an output channel (t >> 2), each summing 32 of its k, added within
// the quad.  The 32 rows of R_V are staged in LDS by coalesced rows (padded
// to 132 floats).  Split sp belongs to span sp / spl.
constexpr int RV_ROWS = 32;
constexpr int RV_STRIDE = D + 4;
// NG: the group size rounded up to 4, 8 or 16 (registers and LDS sized by it)
template <int NG>
__global__ __launch_bounds__(128) void k_decode_span_rot(const float* __restrict__ part_ml,
                                                         const float* __restrict__ part_acc,
                                                         const float* __restrict__ rot,
                                                         float* __restrict__ span_out, int splits,
                                                         int spl, int hq, int hkv) {
  __shared__ float rv[RV_ROWS * RV_STRIDE];
  __shared__ float o1[NG * D], red[NG];
  const int s = blockIdx.x, span = blockIdx.y, n_span = gridDim.y, t = threadIdx.x;
  const int c0 = RV_ROWS * blockIdx.z;
  const int G = hq / hkv;
  const int b = s / hkv, h = s - b * hkv;
  const int row0 = b * hq + h * G;
  const float4* RV4 = reinterpret_cast<const float4*>(
      rot + (((uint64_t)s * n_span + span) * 2 + 1) * D * D + (uint64_t)c0 * D);
  // the R_V rows' loads go out first and land in LDS after the maxima, so
  // that their latency overlaps the split loads
  constexpr int NRV = RV_ROWS * D / 4 / D;
  float4 rvr[NRV];
#pragma unroll
  for (int u = 0; u < NRV; ++u) rvr[u] = RV4[t + D * u];
  // groups of up to 4 heads over at most 8 splits per span (the per-span
  // case): the span's own partial rows go out with them too, so that one
  // round trip brings every operand (their weights wait for the maxima)
  constexpr int PSP = 8;
  const int sp_lo = span * spl;
  const bool pre = NG == 4 && spl <= PSP;  // block-uniform
  float pm[NG == 4 ? 4 : 1][PSP], pa[NG == 4 ? 4 : 1][PSP];
  if constexpr (NG == 4) {
    if (pre) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gr = row0 + min(g, G - 1);
#pragma unroll
        for (int u = 0; u < PSP; ++u) {
          const int sp = sp_lo + min(u, spl - 1);
          pm[g][u] = part_ml[((uint64_t)gr * splits + sp) * 2];
          pa[g][u] = part_acc[((uint64_t)gr * splits + sp) * D + t];
        }
      }
    }
  }
  // M_g of every head: 32 threads per head, four heads per pass
  for (int g0 = 0; g0 < G; g0 += 4) {
    const int g = g0 + (t >> 5);
    float m = -INFINITY;
    if (g < G) {
      const float* ml = part_ml + (uint64_t)(row0 + g) * splits * 2;
      // four loads in flight per pass (a clamped index repeats a split,
      // which leaves the maximum unchanged)
      for (int sp0 = t & 31; sp0 < splits; sp0 += 128) {
        float mm[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) mm[u] = ml[2 * min(sp0 + 32 * u, splits - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) m = fmaxf(m, mm[u]);
      }
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((t & 31) == 0 && g < G) red[g] = m;
  }
#pragma unroll
  for (int u = 0; u < NRV; ++u) {
    const int i = t + D * u;
    *reinterpret_cast<float4*>(rv + (i >> 5) * RV_STRIDE + 4 * (i & 31)) = rvr[u];
  }
  __syncthreads();
  if constexpr (NG == 4) {
    if (pre) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < G) {
          const float M = red[g];
          float a = 0.0f;
          if (M != -INFINITY) {
#pragma unroll
            for (int u = 0; u < PSP; ++u)
              if (u < spl && pm[g][u] != -INFINITY) a += pa[g][u] * exp2f(pm[g][u] - M);
          }
          o1[g * D + t] = a;
        }
      }
    }
  }
  for (int g = 0; g < (pre ? 0 : G); ++g) {
    const float M = red[g];
    const float* ml = part_ml + (uint64_t)(row0 + g) * splits * 2;
    const float* acc = part_acc + (uint64_t)(row0 + g) * splits * D;
    float a = 0.0f;
    if (M != -INFINITY) {
      // eight splits' loads in flight per pass, clamped to the span
      const int sp1 = (span + 1) * spl;
      for (int sp0 = span * spl; sp0 < sp1; sp0 += 8) {
        float mv[8], av[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sp = min(sp0 + u, sp1 - 1);
          mv[u] = ml[2 * sp];
          av[u] = acc[(uint64_t)sp * D + t];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (sp0 + u < sp1 && mv[u] != -INFINITY) a += av[u] * exp2f(mv[u] - M);
      }
    }
    o1[g * D + t] = a;
  }
  __syncthreads();
  const int row = t >> 2, k0 = (D / 4) * (t & 3);
  float y[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) y[g] = 0.0f;
  const float* r = rv + row * RV_STRIDE + k0;
#pragma unroll 4
  for (int j = 0; j < D / 4; ++j) {
    const float rk = r[j];
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (g < G) y[g] = __builtin_fmaf(rk, o1[g * D + k0 + j], y[g]);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g < G) {
      float v = y[g] + __shfl_xor(y[g], 1, 64);
      v += __shfl_xor(v, 2, 64);
      if ((t & 3) == 0) span_out[((uint64_t)(row0 + g) * n_span + span) * D + c0 + row] = v;
    }
  }
}

// Rotated cache, second pass: out = (sum over spans, in span order, of the
// first pass's y) / L, with L the merged denominator, then the single bf16
// rounding; lse from M and L.  grid (batch * hq), 128 threads.
__global__ __launch_bounds__(128) void k_decode_rot_final(const float* __restrict__ part_ml,
                                                          const float* __restrict__ span_out,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse, int splits,
                                                          int n_span) {
  __shared__ float red[D];
  const int r = blockIdx.x, c = threadIdx.x;
  const float* ml = part_ml + (uint64_t)r * splits * 2;
  float m = -INFINITY;
  for (int sp = c; sp < splits; sp += D) m = fmaxf(m, ml[2 * sp]);
  red[c] = m;
  __syncthreads();
  for (int w = D / 2; w >= 1; w >>= 1) {
    if (c < w) red[c] = fmaxf(red[c], red[c + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float l = 0.0f;
  if (M != -INFINITY)
    for (int sp = c; sp < splits; sp += D) l += ml[2 * sp + 1] * exp2f(ml[2 * sp] - M);
  red[c] = l;
  __syncthreads();
  for (int w = D / 2; w >= 1; w >>= 1) {
    if (c < w) red[c] += red[c + w];
    __syncthreads();
  }
  const float L = red[0];
  const bool any = M != -INFINITY;
  float v = 0.0f;
  for (int span = 0; span < n_span; ++span) v += span_out[((uint64_t)r * n_span + span) * D + c];
  out[(uint64_t)r * D + c] = any ? (uint16_t)f2bf(v / L) : (uint16_t)0;
  if (lse && c == 0) lse[r] = any ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

// Rotated queries for a rotated cache: q'[k] = sum over i of q[i] R_K[i][k]
// in fp32 with the R_K of each span (four fma chains over quarters of i,
// then added), stored as its bf16 rounding hi and the bf16 rounding of the
// remainder lo, [row][n_span][128].  grid (streams, n_span), 128 threads:
// thread t takes k = 4 (t & 31) .. +3 over the quarter t >> 5 of i, for every
// q head of the group (R_K read once per stream and span, 16 bytes per lane).
template <int NG>
__global__ __launch_bounds__(128) void k_rotate_q(const uint16_t* __restrict__ q,
                                                  const float* __restrict__ rot,
                                                  uint16_t* __restrict__ qhi,
                                                  uint16_t* __restrict__ qlo, int hq, int hkv) {
  __shared__ float qs[NG][D];
  __shared__ float part[4][NG][D];
  const int s = blockIdx.x, span = blockIdx.y, n_span = gridDim.y, t = threadIdx.x;
  const int G = hq / hkv;
  const int b = s / hkv, h = s - b * hkv;
  const int row0 = b * hq + h * G;
  for (int g = 0; g < G; ++g) qs[g][t] = bf2f(q[(uint64_t)(row0 + g) * D + t]);
  __syncthreads();
  const int kq = t & 31, iq = t >> 5;
  const float4* RK4 =
      reinterpret_cast<const float4*>(rot + ((uint64_t)s * n_span + span) * 2 * D * D) + kq;
  float4 acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 16
  for (int j = 0; j < D / 4; ++j) {
    const int i = (D / 4) * iq + j;
    const float4 r = RK4[i * (D / 4)];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g < G) {
        const float qi = qs[g][i];
        acc[g].x = __builtin_fmaf(qi, r.x, acc[g].x);
        acc[g].y = __builtin_fmaf(qi, r.y, acc[g].y);
        acc[g].z = __builtin_fmaf(qi, r.z, acc[g].z);
        acc[g].w = __builtin_fmaf(qi, r.w, acc[g].w);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g)
    if (g < G) *reinterpret_cast<float4*>(&part[iq][g][4 * kq]) = acc[g];
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const float v = (part[0][g][t] + part[1][g][t]) + (part[2][g][t] + part[3][g][t]);
    const uint32_t hi = f2bf(v);
    const uint64_t o = ((uint64_t)(row0 + g) * n_span + span) * D + t;
    qhi[o] = (uint16_t)hi;
    qlo[o] = (uint16_t)f2bf(v - bf2f(hi));
  }
}

// Fixed decode scratch for kv_attend_decode_noalloc: the split partials of
// a call live here instead of in a caller's workspace.  Every GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name is only a stand-in; the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[KVC_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodePlan& p, hipStream_t st) {
  DecodeArgs a;
  a.q = p.rot ? p.qhi : p.q;
  a.q_lo = p.rot ? p.qlo : nullptr;
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
  a.items = p.streams * p.splits;
  a.n_span = p.n_span;
  a.span_desc = p.span_desc;
  a.spl = p.spl;
  a.sl2 = p.scale * KVC_LOG2E;
  a.wg_merge = (!p.rot && p.splits % WAVES == 0) ? 1 : 0;
  const dim3 grid((a.items + WAVES - 1) / WAVES);
  if (p.rot) {
    const dim3 gq(p.streams, p.n_span);
    if (p.G <= 4)
      hipLaunchKernelGGL(k_rotate_q<4>, gq, dim3(128), 0, st, p.q, p.rot, p.qhi, p.qlo, p.hq, p.hkv);
    else if (p.G <= 8)
      hipLaunchKernelGGL(k_rotate_q<8>, gq, dim3(128), 0, st, p.q, p.rot, p.qhi, p.qlo, p.hq, p.hkv);
    else
      hipLaunchKernelGGL(k_rotate_q<16>, gq, dim3(128), 0, st, p.q, p.rot, p.qhi, p.qlo, p.hq, p.hkv);
    if (p.G <= 4)
      hipLaunchKernelGGL((k_decode_split<1, true>), grid, dim3(64 * WAVES), 0, st, a);
    else if (p.G <= 8)
      hipLaunchKernelGGL((k_decode_split<2, true>), grid, dim3(64 * WAVES), 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_split<4, true>), grid, dim3(64 * WAVES), 0, st, a);
    const dim3 gs(p.streams, p.n_span, D / RV_ROWS);
    if (p.G <= 4)
      hipLaunchKernelGGL(k_decode_span_rot<4>, gs, dim3(D), 0, st, p.part_ml, p.part_acc, p.rot,
                         p.span_out, p.splits, p.spl, p.hq, p.hkv);
    else if (p.G <= 8)
      hipLaunchKernelGGL(k_decode_span_rot<8>, gs, dim3(D), 0, st, p.part_ml, p.part_acc, p.rot,
                         p.span_out, p.splits, p.spl, p.hq, p.hkv);
    else
      hipLaunchKernelGGL(k_decode_span_rot<16>, gs, dim3(D), 0, st, p.part_ml, p.part_acc, p.rot,
                         p.span_out, p.splits, p.spl, p.hq, p.hkv);
    hipLaunchKernelGGL(k_decode_rot_final, dim3(p.batch * p.hq), dim3(D), 0, st, p.part_ml,
                       p.span_out, p.out, p.lse, p.splits, p.n_span);
    return hipGetLastError();
  }
  if (p.G <= 4)
    hipLaunchKernelGGL((k_decode_split<1, false>), grid, dim3(64 * WAVES), 0, st, a);
  else if (p.G <= 8)
    hipLaunchKernelGGL((k_decode_split<2, false>), grid, dim3(64 * WAVES), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode_split<4, false>), grid, dim3(64 * WAVES), 0, st, a);
  const int parts = a.wg_merge ? p.splits / WAVES : p.splits;  // partials per row
  if (parts > 32)
    hipLaunchKernelGGL((k_decode_reduce<32, 32>), dim3(p.batch * p.hq, D / 32), dim3(1024), 0, st,
                       p.part_ml, p.part_acc, p.out, p.lse, parts);
  else if (parts > 8)
    hipLaunchKernelGGL((k_decode_reduce<8, 128>), dim3(p.batch * p.hq, 1), dim3(1024), 0, st,
                       p.part_ml, p.part_acc, p.out, p.lse, parts);
  else
    hipLaunchKernelGGL((k_decode_reduce<1, 128>), dim3(p.batch * p.hq, 1), dim3(128), 0, st,
                       p.part_ml, p.part_acc, p.out, p.lse, parts);
  return hipGetLastError();
}

}  // namespace kvc
